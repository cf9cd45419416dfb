"""The oracle's arithmetic with the HIP path's low-precision stores.

Test infrastructure, used only by tests/. It composes the oracle's own
functions (oracle/kimodo_oracle.py) in float64 and rounds each value at the
points where the HIP library's fp16 path stores it in 16 bits (or, for the
precision-floor measurement, in bf16). It implements none of the HIP path and
shares no code with it. Two uses:

* the per-element parity bound of the fp16 path. An fp16 store of x returns
  x (1 + d) with |d| <= u = 2^-11 (round to nearest). The error that these
  stores cause in a stage's output is the propagated sum of such relative
  perturbations. One realisation of it is ``stored - exact`` below, with the
  stores at the same points as the kernels; its RMS over a 1024-wide token row
  is the scale of the rounding noise on that row (1024 samples put the
  estimate within a few percent). The parity tests bound every element of the
  GPU's error by a multiple of that scale plus the element's own last rounding.

* the precision floor (which 16-bit type the activations can use): one DDIM
  step of the full model with every store rounded, against the exact oracle.

Store points of the fp16 path (the library's activation buffers):
  conditioning  text embedding, timestep sinusoid, SiLU hidden layer,
                timestep token, text token;
  stage input   per-frame inputs (root stream; local root + body stream),
                assembled tokens (token + position);
  each layer    Q, K, V; softmax weights entering the P V product (the
                normaliser sums them unrounded); attention output; output
                projection (stored only where no split-K partial sums are
                used, modelled always: it only enlarges the bound); LN1
                output; GELU output; FFN2 output (likewise); LN2 output.
Heads, root conversion, CFG and DDIM are fp32 on the GPU and are checked
against fp32 bounds instead.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

from oracle import kimodo_oracle as O
from synthetic.inputs import bf16_bits_to_f32, round_to_bf16_bits

U_FP16 = 2.0 ** -11  # unit roundoff of fp16 (11-bit significand)
U_BF16 = 2.0 ** -8
U_FP32 = 2.0 ** -24

Rounder = Callable[[np.ndarray], np.ndarray]


def exact(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, np.float64)


def to_fp16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest fp16 (ties to even), back to float64; values past
    the fp16 range become inf."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even) via fp32, back to float64."""
    a = np.asarray(x, np.float64)
    return bf16_bits_to_f32(round_to_bf16_bits(a.astype(np.float32).reshape(-1))).reshape(a.shape).astype(np.float64)


class Recorder:
    """A rounder that also records the largest magnitude it was given
    (the fp16 range check)."""

    def __init__(self, rnd: Rounder):
        self.rnd = rnd
        self.max_abs = 0.0

    def __call__(self, x):
        x = np.asarray(x, np.float64)
        if x.size:
            self.max_abs = max(self.max_abs, float(np.max(np.abs(x))))
        return self.rnd(x)


def attention_stored(q, k, v, n_valid: int, n_heads: int, rnd: Rounder) -> np.ndarray:
    """oracle.masked_attention with the softmax weights rounded where they
    enter the P V product; the normaliser is the sum of the unrounded weights.
    With rnd = exact it equals oracle.masked_attention up to summation order."""
    S, d = q.shape
    dh = d // n_heads
    out = np.empty((S, d))
    for j in range(n_heads):
        c = slice(j * dh, (j + 1) * dh)
        s = q[:, c] @ k[:n_valid, c].T / np.sqrt(dh)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, c] = (rnd(p) @ v[:n_valid, c]) / p.sum(axis=1, keepdims=True)
    return out


def encoder_layer_stored(h, lp, n_valid: int, n_heads: int, rnd: Rounder) -> np.ndarray:
    """oracle.encoder_layer with every activation store rounded by rnd."""
    d = h.shape[1]
    qkv = rnd(O.linear(h, lp["qkv.W"], lp["qkv.b"]))
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    o = rnd(attention_stored(q, k, v, n_valid, n_heads, rnd))
    a = rnd(O.linear(o, lp["o.W"], lp["o.b"]))
    h1 = rnd(O.layer_norm(h + a, lp["ln1.g"], lp["ln1.b"]))
    f1 = rnd(O.gelu(O.linear(h1, lp["ff1.W"], lp["ff1.b"])))
    f = rnd(O.linear(f1, lp["ff2.W"], lp["ff2.b"]))
    return rnd(O.layer_norm(h1 + f, lp["ln2.g"], lp["ln2.b"]))


def tokens_stored(net: dict, x_in: np.ndarray, t: int, emb: Optional[np.ndarray], rnd: Rounder) -> np.ndarray:
    """A sub-network's assembled input tokens [T + 2, d] (the oracle's
    ``subnetwork`` up to its first layer), with the conditioning and
    stage-input stores rounded. emb None = the unconditional row."""
    d = net["t1.W"].shape[0]
    e = rnd(O.sinusoid([t], d)[0])
    t_tok = rnd(O.linear(rnd(O.silu(O.linear(e, net["t1.W"], net["t1.b"]))), net["t2.W"], net["t2.b"]))
    emb = np.zeros(net["txt.W"].shape[1]) if emb is None else rnd(np.asarray(emb, np.float64))
    txt_tok = rnd(O.linear(emb, net["txt.W"], net["txt.b"]))
    frames = O.linear(rnd(np.asarray(x_in, np.float64)), net["in.W"], net["in.b"])
    h = np.concatenate([t_tok[None, :], txt_tok[None, :], frames], axis=0)
    return rnd(h + O.sinusoid(np.arange(h.shape[0]), d))


def subnetwork_stored(net: dict, x_in, t: int, emb, n_frames: int, n_heads: int, rnd: Rounder) -> np.ndarray:
    """oracle.subnetwork (for one sequence) with the stores rounded; the head is fp32 on the GPU and
    is computed exactly here."""
    h = tokens_stored(net, x_in, t, emb, rnd)
    n = n_frames + 2
    for lp in net["layers"]:
        h = encoder_layer_stored(h, lp, n, n_heads, rnd)
    return O.linear(h[2:], net["out.W"], net["out.b"])


def denoise_step_stored(nets: dict, dims, x_t, text, lengths, t: int, abar_t: float, abar_prev: float, w: float,
                        rnd: Rounder) -> np.ndarray:
    """oracle.denoise_step (no constraint) with every activation store of both
    sub-networks rounded by rnd. Each clip runs at its own length (the
    oracle's result does not depend on padding)."""
    x_t = np.asarray(x_t, np.float64)
    B, T, _ = x_t.shape
    rf, H = dims.root_feats, dims.n_heads
    x0 = np.zeros((2 * B, T, dims.feats))
    for p in range(2 * B):
        b = p % B
        n = int(lengths[b])
        emb = text[b] if p < B else None
        r = subnetwork_stored(nets["root"], x_t[b, :n, :rf], t, emb, n, H, rnd)
        body_in = np.concatenate([O.global_to_local_root(r), x_t[b, :n, rf:]], axis=1)
        x0[p, :n, :rf] = r
        x0[p, :n, rf:] = subnetwork_stored(nets["body"], body_in, t, emb, n, H, rnd)
    x_prev = O.ddim_step(x_t, O.cfg_combine(x0[:B], x0[B:], w), abar_t, abar_prev)
    for b in range(B):
        x_prev[b, int(lengths[b]):] = 0.0
    return x_prev


# ---------------------------------------------------------------------------
# Per-element bounds used by the GPU parity tests
# ---------------------------------------------------------------------------
ROW_SIGMAS = 8.0  # multiples of the row's rounding-noise scale


def row_noise_bound(stored: np.ndarray, ref: np.ndarray, u: float = U_FP16) -> np.ndarray:
    """Per-element bound for a stage whose output rows are 1024-wide fp16
    token rows: ROW_SIGMAS times the row's rounding-noise scale (the RMS of
    one realisation, ``stored - ref``, together with the element's own last
    rounding, whose RMS is at most u |y| / sqrt(3)), plus one unit in the last
    place of fp32 so an exactly representable row still has a positive bound."""
    sigma_row = np.sqrt(np.mean((stored - ref) ** 2, axis=-1, keepdims=True))
    last = u * np.abs(ref) / np.sqrt(3.0)
    return ROW_SIGMAS * np.sqrt(sigma_row ** 2 + last ** 2) + U_FP32 * np.abs(ref) + 1e-30


def linear_fp32_bound(x: np.ndarray, W: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Rounding-error bound of y = x W^T + b summed in fp32 in any order from
    exactly representable operands (each product of two fp16 values is exact
    in fp32): |y_fp32 - y| <= gamma_{K+1} (|x| |W|^T + |b|), gamma_n =
    n u / (1 - n u) with u = 2^-24 (the standard bound for a sum of K + 1
    terms in floating point), plus the final rounding u |y|."""
    K = x.shape[-1]
    g = (K + 1) * U_FP32 / (1.0 - (K + 1) * U_FP32)
    return g * (np.abs(x) @ np.abs(W).T + np.abs(b)) + U_FP32 * np.abs(O.linear(x, W, b)) + 1e-30
