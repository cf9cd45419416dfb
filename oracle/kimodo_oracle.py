"""Plain, slow CPU oracle of one batched DDIM sampling loop of Kimodo's
two-stage denoiser, in numpy float64.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module. It shares no code with the HIP
library (text_motion_diffusion_amd): the only thing both sides consume is the
seeded input arrays from the ``synthetic`` package.

What is computed, in the pages' order (Kimodo WebGPU README, "Architecture"
diagram: DDIM loop = root model -> globalRootToLocalRoot -> body model -> CFG
guidance -> DDIM update; the kimodo.cpp forum introduction lists the same stage
boundaries in its fixture table under "kimodo.cpp가 원본과의 일치를 확인하는 방법"):

  per DDIM step, for every clip b and for both guidance rows (conditional and
  text-zeroed):
    root transformer  (its own root stream, K = 5)  -> root prediction R
    global -> local root conversion of R            -> l
    body transformer  ([l || noisy body stream], K = 279) -> body prediction
  x0_hat = [R || body] per row; CFG combine of the two rows; DDIM (eta = 0)
  update; frames past a clip's length are written as 0.

Each transformer: two prepended tokens (timestep token, text token), sinusoidal
positions, L post-norm encoder layers with 8 heads x 128, hidden 1024, GELU FFN
2048 (Kimodo WebGPU README, "Model details" table), optional key masking
("WGSL compute shaders" table, attention row), an output Linear.

The pages print no equation for any of this. Every place where they are silent
takes the plainest reading, and the same reading is implemented in the HIP
library:
  * the network predicts the clean motion x0 (the root output is converted
    global -> local and fed to the body net, which only makes sense for a clean
    trajectory);
  * CFG: x0_hat = u + w (c - u) once, after both stages; the unconditional row
    has its 4096-float embedding set to zero;
  * schedule: linear betas 1e-4 .. 0.02 over 100 training steps (the workload
    definition; the WebGPU page's model table says "cosine"); alpha_bar is the
    cumulative product of (1 - beta); S sampling steps visit
    tau_k = floor(k * 100 / S), k = S-1 .. 0, and the last step has
    alpha_bar_prev = 1;
  * token order [timestep, text, frames]; interleaved sin/cos positional
    encoding (base 10000) added to all tokens; the same sinusoid embeds the
    integer timestep before a Linear-SiLU-Linear MLP;
  * GELU is the exact erf form; LayerNorm eps 1e-5 with biased variance;
  * attention scale 1/sqrt(128); keys at positions >= length + 2 get -inf;
  * fused QKV weight = [Wq; Wk; Wv] on the output dim, head j at rows
    128j .. 128j + 127 of each block; Linear weights are [out, in];
  * the global -> local root conversion: see ``global_to_local_root``;
  * known-entry constraints (timelines, pinned root paths): see
    ``apply_known`` and ``timeline``.

Parity with the real, trained Kimodo network is unpinned: the pages print no
intermediate value that can be reproduced without the trained checkpoint.
Every function here is pinned by the CPU tests (tests/test_oracle_*.py) to
closed forms, invariants and brute-force loops.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
from scipy.special import erf

LN_EPS = 1e-5
G2L_EPS = 1e-8
N_TRAIN_STEPS = 100
BETA_START = 1e-4
BETA_END = 0.02
PE_BASE = 10000.0


# ---------------------------------------------------------------------------
# Elementary ops (Kimodo WebGPU README, "WGSL compute shaders" table: linear,
# attention, layernorm, gelu, silu, elementwise).
# ---------------------------------------------------------------------------
def linear(x: np.ndarray, W: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Linear layer in the torch convention: y = x W^T + b, W [out, in]."""
    return x @ W.T + b


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = x/2 * (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU (timestep MLP activation): x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis, biased variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def sinusoid(pos, d: int) -> np.ndarray:
    """[len(pos), d]: column 2i = sin(pos * base^(-2i/d)), column 2i+1 = cos(same)."""
    pos = np.asarray(pos, dtype=np.float64).reshape(-1)
    i = np.arange(d // 2, dtype=np.float64)
    ang = pos[:, None] * PE_BASE ** (-2.0 * i / d)[None, :]
    out = np.empty((pos.shape[0], d))
    out[:, 0::2] = np.sin(ang)
    out[:, 1::2] = np.cos(ang)
    return out


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_valid: int, n_heads: int) -> np.ndarray:
    """Multi-head self-attention of one sequence with key masking.

    q, k, v: [S, d]; head j uses columns j*dh .. (j+1)*dh. Keys at positions
    >= n_valid get score -inf. Every query row (padded ones too) attends to the
    valid keys. Returns the heads concatenated in order, [S, d].
    """
    S, d = q.shape
    dh = d // n_heads
    mask = np.zeros(S)
    mask[n_valid:] = -np.inf
    out = np.empty((S, d))
    for j in range(n_heads):
        c = slice(j * dh, (j + 1) * dh)
        scores = q[:, c] @ k[:, c].T / np.sqrt(dh) + mask[None, :]
        scores = scores - scores.max(axis=1, keepdims=True)
        p = np.exp(scores)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, c] = p @ v[:, c]
    return out


def encoder_layer(h: np.ndarray, lp: Dict[str, np.ndarray], n_valid: int, n_heads: int) -> np.ndarray:
    """One post-norm TransformerEncoder layer (Kimodo WebGPU README, "Model
    details": post-norm, GELU):  h1 = LN1(h + MHSA(h)),  out = LN2(h1 + FFN(h1))."""
    d = h.shape[1]
    qkv = linear(h, lp["qkv.W"], lp["qkv.b"])
    q, k, v = qkv[:, :d], qkv[:, d : 2 * d], qkv[:, 2 * d :]
    a = linear(masked_attention(q, k, v, n_valid, n_heads), lp["o.W"], lp["o.b"])
    h1 = layer_norm(h + a, lp["ln1.g"], lp["ln1.b"])
    f = linear(gelu(linear(h1, lp["ff1.W"], lp["ff1.b"])), lp["ff2.W"], lp["ff2.b"])
    return layer_norm(h1 + f, lp["ln2.g"], lp["ln2.b"])


# ---------------------------------------------------------------------------
# Diffusion schedule and sampler (Kimodo WebGPU README, "What it does": DDIM
# noise scheduling on the client; "Model details": DDIM, 50-100 steps).
# ---------------------------------------------------------------------------
def linear_beta_schedule(n: int = N_TRAIN_STEPS, start: float = BETA_START, end: float = BETA_END):
    """betas[i] = start + (end - start) * i / (n - 1); alpha_bar[i] = prod_{j<=i} (1 - betas[j])."""
    betas = start + (end - start) * np.arange(n, dtype=np.float64) / (n - 1)
    alpha_bar = np.cumprod(1.0 - betas)
    return betas, alpha_bar


def cosine_beta_schedule(n: int = N_TRAIN_STEPS, s: float = 0.008, max_beta: float = 0.999):
    """Cosine schedule (the WebGPU README's "Model details" table names a cosine
    beta schedule; its form is the one published by Nichol & Dhariwal,
    "Improved Denoising Diffusion Probabilistic Models", 2021, section 3.2):
    alpha_bar(u) = f(u) / f(0) with f(u) = cos^2(pi/2 * (u + s) / (1 + s)) over
    u in [0, 1]. Discretised over n training steps as
    betas[i] = min(1 - f((i + 1) / n) / f(i / n), max_beta), so that, where no
    beta is clipped, alpha_bar[i] = prod_{j<=i} (1 - betas[j]) = f((i + 1) / n) / f(0).
    (Reading: step index i counts from 0, so alpha_bar[i] is the level after
    i + 1 noising steps, the same convention as the linear schedule.)"""
    def f(u):
        return np.cos(0.5 * np.pi * (u + s) / (1.0 + s)) ** 2
    i = np.arange(n, dtype=np.float64)
    betas = np.minimum(1.0 - f((i + 1.0) / n) / f(i / n), max_beta)
    alpha_bar = np.cumprod(1.0 - betas)
    return betas, alpha_bar


def ddim_timesteps(S: int, n_train: int = N_TRAIN_STEPS) -> np.ndarray:
    """Sampling timesteps tau_k = floor(k * n_train / S), k = 0..S-1 (ascending;
    the sampler visits them from k = S-1 down to 0)."""
    return (np.arange(S, dtype=np.int64) * n_train) // S


def global_to_local_root(g: np.ndarray) -> np.ndarray:
    """globalRootToLocalRoot (Kimodo WebGPU README, "Architecture" diagram; the
    representation-conversion row of the kimodo.cpp forum introduction's fixture
    table).

    g: [T, 5] global root per frame = (x, y, z, c, s): position with y up, and
    the heading as the 2-vector (c, s) = (cos psi, sin psi), not necessarily of
    unit length. With p_f = x_f + i z_f, unit heading h_f = (c_f + i s_f) /
    max(|c_f + i s_f|, 1e-8), displacement d_f = p_f - p_{f-1} (d_0 = 0):
        v_f = conj(h_f) d_f          (displacement in the frame's own heading)
        r_f = conj(h_{f-1}) h_f      (heading change, r_0 = 1)
    returns [T, 5] = (Re v_f, y_f, Im v_f, Re r_f, Im r_f).
    Frame f reads frames f and f-1 only.
    """
    g = np.asarray(g, dtype=np.float64)
    p = g[:, 0] + 1j * g[:, 2]
    hraw = g[:, 3] + 1j * g[:, 4]
    h = hraw / np.maximum(np.abs(hraw), G2L_EPS)
    d = np.zeros_like(p)
    d[1:] = p[1:] - p[:-1]
    v = np.conj(h) * d
    r = np.ones_like(h)
    r[1:] = np.conj(h[:-1]) * h[1:]
    return np.stack([v.real, g[:, 1], v.imag, r.real, r.imag], axis=1)


def apply_known(pred: np.ndarray, values: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Known-entry constraint on a clean-motion prediction: where ``mask`` is
    set the prediction is replaced by the caller's value.

    The pages name the uses (a timeline segment conditioned on the previous
    segment's last frames, a pinned root path: kimodo-fast README, "Timelines"
    and "Python") but give no equation. The reading here is replacement of the
    x0 prediction ("inpainting"): applied to each guidance row's prediction,
    to the root prediction before the global -> local conversion (so the body
    network sees the constrained root) and to the body prediction before CFG.
    Both rows then carry the same value, CFG returns it unchanged, and the last
    DDIM step (alpha_bar_prev = 1) returns it exactly.
    """
    return np.where(np.asarray(mask, dtype=bool), values, pred)


def cfg_combine(cond: np.ndarray, uncond: np.ndarray, w: float) -> np.ndarray:
    """Classifier-free guidance on the clean-motion prediction: u + w (c - u)."""
    return uncond + w * (cond - uncond)


def ddim_step(x_t: np.ndarray, x0_hat: np.ndarray, abar_t: float, abar_prev: float) -> np.ndarray:
    """Deterministic DDIM (eta = 0) from a clean-motion prediction:
    eps_hat = (x_t - sqrt(abar_t) x0_hat) / sqrt(1 - abar_t);
    x_prev  = sqrt(abar_prev) x0_hat + sqrt(1 - abar_prev) eps_hat."""
    eps_hat = (x_t - np.sqrt(abar_t) * x0_hat) / np.sqrt(1.0 - abar_t)
    return np.sqrt(abar_prev) * x0_hat + np.sqrt(1.0 - abar_prev) * eps_hat


# ---------------------------------------------------------------------------
# Parameters in canonical order: per sub-network (root, then body)
#   txt.W txt.b t1.W t1.b t2.W t2.b in.W in.b
#   {qkv.W qkv.b o.W o.b ln1.g ln1.b ff1.W ff1.b ff2.W ff2.b ln2.g ln2.b} x L
#   out.W out.b
# ---------------------------------------------------------------------------
_LAYER_KEYS = ("qkv.W", "qkv.b", "o.W", "o.b", "ln1.g", "ln1.b", "ff1.W", "ff1.b", "ff2.W", "ff2.b", "ln2.g", "ln2.b")


def unpack_params(flat: Sequence[np.ndarray], dims) -> Dict[str, dict]:
    """Split the flat canonical list into {'root': net, 'body': net} (fp64),
    checking every shape."""
    D, F, Tx = dims.d_model, dims.d_ff, dims.text_dim
    it = iter(flat)

    def take(shape):
        a = np.asarray(next(it), dtype=np.float64)
        if a.shape != tuple(shape):
            raise ValueError(f"parameter shape {a.shape} != expected {tuple(shape)}")
        return a

    nets = {}
    for name, L, k_in, n_out in (
        ("root", dims.layers_root, dims.root_feats, dims.root_feats),
        ("body", dims.layers_body, dims.root_feats + dims.body_feats, dims.body_feats),
    ):
        net = {
            "txt.W": take((D, Tx)), "txt.b": take((D,)),
            "t1.W": take((D, D)), "t1.b": take((D,)),
            "t2.W": take((D, D)), "t2.b": take((D,)),
            "in.W": take((D, k_in)), "in.b": take((D,)),
        }
        layers = []
        for _ in range(L):
            shapes = ((3 * D, D), (3 * D,), (D, D), (D,), (D,), (D,), (F, D), (F,), (D, F), (D,), (D,), (D,))
            layers.append({k: take(s) for k, s in zip(_LAYER_KEYS, shapes)})
        net["layers"] = layers
        net["out.W"] = take((n_out, D))
        net["out.b"] = take((n_out,))
        nets[name] = net
    try:
        next(it)
    except StopIteration:
        return nets
    raise ValueError("more parameter tensors than the model has")


def timestep_token(net: dict, t: int, d_model: int) -> np.ndarray:
    """Sinusoid of the integer timestep through Linear -> SiLU -> Linear
    (Kimodo WebGPU README, "WGSL compute shaders" table, silu.wgsl row: SiLU is
    the timestep MLP's activation)."""
    e = sinusoid([t], d_model)[0]
    return linear(silu(linear(e, net["t1.W"], net["t1.b"])), net["t2.W"], net["t2.b"])


def text_token(net: dict, emb: Optional[np.ndarray]) -> np.ndarray:
    """Projection of the 4096-float text embedding to the model width; the
    unconditional row projects an all-zero embedding."""
    if emb is None:
        emb = np.zeros(net["txt.W"].shape[1])
    return linear(np.asarray(emb, np.float64), net["txt.W"], net["txt.b"])


def subnetwork(net: dict, x_in: np.ndarray, t_tok: np.ndarray, txt_tok: np.ndarray, n_frames: int,
               n_heads: int, layer_trace: Optional[list] = None) -> np.ndarray:
    """One transformer of the two-stage denoiser for one sequence.

    x_in: [T, K] per-frame inputs. Tokens = [timestep token, text token,
    x_in W_in^T + b_in], plus sinusoidal positions 0..T+1; keys past
    n_frames + 2 are masked. Returns the output Linear on the T frame tokens,
    [T, n_out]. If layer_trace is a list, each layer's output [T+2, d] is
    appended to it.
    """
    T = x_in.shape[0]
    d = t_tok.shape[0]
    h = np.concatenate([t_tok[None, :], txt_tok[None, :], linear(x_in, net["in.W"], net["in.b"])], axis=0)
    h = h + sinusoid(np.arange(T + 2), d)
    for lp in net["layers"]:
        h = encoder_layer(h, lp, n_frames + 2, n_heads)
        if layer_trace is not None:
            layer_trace.append(h.copy())
    return linear(h[2:], net["out.W"], net["out.b"])


def denoise_step(nets: Dict[str, dict], dims, x_t: np.ndarray, text: np.ndarray, lengths: Sequence[int],
                 t: int, abar_t: float, abar_prev: float, w: float, trace: Optional[dict] = None,
                 known: Optional[np.ndarray] = None, known_mask: Optional[np.ndarray] = None) -> np.ndarray:
    """One DDIM step of the whole batch.

    x_t [B, T, 279], text [B, 4096], lengths [B]. Sequence rows p = 0..B-1 are
    conditional and p = B..2B-1 unconditional (same order as the HIP path).
    If ``trace`` is a dict it receives the stage outputs: 'layers_root' and
    'layers_body' [L, 2B, T+2, d], 'root_out' [2B, T, 5] and 'body_out'
    [2B, T, 274] (the networks' own predictions), 'local_root' [2B, T, 5],
    'x0_hat' [B, T, 279].

    known / known_mask ([B, T, 279] values and booleans, or both None): entries
    of the clean motion fixed by the caller (a timeline's carried-over frames,
    a pinned root path; kimodo-fast README, "Timelines" and "Python"). Each
    guidance row's prediction is overwritten there, see ``apply_known``.
    """
    x_t = np.asarray(x_t, np.float64)
    B, T, _ = x_t.shape
    rf = dims.root_feats
    H = dims.n_heads
    root, body = nets["root"], nets["body"]
    tok = {n: timestep_token(nets[n], t, dims.d_model) for n in ("root", "body")}
    root_out = np.zeros((2 * B, T, rf))
    local = np.zeros((2 * B, T, rf))
    body_out = np.zeros((2 * B, T, dims.body_feats))
    traces = {"root": [], "body": []}
    for p in range(2 * B):
        b = p % B
        emb = text[b] if p < B else None
        n = int(lengths[b])
        lt_r = [] if trace is not None else None
        lt_b = [] if trace is not None else None
        root_out[p] = subnetwork(root, x_t[b, :, :rf], tok["root"], text_token(root, emb), n, H, lt_r)
        r_used = root_out[p] if known is None else apply_known(root_out[p], known[b, :, :rf], known_mask[b, :, :rf])
        local[p] = global_to_local_root(r_used)
        x_body = np.concatenate([local[p], x_t[b, :, rf:]], axis=1)
        body_out[p] = subnetwork(body, x_body, tok["body"], text_token(body, emb), n, H, lt_b)
        if trace is not None:
            traces["root"].append(np.stack(lt_r))
            traces["body"].append(np.stack(lt_b))
    x0 = np.concatenate([root_out, body_out], axis=2)
    if known is not None:
        for p in range(2 * B):
            x0[p] = apply_known(x0[p], known[p % B], known_mask[p % B])
    x0_hat = cfg_combine(x0[:B], x0[B:], w)
    x_prev = ddim_step(x_t, x0_hat, abar_t, abar_prev)
    for b in range(B):
        x_prev[b, int(lengths[b]):, :] = 0.0
    if trace is not None:
        trace["layers_root"] = np.stack(traces["root"], axis=1)
        trace["layers_body"] = np.stack(traces["body"], axis=1)
        trace.update(root_out=root_out, local_root=local, body_out=body_out, x0_hat=x0_hat)
    return x_prev


def sample(nets: Dict[str, dict], dims, noise: np.ndarray, text: np.ndarray, lengths: Sequence[int],
           timesteps: Sequence[int], alpha_bar: Sequence[float], w: float,
           step_callback=None, known: Optional[np.ndarray] = None,
           known_mask: Optional[np.ndarray] = None) -> np.ndarray:
    """The DDIM sampling loop: start at x = noise, visit timesteps[S-1] .. timesteps[0];
    at step k, abar_t = alpha_bar[timesteps[k]] and abar_prev =
    alpha_bar[timesteps[k-1]] (1 at k = 0). Returns x_0 [B, T, 279].
    known / known_mask: the same constraint at every step (``apply_known``)."""
    x = np.asarray(noise, np.float64)
    S = len(timesteps)
    for k in range(S - 1, -1, -1):
        t = int(timesteps[k])
        a_t = float(alpha_bar[t])
        a_prev = float(alpha_bar[int(timesteps[k - 1])]) if k > 0 else 1.0
        x = denoise_step(nets, dims, x, text, lengths, t, a_t, a_prev, w, known=known, known_mask=known_mask)
        if step_callback is not None:
            step_callback(k, x)
    return x


def timeline(nets: Dict[str, dict], dims, seg_frames: Sequence[int], seg_text: np.ndarray,
             seg_noise: Sequence[np.ndarray], n_transition: int, timesteps: Sequence[int],
             alpha_bar: Sequence[float], w: float, segments: Optional[list] = None) -> np.ndarray:
    """One continuous motion from several segments, V takes at once
    (kimodo-fast README, "Timelines": each segment is conditioned on the end of
    the previous one; transition frames default to 2; only the takes of a
    timeline share a batch, the segments run one after another).

    seg_frames [n_seg]; seg_text [n_seg, V, 4096]; seg_noise[k] [V, T_k, 279].
    Segment 0 is sampled freely. Segment k > 0 is sampled with its first
    n_transition frames (all 279 features) known and equal to the last
    n_transition frames of segment k - 1 (``apply_known``); every segment is
    in the same global root frame. The timeline is segment 0 followed by each
    later segment without its first n_transition frames, which duplicate the
    previous segment's end: [V, T_0 + sum_{k>0} (T_k - n_transition), 279].
    If ``segments`` is a list it receives each segment's whole [V, T_k, 279].
    """
    parts, prev = [], None
    for k, Tk in enumerate(seg_frames):
        V = seg_noise[k].shape[0]
        known = mask = None
        if k > 0 and n_transition > 0:
            known = np.zeros((V, Tk, dims.root_feats + dims.body_feats))
            mask = np.zeros(known.shape, dtype=bool)
            known[:, :n_transition] = prev[:, prev.shape[1] - n_transition:]
            mask[:, :n_transition] = True
        x = sample(nets, dims, seg_noise[k], seg_text[k], [Tk] * V, timesteps, alpha_bar, w,
                   known=known, known_mask=mask)
        parts.append(x if k == 0 else x[:, n_transition:])
        if segments is not None:
            segments.append(x)
        prev = x
    return np.concatenate(parts, axis=1)


def run_config_sample(flat_weights: List[np.ndarray], dims, noise, text, lengths, steps: int, w: float,
                      step_callback=None) -> np.ndarray:
    """Convenience: linear schedule, uniform timesteps, full sample."""
    nets = unpack_params(flat_weights, dims)
    _, abar = linear_beta_schedule()
    return sample(nets, dims, noise, text, lengths, ddim_timesteps(steps), abar, w, step_callback)
