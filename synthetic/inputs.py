"""Seeded synthetic inputs: weights, text embeddings, initial noise, clip lengths.

Both the CPU oracle and the HIP library consume exactly these arrays, so the two
sides never need to share a random-number generator: as in the kimodo.cpp forum
introduction ("원본과의 일치를 확인하는 방법": the initial noise is stored and read
back, never regenerated), the noise is an input here, not something the sampler
draws.

Workload shapes follow the pages: 5 s clips are 150 frames at 30 fps
(kimodo-fast README, first table), 6 s clips are 180 frames (Kimodo WebGPU README,
"What it does"), 10 s is the length the model is trained to (kimodo-fast README,
flags table). A prompt arrives as one 4096-float LLM2Vec embedding (Kimodo WebGPU
README, "What it does"); here it is N(0,1) noise of that shape, a stand-in for
mean-pooled Llama-3 states. Weights are random N(0, 0.02) draws, not the trained
checkpoint, which is not available.

Nothing in this module computes any part of the denoiser.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Tuple

import numpy as np

WEIGHT_SEED = 0
TEXT_SEED = 1
NOISE_SEED = 2
LENGTH_SEED = 3
INIT_STD = 0.02


@dataclass(frozen=True)
class Dims:
    """Model dimensions. Defaults are the full model: 8 heads x 128, hidden
    1024, FFN 2048 (Kimodo WebGPU README, "Model details" table); root stream
    5 features and body stream 30 joints x 9 + 4 contacts = 274 features per
    frame."""

    layers_root: int = 16
    layers_body: int = 16
    d_model: int = 1024
    n_heads: int = 8
    d_ff: int = 2048
    root_feats: int = 5
    body_feats: int = 274
    text_dim: int = 4096

    @property
    def d_head(self) -> int:
        return self.d_model // self.n_heads

    @property
    def feats(self) -> int:
        return self.root_feats + self.body_feats


# The five workloads. "lengths" names the per-clip length recipe.
CONFIGS: Dict[int, dict] = {
    0: dict(B=1, T=60, layers=2, dtype="f32", steps=1, t=50, cfg_scale=2.5, lengths="full"),
    1: dict(B=1, T=150, layers=16, dtype="bf16", steps=100, cfg_scale=2.5, lengths="full"),
    2: dict(B=16, T=150, layers=16, dtype="bf16", steps=100, cfg_scale=2.5, lengths="full"),
    3: dict(B=32, T=180, layers=16, dtype="bf16", steps=50, cfg_scale=2.5, lengths="uniform60"),
    4: dict(B=128, T=300, layers=16, dtype="bf16", steps=100, cfg_scale=2.5, lengths="quarter150"),
}


def dims_for(config: int) -> Dims:
    L = CONFIGS[config]["layers"]
    return Dims(layers_root=L, layers_body=L)


def _subnet_specs(prefix: str, d: Dims, k_in: int, n_out: int) -> List[Tuple[str, Tuple[int, ...], str]]:
    D, F = d.d_model, d.d_ff
    L = d.layers_root if prefix == "root" else d.layers_body
    s: List[Tuple[str, Tuple[int, ...], str]] = [
        (f"{prefix}.txt.W", (D, d.text_dim), "w"),
        (f"{prefix}.txt.b", (D,), "w"),
        (f"{prefix}.t1.W", (D, D), "w"),
        (f"{prefix}.t1.b", (D,), "w"),
        (f"{prefix}.t2.W", (D, D), "w"),
        (f"{prefix}.t2.b", (D,), "w"),
        (f"{prefix}.in.W", (D, k_in), "w"),
        (f"{prefix}.in.b", (D,), "w"),
    ]
    for l in range(L):
        p = f"{prefix}.layer{l}"
        s += [
            (f"{p}.qkv.W", (3 * D, D), "w"),
            (f"{p}.qkv.b", (3 * D,), "w"),
            (f"{p}.o.W", (D, D), "w"),
            (f"{p}.o.b", (D,), "w"),
            (f"{p}.ln1.g", (D,), "gamma"),
            (f"{p}.ln1.b", (D,), "w"),
            (f"{p}.ff1.W", (F, D), "w"),
            (f"{p}.ff1.b", (F,), "w"),
            (f"{p}.ff2.W", (D, F), "w"),
            (f"{p}.ff2.b", (D,), "w"),
            (f"{p}.ln2.g", (D,), "gamma"),
            (f"{p}.ln2.b", (D,), "w"),
        ]
    s += [(f"{prefix}.out.W", (n_out, D), "w"), (f"{prefix}.out.b", (n_out,), "w")]
    return s


def weight_specs(d: Dims) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) of every parameter tensor in canonical order: the
    root sub-network first, then the body sub-network; Linear weights are
    [out, in]. The root network reads the 5 root features, the body network
    reads 5 local-root features plus the 274 body features."""
    return _subnet_specs("root", d, d.root_feats, d.root_feats) + _subnet_specs(
        "body", d, d.root_feats + d.body_feats, d.body_feats
    )


def param_count(d: Dims) -> int:
    return int(sum(int(np.prod(s)) for _, s, _ in weight_specs(d)))


def make_weights(d: Dims, seed: int = WEIGHT_SEED) -> List[np.ndarray]:
    """fp32 draws in canonical order from one PCG64 stream: Linear weights and
    biases and LayerNorm shifts ~ N(0, 0.02^2); LayerNorm gains ~ 1 + N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    out = []
    std = np.float32(INIT_STD)
    for _, shape, kind in weight_specs(d):
        z = rng.standard_normal(shape, dtype=np.float32) * std
        if kind == "gamma":
            z = z + np.float32(1.0)
        out.append(z)
    return out


def make_text(B: int, d: Dims = Dims(), seed: int = TEXT_SEED) -> np.ndarray:
    """[B, 4096] fp32, N(0, 1)."""
    return np.random.default_rng(seed).standard_normal((B, d.text_dim), dtype=np.float32)


def make_noise(B: int, T: int, d: Dims = Dims(), seed: int = NOISE_SEED) -> np.ndarray:
    """Initial diffusion state x_T, [B, T, 279] fp32, N(0, 1)."""
    return np.random.default_rng(seed).standard_normal((B, T, d.feats), dtype=np.float32)


def make_lengths(B: int, T: int, recipe: str = "full", seed: int = LENGTH_SEED) -> np.ndarray:
    """int32 [B] valid frame counts.

    "full": every clip has T frames. "uniform60": U{60..T} per clip.
    "quarter150": a seeded 25% of the clips get U{150..T}, the rest T.
    """
    rng = np.random.default_rng(seed)
    if recipe == "full":
        return np.full(B, T, np.int32)
    if recipe == "uniform60":
        return rng.integers(60, T + 1, size=B).astype(np.int32)
    if recipe == "quarter150":
        lens = np.full(B, T, np.int32)
        idx = rng.choice(B, size=B // 4, replace=False)
        lens[idx] = rng.integers(150, T + 1, size=len(idx))
        return lens
    raise ValueError(f"unknown length recipe {recipe!r}")


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    Inputs must be finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# A timeline workload: three 3 s segments at 30 fps with the default 2
# transition frames, 35 DDIM steps (the default step count) and 4 takes in one
# batch (kimodo-fast README, "Timelines" and flags table).
TIMELINE = dict(V=4, frames=(90, 90, 90), n_transition=2, steps=35, cfg_scale=2.5)


def timeline_inputs(V: int, frames, d: Dims = Dims(), seed: int = 0) -> dict:
    """Segment k's text [V, 4096] (seed 40 + seed + k) and noise [V, T_k, 279]
    (seed 60 + seed + k); text stacked to [n_seg, V, 4096]."""
    return dict(text=np.stack([make_text(V, d, seed=40 + seed + k) for k in range(len(frames))]),
                noise=[make_noise(V, T, d, seed=60 + seed + k) for k, T in enumerate(frames)])


# A 30-joint humanoid tree standing in for the SOMA30 skeleton (hips, spine,
# head, arms, legs, hands, feet: Kimodo WebGPU README, "Model details"), whose
# hierarchy and bone offsets are not on the pages. Joints are in topological
# order (every parent before its children); offsets are in metres in the
# parent's frame, y up.
SKELETON_JOINTS = (
    ("Hips", -1, (0.0, 0.0, 0.0)),
    ("Spine", 0, (0.0, 0.10, 0.0)), ("Spine1", 1, (0.0, 0.12, 0.0)), ("Spine2", 2, (0.0, 0.12, 0.0)),
    ("Neck", 3, (0.0, 0.15, 0.0)), ("Head", 4, (0.0, 0.10, 0.02)), ("HeadEnd", 5, (0.0, 0.18, 0.0)),
    ("LeftShoulder", 3, (0.05, 0.12, 0.0)), ("LeftArm", 7, (0.13, 0.0, 0.0)), ("LeftForeArm", 8, (0.27, 0.0, 0.0)),
    ("LeftHand", 9, (0.25, 0.0, 0.0)), ("LeftHandEnd", 10, (0.10, 0.0, 0.0)),
    ("RightShoulder", 3, (-0.05, 0.12, 0.0)), ("RightArm", 12, (-0.13, 0.0, 0.0)),
    ("RightForeArm", 13, (-0.27, 0.0, 0.0)), ("RightHand", 14, (-0.25, 0.0, 0.0)), ("RightHandEnd", 15, (-0.10, 0.0, 0.0)),
    ("LeftLeg", 0, (0.09, -0.05, 0.0)), ("LeftShin", 17, (0.0, -0.42, 0.0)), ("LeftFoot", 18, (0.0, -0.41, 0.0)),
    ("LeftToe", 19, (0.0, -0.05, 0.13)), ("LeftToeEnd", 20, (0.0, 0.0, 0.05)),
    ("RightLeg", 0, (-0.09, -0.05, 0.0)), ("RightShin", 22, (0.0, -0.42, 0.0)), ("RightFoot", 23, (0.0, -0.41, 0.0)),
    ("RightToe", 24, (0.0, -0.05, 0.13)), ("RightToeEnd", 25, (0.0, 0.0, 0.05)),
    ("Jaw", 5, (0.0, 0.02, 0.06)), ("LeftEye", 5, (0.03, 0.08, 0.07)), ("RightEye", 5, (-0.03, 0.08, 0.07)),
)
SKELETON_SEED = 4


def make_skeleton(seed: int = SKELETON_SEED):
    """(names, parents int32 [30], offsets fp32 [30, 3]): the tree above with
    every bone length scaled by a seeded factor in [0.9, 1.1]."""
    names = [n for n, _, _ in SKELETON_JOINTS]
    parents = np.array([p for _, p, _ in SKELETON_JOINTS], np.int32)
    scale = np.random.default_rng(seed).uniform(0.9, 1.1, size=(len(names), 1))
    offsets = (np.array([o for _, _, o in SKELETON_JOINTS]) * scale).astype(np.float32)
    return names, parents, offsets


def config_inputs(config: int) -> dict:
    """All inputs of one workload: dims, weights (fp32 draws; bf16-rounded for
    bf16 workloads, both as values and bits), text, noise, lengths."""
    c = CONFIGS[config]
    d = dims_for(config)
    w = make_weights(d)
    bits = None
    if c["dtype"] == "bf16":
        bits = [round_to_bf16_bits(a) for a in w]
        w = [bf16_bits_to_f32(b) for b in bits]
    return dict(
        dims=d,
        weights=w,
        weight_bits=bits,
        text=make_text(c["B"], d),
        noise=make_noise(c["B"], c["T"], d),
        lengths=make_lengths(c["B"], c["T"], c["lengths"]),
        length_recipe=c["lengths"],
        **{k: v for k, v in c.items() if k != "lengths"},
    )
