"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package draws numbers and nothing else: it holds none of the denoiser's
arithmetic. See :mod:`synthetic.inputs`.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    Dims,
    dims_for,
    weight_specs,
    param_count,
    make_weights,
    make_text,
    make_noise,
    make_lengths,
    round_to_bf16_bits,
    bf16_bits_to_f32,
)
