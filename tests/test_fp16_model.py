"""Pins of the storage-rounding model (tests/fp16_model.py) that the fp16
path's per-element parity bound comes from, and the precision-floor
measurement behind the choice of fp16 over bf16 activations.

With exact rounding the model must be the oracle itself; its rounders must be
IEEE round-to-nearest-even at 11 (fp16) and 8 (bf16) significand bits; the
bound built from one rounding realisation must cover other, independent
realisations of the same stores."""
import numpy as np
import pytest

import fp16_model as F
from oracle import kimodo_oracle as O
from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text, make_weights, round_to_bf16_bits


def _nets(dims, seed=0):
    return O.unpack_params([bf16_bits_to_f32(round_to_bf16_bits(a)) for a in make_weights(dims, seed=seed)], dims)


def test_rounders_are_round_to_nearest_even():
    # fp16: 11 significand bits; halfway cases go to the even neighbour
    one = 1.0
    assert F.to_fp16(np.array([one + 2.0 ** -11]))[0] == one              # tie -> even (1.0)
    assert F.to_fp16(np.array([one + 3 * 2.0 ** -11]))[0] == one + 2.0 ** -9   # tie -> even (1 + 4 u)
    assert F.to_fp16(np.array([one + 1.1 * 2.0 ** -11]))[0] == one + 2.0 ** -10
    assert F.to_fp16(np.array([65504.0]))[0] == 65504.0
    assert np.isinf(F.to_fp16(np.array([65520.0]))[0])                   # rounds past the largest finite value
    # bf16: 8 significand bits
    assert F.to_bf16(np.array([one + 2.0 ** -8]))[0] == one
    assert F.to_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6
    assert F.to_bf16(np.array([-(one + 1.5 * 2.0 ** -8)]))[0] == -(one + 2.0 ** -7)
    x = np.random.default_rng(0).standard_normal(10000)
    assert np.max(np.abs(F.to_fp16(x) - x) / np.abs(x)) <= F.U_FP16
    assert np.max(np.abs(F.to_bf16(x) - x) / np.abs(x)) <= F.U_BF16


def test_exact_rounding_is_the_oracle_layer():
    dims = Dims(layers_root=1, layers_body=0)
    lp = _nets(dims)["root"]["layers"][0]
    h = np.random.default_rng(1).standard_normal((40, 1024))
    for n_valid in (40, 17, 2):  # masked keys
        want = O.encoder_layer(h, lp, n_valid, 8)
        got = F.encoder_layer_stored(h, lp, n_valid, 8, F.exact)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_exact_rounding_is_the_oracle_tokens_and_step():
    dims = Dims(layers_root=1, layers_body=1)
    nets = _nets(dims)
    B, T, t = 2, 9, 37
    x, text = make_noise(B, T, dims), make_text(B, dims)
    lengths = [9, 4]
    # the prefix tokens are the oracle's conditioning tokens plus positions 0 and 1
    net = nets["root"]
    tok = F.tokens_stored(net, x[0, :, :5], t, text[0], F.exact)
    pe = O.sinusoid(np.arange(T + 2), 1024)
    np.testing.assert_allclose(tok[0], O.timestep_token(net, t, 1024) + pe[0], atol=1e-12)
    np.testing.assert_allclose(tok[1], O.text_token(net, text[0]) + pe[1], atol=1e-12)
    tok_u = F.tokens_stored(net, x[0, :, :5], t, None, F.exact)
    np.testing.assert_allclose(tok_u[1], O.text_token(net, None) + pe[1], atol=1e-12)
    np.testing.assert_allclose(tok[2:] - pe[2:], O.linear(x[0, :, :5].astype(np.float64), net["in.W"], net["in.b"]),
                               atol=1e-12)
    _, ab = O.linear_beta_schedule()
    want = O.denoise_step(nets, dims, x, text, lengths, t, ab[t], ab[t - 1], 2.5)
    got = F.denoise_step_stored(nets, dims, x, text, lengths, t, ab[t], ab[t - 1], 2.5, F.exact)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-10)


def test_row_noise_bound_covers_independent_rounding_realisations():
    """The bound is built from the deterministic round-to-nearest realisation;
    independent realisations (each stored value perturbed by a relative error
    drawn uniformly from [-u, u]) must stay inside it, with margin."""
    dims = Dims(layers_root=2, layers_body=0)
    layers = _nets(dims)["root"]["layers"]
    rng = np.random.default_rng(2)

    def perturb(v):
        v = np.asarray(v, np.float64)
        return v * (1.0 + rng.uniform(-F.U_FP16, F.U_FP16, v.shape))

    worst = 0.0
    for i, lp in enumerate(layers):
        for n in (64, 23, 3):
            h = F.to_fp16(np.random.default_rng(10 * i + n).standard_normal((n, 1024)))
            want = O.encoder_layer(h, lp, n, 8)
            bound = F.row_noise_bound(F.encoder_layer_stored(h, lp, n, 8, F.to_fp16), want)
            for _ in range(2):
                worst = max(worst, float(np.max(np.abs(F.encoder_layer_stored(h, lp, n, 8, perturb) - want) / bound)))
    print(f"largest |error| / bound over the realisations: {worst:.3f}")
    assert worst < 0.8


def test_bound_catches_a_planted_masking_mistake():
    """A mistake planted in the oracle side (attention that also weighs one
    masked key) moves the layer output far outside the bound."""
    dims = Dims(layers_root=1, layers_body=0)
    lp = _nets(dims)["root"]["layers"][0]
    n = 30
    h = F.to_fp16(np.random.default_rng(3).standard_normal((40, 1024)))
    want = O.encoder_layer(h[:n], lp, n, 8)
    bound = F.row_noise_bound(F.encoder_layer_stored(h[:n], lp, n, 8, F.to_fp16), want)
    wrong = O.encoder_layer(h[:n + 1], lp, n + 1, 8)[:n]  # one padded key leaks in
    assert np.max(np.abs(wrong - want) / bound) > 10.0


@pytest.fixture(scope="module")
def floor_case():
    dims = Dims()
    nets = _nets(dims)
    B, T = 1, 150
    x, text = make_noise(B, T, dims), make_text(B, dims)
    _, ab = O.linear_beta_schedule()
    # the last step of a sample (t = 0, abar_prev = 1) returns the guided
    # clean-motion prediction itself, so its error is the network's
    want = O.denoise_step(nets, dims, x, text, [T], 0, ab[0], 1.0, 2.5)
    return dims, nets, x, text, ab, want


@pytest.mark.parametrize("name,rnd,lo,hi", [("bf16", F.to_bf16, 1e-2, 1.0), ("fp16", F.to_fp16, 0.0, 5e-3)])
def test_precision_floor_of_16_bit_activations(floor_case, name, rnd, lo, hi):
    """One DDIM step of the full 16 + 16 layer model (1 clip x 150 frames,
    bf16 weights exact in both cases), every activation store rounded to the
    16-bit type, fp64 arithmetic otherwise, against the exact oracle: bf16
    storage alone already exceeds the 1e-2 relative L2 tolerance of the final
    motion, fp16 storage stays well inside it."""
    dims, nets, x, text, ab, want = floor_case
    got = F.denoise_step_stored(nets, dims, x, text, [150], 0, ab[0], 1.0, 2.5, rnd)
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    print(f"{name} activation storage: relative L2 {rel:.3e}")
    assert lo < rel < hi
