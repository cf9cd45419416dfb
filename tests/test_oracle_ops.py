"""Pins of the oracle's elementary operations (CPU only).

Each check compares the oracle with something other than itself: pure-Python
loops on tiny inputs, textbook constants, identities, or an independent library
routine (torch CPU float64, scipy).
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import kimodo_oracle as O

RNG = np.random.default_rng(1234)


def test_linear_matches_triple_loop():
    x = RNG.standard_normal((3, 4))
    W = RNG.standard_normal((5, 4))  # [out, in]
    b = RNG.standard_normal(5)
    want = [[b[n] + sum(x[m][k] * W[n][k] for k in range(4)) for n in range(5)] for m in range(3)]
    np.testing.assert_allclose(O.linear(x, W, b), np.array(want), rtol=0, atol=1e-13)


def test_gelu_is_exact_erf_form():
    # textbook standard-normal CDF values: Phi(1), Phi(-1), Phi(2.7)
    assert O.gelu(np.array(0.0)) == 0.0
    assert abs(O.gelu(np.array(1.0)) - 0.8413447460685429) < 1e-15
    assert abs(O.gelu(np.array(-1.0)) - (-0.15865525393145707)) < 1e-15
    x = np.linspace(-6, 6, 241)
    np.testing.assert_allclose(O.gelu(x), x * scipy.stats.norm.cdf(x), rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.gelu(x) - O.gelu(-x), x, rtol=0, atol=1e-13)
    # not the tanh approximation: the two differ by ~4.7e-4 near |x| = 2.7
    tanh_form = 0.5 * 2.7 * (1 + math.tanh(math.sqrt(2 / math.pi) * (2.7 + 0.044715 * 2.7 ** 3)))
    assert abs(float(O.gelu(np.array(2.7))) - tanh_form) > 3e-4


def test_silu():
    x = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(O.silu(x), x * scipy.special.expit(x), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(O.silu(x) - O.silu(-x), x, rtol=0, atol=1e-12)
    assert O.silu(np.array(0.0)) == 0.0


def test_layer_norm_against_torch_and_moments():
    x = RNG.standard_normal((7, 64)) * 3 + 1.5
    g = RNG.standard_normal(64)
    b = RNG.standard_normal(64)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), torch.from_numpy(b), eps=1e-5)
    np.testing.assert_allclose(O.layer_norm(x, g, b), want.numpy(), rtol=0, atol=1e-12)
    y = O.layer_norm(x, np.ones(64), np.zeros(64))
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    # invariant to adding a constant per row
    np.testing.assert_allclose(O.layer_norm(x + 7.0, g, b), O.layer_norm(x, g, b), atol=1e-11)


def test_sinusoid_closed_forms():
    d = 1024
    e0 = O.sinusoid([0], d)[0]
    np.testing.assert_array_equal(e0[0::2], 0.0)
    np.testing.assert_array_equal(e0[1::2], 1.0)
    for t in (1, 17, 99, 301):
        e = O.sinusoid([t], d)[0]
        assert abs(e @ e - d / 2) < 1e-9
        assert abs(e[0] - math.sin(t)) < 1e-15 and abs(e[1] - math.cos(t)) < 1e-15
        # last pair: frequency 10000^(-(d-2)/d)
        f = 10000.0 ** (-(d - 2) / d)
        assert abs(e[-2] - math.sin(t * f)) < 1e-12 and abs(e[-1] - math.cos(t * f)) < 1e-12


def _attention_loops(q, k, v, n_valid, H):
    S, d = q.shape
    dh = d // H
    out = np.zeros((S, d))
    for j in range(H):
        for i in range(S):
            s = [sum(q[i][j * dh + c] * k[t][j * dh + c] for c in range(dh)) / math.sqrt(dh) for t in range(n_valid)]
            m = max(s)
            e = [math.exp(z - m) for z in s]
            tot = sum(e)
            for c in range(dh):
                out[i][j * dh + c] = sum(e[t] * v[t][j * dh + c] for t in range(n_valid)) / tot
    return out


@pytest.mark.parametrize("n_valid", [5, 3, 1])
def test_attention_matches_loops(n_valid):
    q, k, v = (RNG.standard_normal((5, 8)) for _ in range(3))
    np.testing.assert_allclose(O.masked_attention(q, k, v, n_valid, 2), _attention_loops(q, k, v, n_valid, 2), atol=1e-13)


def test_attention_against_torch_sdpa_with_mask():
    S, d, H = 11, 32, 4
    dh = d // H
    q, k, v = (RNG.standard_normal((S, d)) for _ in range(3))
    n_valid = 7
    tq, tk, tv = (torch.from_numpy(a).reshape(S, H, dh).transpose(0, 1).contiguous() for a in (q, k, v))
    mask = torch.zeros(S, S, dtype=torch.bool)
    mask[:, :n_valid] = True  # True = may attend
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    ref = ref.transpose(0, 1).reshape(S, d).numpy()
    np.testing.assert_allclose(O.masked_attention(q, k, v, n_valid, H), ref, atol=1e-12)


def test_attention_invariants():
    S, d, H = 9, 16, 2
    q, k, v = (RNG.standard_normal((S, d)) for _ in range(3))
    # rows of the softmax sum to one: V = 1 gives 1
    np.testing.assert_allclose(O.masked_attention(q, k, np.ones((S, d)), 6, H), 1.0, atol=1e-14)
    # identical keys -> mean of the valid values
    kk = np.tile(k[:1], (S, 1))
    np.testing.assert_allclose(O.masked_attention(q, kk, v, 6, H), np.tile(v[:6].mean(0), (S, 1)), atol=1e-13)
    # masked keys == the truncated sequence, on every query row
    np.testing.assert_allclose(O.masked_attention(q, k, v, 6, H)[:6], O.masked_attention(q[:6], k[:6], v[:6], 6, H), atol=1e-13)
    # masked keys carry no information: garbage there changes nothing
    k2, v2 = k.copy(), v.copy()
    k2[6:] = 1e3
    v2[6:] = -1e3
    np.testing.assert_allclose(O.masked_attention(q, k2, v2, 6, H), O.masked_attention(q, k, v, 6, H), atol=1e-13)
    # query permutation equivariance
    perm = RNG.permutation(S)
    np.testing.assert_allclose(O.masked_attention(q[perm], k, v, S, H), O.masked_attention(q, k, v, S, H)[perm], atol=1e-13)
