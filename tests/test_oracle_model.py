"""Pins of the oracle's model, conversion, guidance, schedule and sampler (CPU only)."""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import kimodo_oracle as O
from synthetic.inputs import (
    Dims,
    bf16_bits_to_f32,
    make_lengths,
    make_noise,
    make_text,
    make_weights,
    param_count,
    round_to_bf16_bits,
    weight_specs,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = Dims(layers_root=2, layers_body=2, d_model=16, n_heads=2, d_ff=24, root_feats=5, body_feats=7, text_dim=12)
RNG = np.random.default_rng(99)


def _tiny_nets(d=TINY, seed=5, scale=1.0):
    w = make_weights(d, seed=seed)
    if scale != 1.0:
        w = [a * np.float32(scale) if kind == "w" else a for a, (_, _, kind) in zip(w, weight_specs(d))]
    return O.unpack_params(w, d)


def _torch_layer(lp, d, H, F):
    layer = torch.nn.TransformerEncoderLayer(d, H, F, dropout=0.0, activation="gelu", batch_first=True,
                                             norm_first=False, dtype=torch.float64)
    sd = {
        "self_attn.in_proj_weight": lp["qkv.W"], "self_attn.in_proj_bias": lp["qkv.b"],
        "self_attn.out_proj.weight": lp["o.W"], "self_attn.out_proj.bias": lp["o.b"],
        "linear1.weight": lp["ff1.W"], "linear1.bias": lp["ff1.b"],
        "linear2.weight": lp["ff2.W"], "linear2.bias": lp["ff2.b"],
        "norm1.weight": lp["ln1.g"], "norm1.bias": lp["ln1.b"],
        "norm2.weight": lp["ln2.g"], "norm2.bias": lp["ln2.b"],
    }
    layer.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in sd.items()})
    return layer.eval()


# --- the transformer: PyTorch's own post-norm TransformerEncoderLayer is the
# --- definition the pages point at ("two 16-layer TransformerEncoder
# --- sub-networks", post-norm, GELU: Kimodo WebGPU README, "Model details").
@pytest.mark.parametrize("n_valid", [10, 6])
def test_encoder_layer_matches_torch(n_valid):
    nets = _tiny_nets(scale=10.0)
    lp = nets["root"]["layers"][0]
    S = 10
    h = RNG.standard_normal((S, TINY.d_model))
    layer = _torch_layer(lp, TINY.d_model, TINY.n_heads, TINY.d_ff)
    pad = torch.zeros(1, S, dtype=torch.bool)
    pad[0, n_valid:] = True
    with torch.no_grad():
        ref = layer(torch.from_numpy(h)[None], src_key_padding_mask=pad if n_valid < S else None)[0].numpy()
    got = O.encoder_layer(h, lp, n_valid, TINY.n_heads)
    np.testing.assert_allclose(got[:n_valid], ref[:n_valid], atol=1e-11)


def test_subnetwork_matches_torch_stack():
    d = TINY
    nets = _tiny_nets(scale=10.0)
    net = nets["body"]
    T, n = 8, 6
    x_in = RNG.standard_normal((T, d.root_feats + d.body_feats))
    t_tok = RNG.standard_normal(d.d_model)
    c_tok = RNG.standard_normal(d.d_model)
    layers = [_torch_layer(lp, d.d_model, d.n_heads, d.d_ff) for lp in net["layers"]]
    # token assembly written out independently: [t, c, frames] + PE
    pe = np.zeros((T + 2, d.d_model))
    for pos in range(T + 2):
        for i in range(d.d_model // 2):
            a = pos / 10000 ** (2 * i / d.d_model)
            pe[pos, 2 * i], pe[pos, 2 * i + 1] = math.sin(a), math.cos(a)
    h = np.vstack([t_tok, c_tok, x_in @ net["in.W"].T + net["in.b"]]) + pe
    x = torch.from_numpy(h)[None]
    pad = torch.zeros(1, T + 2, dtype=torch.bool)
    pad[0, n + 2:] = True
    with torch.no_grad():
        for layer in layers:
            x = layer(x, src_key_padding_mask=pad)
    ref = x[0].numpy()[2:] @ net["out.W"].T + net["out.b"]
    got = O.subnetwork(net, x_in, t_tok, c_tok, n, d.n_heads)
    np.testing.assert_allclose(got[:n], ref[:n], atol=1e-11)


def _layer_loops(h, lp, H):
    """One post-norm layer with pure-Python loops (tiny shapes only)."""
    S, D = len(h), len(h[0])
    dh = D // H

    def lin(x, W, b):
        return [[b[n] + sum(x[m][k] * W[n][k] for k in range(len(x[0]))) for n in range(len(W))] for m in range(len(x))]

    def ln(x, g, b):
        out = []
        for row in x:
            mu = sum(row) / len(row)
            var = sum((z - mu) ** 2 for z in row) / len(row)
            out.append([(z - mu) / math.sqrt(var + 1e-5) * g[i] + b[i] for i, z in enumerate(row)])
        return out

    qkv = lin(h, lp["qkv.W"], lp["qkv.b"])
    att = [[0.0] * D for _ in range(S)]
    for j in range(H):
        for i in range(S):
            s = [sum(qkv[i][j * dh + c] * qkv[t][D + j * dh + c] for c in range(dh)) / math.sqrt(dh) for t in range(S)]
            m = max(s)
            e = [math.exp(z - m) for z in s]
            for c in range(dh):
                att[i][j * dh + c] = sum(e[t] * qkv[t][2 * D + j * dh + c] for t in range(S)) / sum(e)
    a = lin(att, lp["o.W"], lp["o.b"])
    h1 = ln([[h[i][c] + a[i][c] for c in range(D)] for i in range(S)], lp["ln1.g"], lp["ln1.b"])
    f1 = [[0.5 * z * (1 + math.erf(z / math.sqrt(2))) for z in row] for row in lin(h1, lp["ff1.W"], lp["ff1.b"])]
    f = lin(f1, lp["ff2.W"], lp["ff2.b"])
    return ln([[h1[i][c] + f[i][c] for c in range(D)] for i in range(S)], lp["ln2.g"], lp["ln2.b"])


def test_encoder_layer_matches_loops():
    d = Dims(layers_root=1, layers_body=1, d_model=4, n_heads=2, d_ff=6, root_feats=5, body_feats=3, text_dim=4)
    nets = O.unpack_params([a * np.float32(20.0) for a in make_weights(d, seed=3)], d)
    lp = nets["root"]["layers"][0]
    h = RNG.standard_normal((3, 4))
    want = _layer_loops(h.tolist(), {k: np.asarray(v).tolist() for k, v in lp.items()}, 2)
    np.testing.assert_allclose(O.encoder_layer(h, lp, 3, 2), np.array(want), atol=1e-12)


def test_conditioning_tokens():
    d = TINY
    net = _tiny_nets()["root"]
    # unconditional row: zero embedding -> exactly the text bias
    np.testing.assert_array_equal(O.text_token(net, None), net["txt.b"])
    e = RNG.standard_normal(d.text_dim)
    np.testing.assert_allclose(O.text_token(net, e), net["txt.W"] @ e + net["txt.b"], atol=1e-13)
    # timestep MLP at t = 0: sinusoid(0) = [0,1,0,1,...]
    s0 = np.tile([0.0, 1.0], d.d_model // 2)
    hidden = net["t1.W"] @ s0 + net["t1.b"]
    hidden = hidden * scipy_expit(hidden)
    np.testing.assert_allclose(O.timestep_token(net, 0, d.d_model), net["t2.W"] @ hidden + net["t2.b"], atol=1e-13)


def scipy_expit(x):
    import scipy.special

    return scipy.special.expit(x)


def test_zero_layers_reduce_to_projections():
    d = Dims(layers_root=0, layers_body=0, d_model=16, n_heads=2, d_ff=24, root_feats=5, body_feats=7, text_dim=12)
    nets = O.unpack_params(make_weights(d, seed=8), d)
    net = nets["root"]
    x_in = RNG.standard_normal((6, 5))
    got = O.subnetwork(net, x_in, np.zeros(16), np.zeros(16), 6, 2)
    pe = O.sinusoid(np.arange(2, 8), 16)
    want = (x_in @ net["in.W"].T + net["in.b"] + pe) @ net["out.W"].T + net["out.b"]
    np.testing.assert_allclose(got, want, atol=1e-13)


# --- global -> local root conversion -------------------------------------
def test_g2l_worked_example():
    with open(os.path.join(GOLDEN, "g2l_worked_example.json")) as f:
        ex = json.load(f)
    np.testing.assert_allclose(O.global_to_local_root(np.array(ex["global"])), np.array(ex["local"]), atol=1e-15)


def test_g2l_invariants_and_round_trip():
    T = 40
    g = RNG.standard_normal((T, 5))
    ell = O.global_to_local_root(g)
    p = g[:, 0] + 1j * g[:, 2]
    h = (g[:, 3] + 1j * g[:, 4]) / np.abs(g[:, 3] + 1j * g[:, 4])
    # |v_f| = |p_f - p_{f-1}|, |r_f| = 1, height passes through
    np.testing.assert_allclose(np.abs(ell[1:, 0] + 1j * ell[1:, 2]), np.abs(np.diff(p)), atol=1e-13)
    np.testing.assert_allclose(np.abs(ell[:, 3] + 1j * ell[:, 4]), 1.0, atol=1e-13)
    np.testing.assert_array_equal(ell[:, 1], g[:, 1])
    # invariant to a global yaw rotation q and translation c, and to heading length
    q = np.exp(1j * 0.7)
    p2 = q * p + (3.0 - 2.0j)
    h2 = q * (g[:, 3] + 1j * g[:, 4]) * RNG.uniform(0.1, 5.0, T)
    g2 = np.stack([p2.real, g[:, 1], p2.imag, h2.real, h2.imag], axis=1)
    np.testing.assert_allclose(O.global_to_local_root(g2), ell, atol=1e-12)
    # exact round trip given frame 0: h_f = h_{f-1} r_f, p_f = p_{f-1} + h_f v_f
    hh, pp = [h[0]], [p[0]]
    for f in range(1, T):
        hh.append(hh[-1] * (ell[f, 3] + 1j * ell[f, 4]))
        pp.append(pp[-1] + hh[-1] * (ell[f, 0] + 1j * ell[f, 2]))
    np.testing.assert_allclose(np.array(pp), p, atol=1e-12)
    np.testing.assert_allclose(np.array(hh), h, atol=1e-12)
    # frame f depends on frames f and f-1 only
    g3 = g.copy()
    g3[25:] = RNG.standard_normal((T - 25, 5))
    np.testing.assert_array_equal(O.global_to_local_root(g3)[:25], ell[:25])


# --- guidance, schedule, sampler -----------------------------------------
def test_cfg_special_cases():
    c, u = RNG.standard_normal((4, 9)), RNG.standard_normal((4, 9))
    np.testing.assert_allclose(O.cfg_combine(c, u, 1.0), c, atol=1e-15)
    np.testing.assert_array_equal(O.cfg_combine(c, u, 0.0), u)
    np.testing.assert_allclose(O.cfg_combine(c, u, 2.5) - O.cfg_combine(c, u, 1.5), c - u, atol=1e-14)


def test_linear_schedule_exact():
    betas, abar = O.linear_beta_schedule()
    assert len(abar) == 100 and abar[0] == 0.9999
    prod = Fraction(1)
    for i in range(100):
        beta = Fraction(1, 10000) + Fraction(199, 10000) * Fraction(i, 99)
        prod *= 1 - beta
        assert abs(Fraction(float(abar[i])) - prod) < Fraction(1, 10 ** 14)
    assert np.all(np.diff(abar) < 0) and abar[-1] > 0
    assert abs(abar[49] - 0.77718008) < 5e-9 and abs(abar[99] - 0.36356325) < 5e-9


def test_cosine_schedule_complementary_levels():
    """With s = 0 the continuous levels are cos^2(pi u / 2), so the noise levels
    after i + 1 and n - 1 - i steps (u and 1 - u) add to exactly 1
    (cos^2 + sin^2); u = 1/3 gives cos^2(pi / 6) = 3/4. Pins the squared cosine,
    the pi/2 scaling and the step-index convention."""
    n = 300
    _, abar = O.cosine_beta_schedule(n, s=0.0)
    i = np.arange(0, n - 2)
    np.testing.assert_allclose(abar[i] + abar[n - 2 - i], 1.0, rtol=0, atol=1e-12)
    assert abs(abar[99] - 0.75) < 1e-12  # after 100 of 300 steps, u = 1/3
    assert abs(abar[149] - 0.5) < 1e-12  # u = 1/2


def test_cosine_schedule_shape():
    """Default s = 0.008, n = 100: betas rise monotonically; the final beta hits
    the 0.999 clip (f(1) = 0); levels fall strictly; the offset s keeps the
    first beta small but nonzero; no beta before the last is clipped."""
    betas, abar = O.cosine_beta_schedule()
    assert np.all(np.diff(betas) > 0)
    assert betas[-1] == 0.999 and np.all(betas[:-1] < 0.999)
    assert np.all(np.diff(abar) < 0) and 0 < abar[-1] < 1e-3 * abar[-2] + 1e-12
    assert 0 < betas[0] < 1e-3
    # the offset only shifts the curve: s = 0.008 lies between s = 0 and a
    # larger offset at every step
    _, a0 = O.cosine_beta_schedule(s=0.0)
    _, a1 = O.cosine_beta_schedule(s=0.05)
    assert np.all((abar[:-1] >= np.minimum(a0, a1)[:-1]) & (abar[:-1] <= np.maximum(a0, a1)[:-1]))


def test_timesteps():
    np.testing.assert_array_equal(O.ddim_timesteps(100), np.arange(100))
    np.testing.assert_array_equal(O.ddim_timesteps(50), np.arange(0, 100, 2))
    np.testing.assert_array_equal(O.ddim_timesteps(35), [k * 100 // 35 for k in range(35)])


def test_ddim_consistency_and_last_step():
    _, abar = O.linear_beta_schedule()
    x0 = RNG.standard_normal((3, 7))
    eps = RNG.standard_normal((3, 7))
    for t, tp in ((99, 98), (50, 49), (60, 10)):
        x_t = math.sqrt(abar[t]) * x0 + math.sqrt(1 - abar[t]) * eps
        want = math.sqrt(abar[tp]) * x0 + math.sqrt(1 - abar[tp]) * eps
        np.testing.assert_allclose(O.ddim_step(x_t, x0, abar[t], abar[tp]), want, atol=1e-13)
    np.testing.assert_allclose(O.ddim_step(RNG.standard_normal((3, 7)), x0, abar[3], 1.0), x0, atol=1e-15)


def test_ddim_coefficients_t50():
    # x_prev = A x0_hat + C x_t with A = sqrt(ab_p) - sqrt(1-ab_p) sqrt(ab_t)/sqrt(1-ab_t),
    # C = sqrt(1-ab_p)/sqrt(1-ab_t), evaluated in 40-digit decimal arithmetic from exact alpha_bar.
    getcontext().prec = 40
    prod = Fraction(1)
    ab = []
    for i in range(100):
        prod *= 1 - (Fraction(1, 10000) + Fraction(199, 10000) * Fraction(i, 99))
        ab.append(prod)
    at = Decimal(ab[50].numerator) / Decimal(ab[50].denominator)
    ap = Decimal(ab[49].numerator) / Decimal(ab[49].denominator)
    C = (1 - ap).sqrt() / (1 - at).sqrt()
    A = ap.sqrt() - C * at.sqrt()
    _, abar = O.linear_beta_schedule()
    got_A = O.ddim_step(np.array(0.0), np.array(1.0), abar[50], abar[49])
    got_C = O.ddim_step(np.array(1.0), np.array(0.0), abar[50], abar[49])
    assert abs(float(got_A) - float(A)) < 1e-14 and abs(float(got_C) - float(C)) < 1e-14
    assert abs(float(A) - 0.019611565) < 1e-9 and abs(float(C) - 0.982754475) < 1e-9


def test_stub_model_sampler_closed_form():
    """Both output heads' weights zeroed: x0_hat = [b_out_root || b_out_body] = x* for
    every input, so eps_hat stays eps_0 = (x_T - sqrt(ab) x*)/sqrt(1-ab) along the
    chain, x after the step to tau is sqrt(ab(tau)) x* + sqrt(1-ab(tau)) eps_0, and
    the final x_0 = x*."""
    d = TINY
    w = make_weights(d, seed=11)
    names = [n for n, _, _ in weight_specs(d)]
    w[names.index("root.out.W")][:] = 0
    w[names.index("body.out.W")][:] = 0
    nets = O.unpack_params(w, d)
    xstar = np.concatenate([nets["root"]["out.b"], nets["body"]["out.b"]])
    B, T, S = 2, 6, 10
    noise = make_noise(B, T, d)
    ts = O.ddim_timesteps(S)
    _, abar = O.linear_beta_schedule()
    a0 = abar[ts[-1]]
    eps0 = (noise - math.sqrt(a0) * xstar) / math.sqrt(1 - a0)
    seen = []

    def cb(k, x):
        a = abar[ts[k - 1]] if k > 0 else 1.0
        np.testing.assert_allclose(x, math.sqrt(a) * xstar + math.sqrt(1 - a) * eps0, atol=1e-12)
        seen.append(k)

    x = O.sample(nets, d, noise, make_text(B, d), [T, T], ts, abar, 2.5, step_callback=cb)
    assert seen == list(range(S - 1, -1, -1))
    np.testing.assert_allclose(x, np.broadcast_to(xstar, x.shape), atol=1e-12)


def test_truncation_invariance_whole_step():
    """A clip of length n padded to T gives, on its valid frames, the result of the
    same clip run at T = n; its padded frames are 0."""
    d = TINY
    nets = _tiny_nets(seed=21, scale=5.0)
    B, T = 2, 9
    lens = [6, 9]
    x_t = make_noise(B, T, d).astype(np.float64)
    text = make_text(B, d)
    _, abar = O.linear_beta_schedule()
    full = O.denoise_step(nets, d, x_t, text, lens, 40, abar[40], abar[39], 2.5)
    short = O.denoise_step(nets, d, x_t[:1, :6], text[:1], [6], 40, abar[40], abar[39], 2.5)
    np.testing.assert_allclose(full[0, :6], short[0], atol=1e-12)
    np.testing.assert_array_equal(full[0, 6:], 0.0)
    # clips are independent: clip 1 alone equals clip 1 in the batch
    alone = O.denoise_step(nets, d, x_t[1:], text[1:], [9], 40, abar[40], abar[39], 2.5)
    np.testing.assert_allclose(full[1], alone[0], atol=1e-12)


def test_step_trace_is_consistent():
    d = TINY
    nets = _tiny_nets(seed=4, scale=5.0)
    B, T = 2, 5
    x_t = make_noise(B, T, d).astype(np.float64)
    text = make_text(B, d)
    _, abar = O.linear_beta_schedule()
    tr = {}
    x = O.denoise_step(nets, d, x_t, text, [5, 4], 30, abar[30], abar[29], 2.5, trace=tr)
    assert tr["layers_root"].shape == (2, 2 * B, T + 2, d.d_model)
    np.testing.assert_allclose(tr["local_root"][1], O.global_to_local_root(tr["root_out"][1]), atol=0)
    x0 = np.concatenate([tr["root_out"], tr["body_out"]], axis=2)
    np.testing.assert_allclose(tr["x0_hat"], x0[B:] + 2.5 * (x0[:B] - x0[B:]), atol=1e-14)
    np.testing.assert_allclose(x[0], O.ddim_step(x_t[0], tr["x0_hat"][0], abar[30], abar[29]), atol=1e-14)


# --- inputs --------------------------------------------------------------
def test_param_count_matches_pages():
    # 282M parameters in two 16-layer sub-networks; 540 MB of fp16 weights
    # (Kimodo WebGPU README, "Model details" table).
    n = param_count(Dims())
    assert n == 281_963_799
    assert round(n / 1e6) == 282 and abs(2 * n / 2 ** 20 - 540) < 3


def test_bf16_rounding_matches_torch():
    x = np.concatenate([RNG.standard_normal(10000).astype(np.float32) * 3,
                        bf16_bits_to_f32(np.arange(0, 0x7F00, 37, dtype=np.uint16)),
                        # exact ties: low half = 0x8000
                        (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(round_to_bf16_bits(x), want)


def test_length_recipes():
    np.testing.assert_array_equal(make_lengths(4, 150), 150)
    l3 = make_lengths(32, 180, "uniform60")
    assert l3.min() >= 60 and l3.max() <= 180
    l4 = make_lengths(128, 300, "quarter150")
    assert (l4 < 300).sum() <= 32 and (l4 == 300).sum() >= 96 and l4.min() >= 150


def test_unconditional_row_ignores_text():
    """w = 0 returns the unconditional prediction, which must not see the text."""
    d = TINY
    nets = _tiny_nets(seed=31, scale=5.0)
    x_t = make_noise(1, 5, d).astype(np.float64)
    _, abar = O.linear_beta_schedule()
    a = O.denoise_step(nets, d, x_t, make_text(1, d), [5], 20, abar[20], abar[19], 0.0)
    b = O.denoise_step(nets, d, x_t, 10 * make_text(1, d, seed=77), [5], 20, abar[20], abar[19], 0.0)
    np.testing.assert_array_equal(a, b)
    c = O.denoise_step(nets, d, x_t, make_text(1, d, seed=77), [5], 20, abar[20], abar[19], 1.0)
    assert np.abs(c - a).max() > 1e-6


def test_body_reads_local_root_not_noisy_root():
    """With the root head's weight zeroed, the root prediction is a constant, so
    the noisy root stream x_t[..., 0:5] may only reach x0_hat through nothing: the
    body network reads the converted root prediction, not the noisy root input."""
    d = TINY
    w = make_weights(d, seed=41)
    names = [n for n, _, _ in weight_specs(d)]
    w[names.index("root.out.W")][:] = 0
    nets = O.unpack_params([a * np.float32(5.0) if n.endswith(".W") and n != "root.out.W" else a
                            for a, n in zip(w, names)], d)
    x_t = make_noise(1, 6, d).astype(np.float64)
    x_t2 = x_t.copy()
    x_t2[..., :5] += RNG.standard_normal((1, 6, 5))
    _, abar = O.linear_beta_schedule()
    tr1, tr2 = {}, {}
    O.denoise_step(nets, d, x_t, make_text(1, d), [6], 20, abar[20], abar[19], 2.5, trace=tr1)
    O.denoise_step(nets, d, x_t2, make_text(1, d), [6], 20, abar[20], abar[19], 2.5, trace=tr2)
    np.testing.assert_allclose(tr1["x0_hat"], tr2["x0_hat"], atol=1e-13)
    # while the body stream does reach it
    x_t3 = x_t.copy()
    x_t3[..., 5:] += RNG.standard_normal((1, 6, d.body_feats))
    tr3 = {}
    O.denoise_step(nets, d, x_t3, make_text(1, d), [6], 20, abar[20], abar[19], 2.5, trace=tr3)
    assert np.abs(tr3["x0_hat"] - tr1["x0_hat"]).max() > 1e-6
