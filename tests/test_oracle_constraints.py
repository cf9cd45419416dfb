"""Pins of the oracle's known-entry constraints and timelines (CPU only).

The pages name the uses (kimodo-fast README, "Timelines": each segment is
conditioned on the end of the previous one, 2 transition frames by default;
"Python": a pinned root path) but give no equation; the reading is replacement
of each guidance row's x0 prediction at the known entries, the root entries
before the global -> local conversion. These tests pin what that reading fixes:
the closed form when every entry is known, exact return of known entries, the
root-before-conversion placement, and the timeline's seams and assembly.
"""
import math

import numpy as np

from oracle import kimodo_oracle as O
from synthetic.inputs import Dims, make_noise, make_text, make_weights, timeline_inputs, weight_specs

TINY = Dims(layers_root=2, layers_body=2, d_model=16, n_heads=2, d_ff=24, root_feats=5, body_feats=7, text_dim=12)
RNG = np.random.default_rng(123)


def _nets(seed=5, scale=5.0, d=TINY):
    w = make_weights(d, seed=seed)
    w = [a * np.float32(scale) if kind == "w" else a for a, (_, _, kind) in zip(w, weight_specs(d))]
    return O.unpack_params(w, d)


def _schedule(S):
    _, abar = O.linear_beta_schedule()
    return O.ddim_timesteps(S), abar


def test_empty_mask_is_unconstrained():
    d = TINY
    nets = _nets()
    B, T = 2, 6
    noise, text = make_noise(B, T, d), make_text(B, d)
    ts, abar = _schedule(4)
    free = O.sample(nets, d, noise, text, [6, 4], ts, abar, 2.5)
    known = RNG.standard_normal((B, T, d.feats))
    masked = O.sample(nets, d, noise, text, [6, 4], ts, abar, 2.5, known=known,
                      known_mask=np.zeros(known.shape, dtype=bool))
    np.testing.assert_array_equal(free, masked)


def test_all_known_closed_form():
    """Every entry known: x0_hat = V at every step whatever the network does, so
    eps_hat stays eps_0 = (x_T - sqrt(ab) V) / sqrt(1 - ab) and the state after
    the step to tau is sqrt(ab(tau)) V + sqrt(1 - ab(tau)) eps_0; x_0 = V."""
    d = TINY
    nets = _nets(seed=8)
    B, T, S = 2, 5, 8
    noise = make_noise(B, T, d).astype(np.float64)
    V = RNG.standard_normal((B, T, d.feats))
    ts, abar = _schedule(S)
    a0 = abar[ts[-1]]
    eps0 = (noise - math.sqrt(a0) * V) / math.sqrt(1 - a0)
    seen = []

    def cb(k, x):
        a = abar[ts[k - 1]] if k > 0 else 1.0
        np.testing.assert_allclose(x, math.sqrt(a) * V + math.sqrt(1 - a) * eps0, atol=1e-12)
        seen.append(k)

    x = O.sample(nets, d, noise, make_text(B, d), [T, T], ts, abar, 2.5, step_callback=cb, known=V,
                 known_mask=np.ones(V.shape, dtype=bool))
    assert seen == list(range(S - 1, -1, -1))
    np.testing.assert_allclose(x, V, atol=1e-12)


def test_known_entries_returned_exactly_and_others_move():
    """Both guidance rows carry V at a known entry, CFG leaves it unchanged and
    the last step (alpha_bar_prev = 1) returns it bit for bit; the constraint
    also changes the unknown entries (it conditions the rest of the motion)."""
    d = TINY
    nets = _nets(seed=9)
    B, T = 2, 7
    lens = [7, 5]
    noise, text = make_noise(B, T, d), make_text(B, d)
    V = RNG.standard_normal((B, T, d.feats))
    mask = RNG.random(V.shape) < 0.3
    ts, abar = _schedule(5)
    x = O.sample(nets, d, noise, text, lens, ts, abar, 2.5, known=V, known_mask=mask)
    free = O.sample(nets, d, noise, text, lens, ts, abar, 2.5)
    for b, n in enumerate(lens):
        np.testing.assert_array_equal(x[b, :n][mask[b, :n]], V[b, :n][mask[b, :n]])
        np.testing.assert_array_equal(x[b, n:], 0.0)
        assert np.abs(x[b, :n][~mask[b, :n]] - free[b, :n][~mask[b, :n]]).max() > 1e-6


def test_root_known_before_conversion():
    """With every root entry known, the body network reads G2L(V_root): the
    step's output no longer depends on the root network at all (a constraint
    applied only after CFG would leave the body reading the root network's own
    prediction)."""
    d = TINY
    B, T = 2, 6
    x_t = make_noise(B, T, d).astype(np.float64)
    text = make_text(B, d)
    V = RNG.standard_normal((B, T, d.feats))
    mask = np.zeros(V.shape, dtype=bool)
    mask[:, :, :d.root_feats] = True
    _, abar = O.linear_beta_schedule()
    a = _nets(seed=10)
    b = _nets(seed=10)
    b["root"] = _nets(seed=77)["root"]
    outs = [O.denoise_step(n, d, x_t, text, [6, 6], 30, abar[30], abar[29], 2.5, known=V, known_mask=mask)
            for n in (a, b)]
    np.testing.assert_array_equal(outs[0], outs[1])
    # the root network does matter without the constraint
    free = [O.denoise_step(n, d, x_t, text, [6, 6], 30, abar[30], abar[29], 2.5) for n in (a, b)]
    assert np.abs(free[0][..., d.root_feats:] - free[1][..., d.root_feats:]).max() > 1e-6
    # and the local root fed to the body is the conversion of V
    tr = {}
    O.denoise_step(a, d, x_t, text, [6, 6], 30, abar[30], abar[29], 2.5, trace=tr, known=V, known_mask=mask)
    np.testing.assert_allclose(tr["local_root"][B + 1], O.global_to_local_root(V[1, :, :5]), atol=0)


def _timeline_inputs(d, V, frames, seed=0):
    inp = timeline_inputs(V, frames, d, seed)
    return inp["text"], inp["noise"]


def test_timeline_seams_and_assembly():
    d = TINY
    nets = _nets(seed=12)
    frames, n_tr, V = [7, 6, 5], 2, 2
    text, noise = _timeline_inputs(d, V, frames)
    ts, abar = _schedule(4)
    segs = []
    out = O.timeline(nets, d, frames, text, noise, n_tr, ts, abar, 2.5, segments=segs)
    assert out.shape == (V, 7 + 4 + 3, d.feats)
    # the carried-over frames equal the previous segment's last frames exactly
    for k in range(1, 3):
        np.testing.assert_array_equal(segs[k][:, :n_tr], segs[k - 1][:, -n_tr:])
    np.testing.assert_array_equal(out, np.concatenate([segs[0], segs[1][:, n_tr:], segs[2][:, n_tr:]], axis=1))
    # segment 0 is an unconstrained sample
    np.testing.assert_array_equal(segs[0], O.sample(nets, d, noise[0], text[0], [7] * V, ts, abar, 2.5))
    # the tail conditions the next segment: without it segment 1 differs
    free1 = O.sample(nets, d, noise[1], text[1], [6] * V, ts, abar, 2.5)
    assert np.abs(free1[:, n_tr:] - segs[1][:, n_tr:]).max() > 1e-6


def test_timeline_without_transition_is_independent_segments():
    d = TINY
    nets = _nets(seed=13)
    frames, V = [5, 4], 2
    text, noise = _timeline_inputs(d, V, frames, seed=5)
    ts, abar = _schedule(3)
    out = O.timeline(nets, d, frames, text, noise, 0, ts, abar, 2.5)
    want = np.concatenate([O.sample(nets, d, noise[k], text[k], [T] * V, ts, abar, 2.5)
                           for k, T in enumerate(frames)], axis=1)
    np.testing.assert_array_equal(out, want)


def test_timeline_is_causal():
    """A later segment's prompt or noise never changes earlier output."""
    d = TINY
    nets = _nets(seed=14)
    frames, n_tr, V = [6, 5, 5], 2, 1
    text, noise = _timeline_inputs(d, V, frames, seed=9)
    ts, abar = _schedule(3)
    a = O.timeline(nets, d, frames, text, noise, n_tr, ts, abar, 2.5)
    text2 = text.copy()
    text2[2] = make_text(V, d, seed=999)
    noise2 = list(noise)
    noise2[2] = make_noise(V, 5, d, seed=998)
    b = O.timeline(nets, d, frames, text2, noise2, n_tr, ts, abar, 2.5)
    np.testing.assert_array_equal(a[:, :6 + 3], b[:, :6 + 3])
    assert np.abs(a[:, 9:] - b[:, 9:]).max() > 1e-6
