"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Tolerances: fp32 runs match the oracle to max-abs 2e-3 on every layer output
and stage; runs with bf16 weights (fp16 activations) match the final sampled
motion to relative L2 1e-2 over valid frames. (Every stage of the fp16 path is
also checked element by element, against bounds derived from fp16 rounding, in
tests/test_gpu_stages.py.) Padded frames must be exactly 0. Full-size
workloads compare against oracle outputs stored by tests/golden/make_golden.py,
after checking their metadata and the oracle source they were made with.
"""
import json
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def env():
    import torch

    from oracle import kimodo_oracle as O
    from text_motion_diffusion_amd import kimodo as K
    from text_motion_diffusion_amd.session import Session

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dict(torch=torch, O=O, K=K, Session=Session, dev=torch.device("cuda:0"))


def _rel_l2(got, want, lengths):
    num = den = 0.0
    for b, n in enumerate(lengths):
        num += float(np.sum((got[b, :n] - want[b, :n]) ** 2))
        den += float(np.sum(want[b, :n] ** 2))
    return (num / den) ** 0.5


def _to_dev(env, a):
    return env["torch"].from_numpy(np.ascontiguousarray(a)).to(env["dev"])


def _step_case(env, dims, dtype, B, T, lengths, t, w_scale=None, seed_shift=0):
    """Runs one traced step on the GPU and in the oracle; returns both."""
    from synthetic.inputs import bf16_bits_to_f32, make_noise, make_text, make_weights, round_to_bf16_bits

    O, K = env["O"], env["K"]
    w = make_weights(dims, seed=seed_shift)
    if dtype == K.KIMODO_BF16:
        bits = [round_to_bf16_bits(a) for a in w]
        w_dev, w_ref = bits, [bf16_bits_to_f32(b) for b in bits]
    else:
        w_dev = w_ref = w
    noise, text = make_noise(B, T, dims), make_text(B, dims)
    lengths = np.asarray(lengths, np.int32)
    _, abar = O.linear_beta_schedule()
    print(f"step case dtype={dtype} L={dims.layers_root}+{dims.layers_body} B={B} T={T} lengths={lengths.tolist()}",
          flush=True)
    sess = env["Session"](w_dev, dims.layers_root, dims.layers_body, B, T, 1, dtype)
    x_prev, tr = sess.denoise_step(_to_dev(env, noise), _to_dev(env, text), lengths, t, float(abar[t]),
                                   float(abar[t - 1]), 2.5, trace=True)
    env["torch"].cuda.synchronize()
    gpu = {k: v.float().cpu().numpy() for k, v in tr.items()}
    gpu["x_prev"] = x_prev.cpu().numpy()
    sess.close()
    ref = {}
    want = O.denoise_step(O.unpack_params(w_ref, dims), dims, noise, text, lengths, t, abar[t], abar[t - 1], 2.5,
                          trace=ref)
    ref["x_prev"] = want
    return gpu, ref, lengths


def _valid_rows_max_err(gpu_layers, ref_layers, lengths, B):
    """max |diff| over valid token rows of [L, 2B, S, d] traces."""
    err = 0.0
    for p in range(2 * B):
        n = int(lengths[p % B]) + 2
        err = max(err, float(np.abs(gpu_layers[:, p, :n] - ref_layers[:, p, :n]).max()))
    return err


def test_config0_per_layer_and_stages(env):
    """One fp32 DDIM step, 2 root + 2 body layers, B=1, T=60, t=50 -> 49."""
    from synthetic.inputs import dims_for

    dims = dims_for(0)
    gpu, ref, lens = _step_case(env, dims, env["K"].KIMODO_F32, 1, 60, [60], 50)
    ref_layers = np.concatenate([ref["layers_root"], ref["layers_body"]])
    per_layer = [_valid_rows_max_err(gpu["layers"][i:i + 1], ref_layers[i:i + 1], lens, 1)
                 for i in range(ref_layers.shape[0])]
    print("per-layer max abs:", per_layer)
    assert max(per_layer) <= 2e-3
    for k in ("root_out", "local_root", "body_out", "x0_hat", "x_prev"):
        e = float(np.abs(gpu[k] - ref[k]).max())
        print(k, e)
        assert e <= 2e-3, k


@pytest.mark.parametrize("B,T,lengths", [(3, 70, [70, 45, 1]), (2, 200, [200, 131]),
                                         (8, 170, [170, 1, 99, 170, 170, 170, 170, 133])])
def test_fp32_ragged_tiles(env, B, T, lengths):
    """Several GEMM and attention tiles with ragged tails, masks, a 1-frame clip.
    The first two shapes run both guidance groups as one chain; 8 x 170 frames
    (2,256 packed token rows) runs them as two concurrent chains."""
    from synthetic.inputs import Dims

    dims = Dims(layers_root=1, layers_body=1)
    gpu, ref, lens = _step_case(env, dims, env["K"].KIMODO_F32, B, T, lengths, 73)
    ref_layers = np.concatenate([ref["layers_root"], ref["layers_body"]])
    assert _valid_rows_max_err(gpu["layers"], ref_layers, lens, B) <= 2e-3
    for b, n in enumerate(lens):
        assert np.abs(gpu["x_prev"][b, :n] - ref["x_prev"][b, :n]).max() <= 2e-3
        assert np.all(gpu["x_prev"][b, n:] == 0.0)


def test_bf16_step_small(env):
    from synthetic.inputs import Dims

    dims = Dims(layers_root=2, layers_body=2)
    gpu, ref, lens = _step_case(env, dims, env["K"].KIMODO_BF16, 2, 70, [70, 33], 60)
    ref_layers = np.concatenate([ref["layers_root"], ref["layers_body"]])
    for i in range(ref_layers.shape[0]):
        num = den = 0.0
        for p in range(4):
            n = int(lens[p % 2]) + 2
            num += float(np.sum((gpu["layers"][i, p, :n] - ref_layers[i, p, :n]) ** 2))
            den += float(np.sum(ref_layers[i, p, :n] ** 2))
        print("layer", i, "rel-L2", (num / den) ** 0.5)
        assert (num / den) ** 0.5 <= 1e-2
    r = _rel_l2(gpu["x_prev"], ref["x_prev"], lens)
    print("x_prev rel-L2", r)
    assert r <= 1e-2
    for b, n in enumerate(lens):
        assert np.all(gpu["x_prev"][b, n:] == 0.0)


@pytest.mark.parametrize("dtype_name,B,T,lengths", [
    ("bf16", 2, 1, [1, 1]),            # 3-token sequences: the fused kernel's 160-row tile is almost all padding
    ("f32", 2, 1, [1, 1]),
    ("bf16", 2, 700, [700, 333]),      # 702 tokens, 2 per chain: the 16-query kernel in 15 chunks, long key loop
    ("f32", 1, 700, [517]),
    ("bf16", 512, 6, "mixed"),         # maximum batch: 1024 sequences per step
])
def test_edge_shapes(env, dtype_name, B, T, lengths):
    """Degenerate and extreme shapes on a 1 + 1 layer model, one step at t = 37:
    fp32 to max-abs 2e-3 on every layer and the update, fp16 compute to rel-L2
    1e-2; padded frames exactly 0."""
    from synthetic.inputs import Dims

    K = env["K"]
    if lengths == "mixed":
        lengths = [1 + (7 * b) % T for b in range(B)]
    dims = Dims(layers_root=1, layers_body=1)
    dtype = K.KIMODO_F32 if dtype_name == "f32" else K.KIMODO_BF16
    gpu, ref, lens = _step_case(env, dims, dtype, B, T, lengths, 37)
    ref_layers = np.concatenate([ref["layers_root"], ref["layers_body"]])
    if dtype == K.KIMODO_F32:
        err = _valid_rows_max_err(gpu["layers"], ref_layers, lens, B)
        print(f"  layers max-abs {err:.3e}", flush=True)
        assert err <= 2e-3
        for b, n in enumerate(lens):
            assert np.abs(gpu["x_prev"][b, :n] - ref["x_prev"][b, :n]).max() <= 2e-3
    else:
        for i in range(ref_layers.shape[0]):
            num = den = 0.0
            for p in range(2 * B):
                n = int(lens[p % B]) + 2
                num += float(np.sum((gpu["layers"][i, p, :n] - ref_layers[i, p, :n]) ** 2))
                den += float(np.sum(ref_layers[i, p, :n] ** 2))
            print(f"  layer {i} rel-L2 {(num / den) ** 0.5:.3e}", flush=True)
            assert (num / den) ** 0.5 <= 1e-2
        r = _rel_l2(gpu["x_prev"], ref["x_prev"], lens)
        print(f"  x_prev rel-L2 {r:.3e}", flush=True)
        assert r <= 1e-2
    for b, n in enumerate(lens):
        assert np.all(gpu["x_prev"][b, n:] == 0.0)


def _bf16_session(env, dims, max_batch, max_frames, max_steps, zero_heads=False):
    from synthetic.inputs import make_weights, round_to_bf16_bits, weight_specs

    w = make_weights(dims)
    if zero_heads:
        names = [n for n, _, _ in weight_specs(dims)]
        for n in ("root.out.W", "body.out.W"):
            w[names.index(n)] = np.zeros_like(w[names.index(n)])
    bits = [round_to_bf16_bits(a) for a in w]
    return env["Session"](bits, dims.layers_root, dims.layers_body, max_batch, max_frames, max_steps,
                          env["K"].KIMODO_BF16), bits


@pytest.mark.parametrize("B,T,lengths", [(2, 40, [40, 29]),
                                         (10, 140, [140, 11, 140, 96, 140, 140, 57, 133, 140, 140])])
def test_graph_replay_equals_eager_steps_and_is_deterministic(env, B, T, lengths):
    """Two samples (graph replays) and the eager steps agree bit for bit, with
    both guidance groups in one chain (2 x 40 frames) and as two concurrent
    chains (10 x 140 frames, 2,368 packed token rows)."""
    from synthetic.inputs import Dims, make_noise, make_text

    K, torch = env["K"], env["torch"]
    dims = Dims(layers_root=2, layers_body=2)
    S = 4
    print(f"graph vs eager B={B} T={T} lengths={lengths}", flush=True)
    sess, _ = _bf16_session(env, dims, B, T, S)
    noise, text = _to_dev(env, make_noise(B, T, dims)), _to_dev(env, make_text(B, dims))
    lengths = np.array(lengths, np.int32)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    out1 = sess.sample(noise, text, lengths, ts, ab, 2.5).clone()
    out2 = sess.sample(noise, text, lengths, ts, ab, 2.5).clone()
    x = noise.clone()
    for k in range(S - 1, -1, -1):
        x = sess.denoise_step(x, text, lengths, int(ts[k]), float(ab[k]), float(ab[k - 1]) if k else 1.0, 2.5)
    torch.cuda.synchronize()
    sess.close()
    for name, other in (("second sample", out2), ("eager steps", x)):
        if not torch.equal(out1, other):
            d = (out1 - other).abs()
            idx = (d > 0).nonzero()
            print(f"  {name} differs: max {d.max().item():.3e}, {idx.shape[0]} elements, clips "
                  f"{sorted(set(idx[:, 0].tolist()))}, frames {idx[:, 1].min().item()}..{idx[:, 1].max().item()}, "
                  f"features {idx[:, 2].min().item()}..{idx[:, 2].max().item()}", flush=True)
    assert torch.equal(out1, out2)
    assert torch.equal(out1, x)


def test_concurrent_chains_do_not_share_buffers(env):
    """Regression: the two guidance groups run as concurrent kernel chains in
    the captured step. Their input-projection rows once overlapped (the root
    and body inputs have different widths), so a chain's root input could be
    overwritten by the other chain's body input when the chains drifted apart
    in time; at 1 clip of 37 frames about half of fresh sessions gave a first
    sample different from the rest. Fresh sessions: two samples and the eager
    steps agree bit for bit."""
    from synthetic.inputs import Dims, make_noise, make_text

    K, torch = env["K"], env["torch"]
    dims = Dims(layers_root=2, layers_body=2)
    # up to 2,048 packed token rows (twice the sum of length + 2 rounded up to
    # 8) the step runs both groups as one chain; the last two shapes run two
    # concurrent chains (P = 10 and P = 9 sequences each)
    for B, T, lens in ((1, 37, [37]), (2, 23, [23, 11]), (10, 140, [140, 77, 140, 3, 120, 140, 64, 101, 140, 140]),
                       (9, 150, [150, 150, 9, 150, 88, 150, 131, 150, 150])):
        S = 3
        noise, text = _to_dev(env, make_noise(B, T, dims)), _to_dev(env, make_text(B, dims))
        ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
        for session in range(4):
            print(f"fresh session {session}, B={B} T={T}", flush=True)
            sess, _ = _bf16_session(env, dims, B, T, S)
            first = sess.sample(noise, text, lens, ts, ab, 2.5).clone()
            second = sess.sample(noise, text, lens, ts, ab, 2.5).clone()
            x = noise.clone()
            for k in range(S - 1, -1, -1):
                x = sess.denoise_step(x, text, lens, int(ts[k]), float(ab[k]), float(ab[k - 1]) if k else 1.0, 2.5)
            torch.cuda.synchronize()
            sess.close()
            assert torch.equal(first, second) and torch.equal(first, x)


def test_stub_heads_sampler_closed_form(env):
    """Output heads' weights zeroed: x0_hat is the heads' bias for every input,
    so the last step returns exactly [b_out_root || b_out_body] on valid frames."""
    from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text, weight_specs

    K, torch = env["K"], env["torch"]
    dims = Dims(layers_root=2, layers_body=2)
    B, T, S = 3, 50, 10
    sess, bits = _bf16_session(env, dims, B, T, S, zero_heads=True)
    names = [n for n, _, _ in weight_specs(dims)]
    xstar = np.concatenate([bf16_bits_to_f32(bits[names.index("root.out.b")]),
                            bf16_bits_to_f32(bits[names.index("body.out.b")])])
    lengths = np.array([50, 17, 1], np.int32)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    out = sess.sample(_to_dev(env, make_noise(B, T, dims)), _to_dev(env, make_text(B, dims)), lengths, ts, ab, 2.5)
    got = out.cpu().numpy()
    sess.close()
    for b, n in enumerate(lengths):
        np.testing.assert_array_equal(got[b, :n], np.broadcast_to(xstar, (n, 279)))
        assert np.all(got[b, n:] == 0.0)


@pytest.mark.parametrize("B,T,T_own,lengths", [
    (1, 64, 37, [37]),
    # 8 x 150 would run two chains by 2 B (T + 2) = 2,432 rows, but its packed
    # rows (752) and those of the same clips at T = 60 both make one chain
    (8, 150, 60, [60, 17, 60, 33, 60, 1, 60, 45]),
    # two concurrent chains of 16 sequences each on the fused QKV + attention
    # kernel, at T = 150 and at the clips' own longest length
    (16, 150, 140, [140, 133, 140, 140, 97, 140, 140, 140, 12, 140, 140, 140, 140, 71, 140, 140]),
])
def test_truncation_invariance(env, B, T, T_own, lengths):
    """Clips padded to T give, bit for bit, the same valid frames as the same
    clips run at T = their longest length: every launch is sized by the packed
    token rows (each sequence's length + 2, rounded up to 8), the choice of one
    or two kernel chains is made on those rows, and attention never gives a
    padded key weight, so both runs take the same kernels, partitions and
    summation orders. Both also match the oracle (fp16 path, rel-L2 1e-2) and
    padded frames are exactly 0."""
    from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text

    K, O = env["K"], env["O"]
    dims = Dims(layers_root=2, layers_body=2)
    assert max(lengths) == T_own
    sess, bits = _bf16_session(env, dims, B, T, 3)
    noise, text = make_noise(B, T, dims), make_text(B, dims)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, 3)
    print(f"truncation B={B} T={T} vs {T_own}", flush=True)
    full = sess.sample(_to_dev(env, noise), _to_dev(env, text), lengths, ts, ab, 2.5).cpu().numpy()
    own = sess.sample(_to_dev(env, noise[:, :T_own]), _to_dev(env, text), lengths, ts, ab, 2.5).cpu().numpy()
    sess.close()
    for b, n in enumerate(lengths):
        assert np.all(full[b, n:] == 0.0) and np.all(own[b, n:] == 0.0)
    diff = np.abs(full[:, :T_own] - own)
    print(f"  padded vs own length: {int((diff > 0).sum())} elements differ, max {diff.max():.3e}", flush=True)
    assert np.array_equal(full[:, :T_own], own)
    _, abar_ref = O.linear_beta_schedule()
    want = O.sample(O.unpack_params([bf16_bits_to_f32(b) for b in bits], dims), dims, noise[:, :T_own], text,
                    lengths, O.ddim_timesteps(3), abar_ref, 2.5)
    r = _rel_l2(own, want, lengths)
    print(f"  rel-L2 against the oracle {r:.3e}", flush=True)
    assert r <= 1e-2


def test_lengths_change_between_samples(env):
    """One session, the same B and T, three samples with different lengths:
    token rows are packed by length, so the lengths fix the step graph's grid
    sizes, and a change of lengths updates the kept graph in place. Each sample
    matches the oracle (fp16 path, rel-L2 1e-2), padded frames are 0, and
    repeating the first lengths reproduces its result bit for bit."""
    from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text

    K, O = env["K"], env["O"]
    dims = Dims(layers_root=2, layers_body=2)
    B, T, S = 3, 40, 3
    sess, bits = _bf16_session(env, dims, B, T, S)
    noise, text = make_noise(B, T, dims), make_text(B, dims)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    _, abar_ref = O.linear_beta_schedule()
    nets = O.unpack_params([bf16_bits_to_f32(b) for b in bits], dims)
    outs = []
    for lens in ([40, 17, 33], [5, 40, 1], [40, 17, 33]):
        print(f"lengths {lens}", flush=True)
        got = sess.sample(_to_dev(env, noise), _to_dev(env, text), lens, ts, ab, 2.5).cpu().numpy()
        want = O.sample(nets, dims, noise, text, lens, O.ddim_timesteps(S), abar_ref, 2.5)
        for b, n in enumerate(lens):
            assert np.all(got[b, n:] == 0.0)
        r = _rel_l2(got, want, lens)
        print(f"  rel-L2 {r:.3e}, graphs (instantiated, updated) {sess.graph_stats()}", flush=True)
        assert r <= 1e-2
        outs.append(got)
    assert sess.graph_stats() == (1, 2)
    sess.close()
    assert np.array_equal(outs[0], outs[2])


def test_fused_attention_short_sequences(env):
    """8 clips x 100 frames: both guidance groups in one chain of 16
    sequences of at most 160 tokens, so the fused QKV + attention kernel
    runs, sized by the longest sequence of the call (4, 1 and 2 row blocks of
    32 below). Each sample matches the oracle (fp16 path, rel-L2 1e-2) and
    padded frames are 0."""
    from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text

    K, O = env["K"], env["O"]
    dims = Dims(layers_root=2, layers_body=2)
    B, T, S = 8, 100, 3
    sess, bits = _bf16_session(env, dims, B, T, S)
    noise, text = make_noise(B, T, dims), make_text(B, dims)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    _, abar_ref = O.linear_beta_schedule()
    nets = O.unpack_params([bf16_bits_to_f32(b) for b in bits], dims)
    for lens in ([100, 37, 64, 90, 12, 77, 50, 99], [30, 20, 25, 12, 1, 30, 7, 16],
                 [60, 61, 62, 1, 5, 40, 62, 33]):
        print(f"lengths {lens}", flush=True)
        got = sess.sample(_to_dev(env, noise), _to_dev(env, text), lens, ts, ab, 2.5).cpu().numpy()
        want = O.sample(nets, dims, noise, text, lens, O.ddim_timesteps(S), abar_ref, 2.5)
        for b, n in enumerate(lens):
            assert np.all(got[b, n:] == 0.0)
        r = _rel_l2(got, want, lens)
        print(f"  rel-L2 {r:.3e}", flush=True)
        assert r <= 1e-2
    sess.close()


def test_fused_attention_odd_sequence_count(env):
    """17 clips x 60 frames: 2,080 packed token rows, so two concurrent chains
    of 17 sequences each take the fused QKV + attention kernel, whose grid
    pairs heads and sequence parities per XCD and leaves one slot empty for
    an odd count. Every clip matches the oracle on its own (fp16 path, rel-L2
    1e-2) and padded frames are 0."""
    from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text

    K, O = env["K"], env["O"]
    dims = Dims(layers_root=2, layers_body=2)
    B, T, S = 17, 60, 2
    lens = [60] * B
    lens[1], lens[8], lens[16] = 45, 23, 59
    assert 2 * sum((n + 2 + 7) // 8 * 8 for n in lens) > 2048  # two chains
    sess, bits = _bf16_session(env, dims, B, T, S)
    noise, text = make_noise(B, T, dims), make_text(B, dims)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    _, abar_ref = O.linear_beta_schedule()
    nets = O.unpack_params([bf16_bits_to_f32(b) for b in bits], dims)
    got = sess.sample(_to_dev(env, noise), _to_dev(env, text), lens, ts, ab, 2.5).cpu().numpy()
    sess.close()
    want = O.sample(nets, dims, noise, text, lens, O.ddim_timesteps(S), abar_ref, 2.5)
    worst = 0.0
    for b, n in enumerate(lens):
        assert np.all(got[b, n:] == 0.0)
        worst = max(worst, _rel_l2(got[b:b + 1], want[b:b + 1], [n]))
    print(f"  worst clip rel-L2 {worst:.3e}", flush=True)
    assert worst <= 1e-2


def test_attention_eight_sequences_past_fused_limit(env):
    """4 clips x 190 frames with the longest at 190 (192 tokens): 8 sequences,
    but past the fused kernel's 160 tokens, so the QKV projection and the
    attention kernel run apart, the latter chunked by the longest sequence.
    Matches the oracle (fp16 path, rel-L2 1e-2); padded frames are 0."""
    from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text

    K, O = env["K"], env["O"]
    dims = Dims(layers_root=2, layers_body=2)
    B, T, S = 4, 190, 2
    lens = [190, 12, 100, 161]
    sess, bits = _bf16_session(env, dims, B, T, S)
    noise, text = make_noise(B, T, dims), make_text(B, dims)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    _, abar_ref = O.linear_beta_schedule()
    nets = O.unpack_params([bf16_bits_to_f32(b) for b in bits], dims)
    got = sess.sample(_to_dev(env, noise), _to_dev(env, text), lens, ts, ab, 2.5).cpu().numpy()
    sess.close()
    want = O.sample(nets, dims, noise, text, lens, O.ddim_timesteps(S), abar_ref, 2.5)
    for b, n in enumerate(lens):
        assert np.all(got[b, n:] == 0.0)
    r = _rel_l2(got, want, lens)
    print(f"rel-L2 {r:.3e}", flush=True)
    assert r <= 1e-2


def test_graph_update_two_chains(env):
    """10 clips x 140 frames (2,144 packed token rows for both length sets: the
    two guidance groups run as two concurrent chains in the graph). A graph
    updated in place for new lengths gives the same bits as a fresh session's
    graph for those lengths."""
    from synthetic.inputs import Dims, make_noise, make_text

    K = env["K"]
    dims = Dims(layers_root=2, layers_body=2)
    B, T, S = 10, 140, 3
    noise, text = make_noise(B, T, dims), make_text(B, dims)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    lens_a = [140, 90, 33, 140, 7, 121, 140, 64, 140, 140]
    lens_b = [12, 140, 140, 71, 140, 1, 99, 140, 140, 140]
    s1, _ = _bf16_session(env, dims, B, T, S)
    print("session 1: lengths a, then b", flush=True)
    s1.sample(_to_dev(env, noise), _to_dev(env, text), lens_a, ts, ab, 2.5)
    got = s1.sample(_to_dev(env, noise), _to_dev(env, text), lens_b, ts, ab, 2.5).cpu().numpy()
    print(f"  graphs (instantiated, updated) {s1.graph_stats()}", flush=True)
    assert s1.graph_stats() == (1, 1)
    s1.close()
    s2, _ = _bf16_session(env, dims, B, T, S)
    print("session 2: lengths b", flush=True)
    want = s2.sample(_to_dev(env, noise), _to_dev(env, text), lens_b, ts, ab, 2.5).cpu().numpy()
    s2.close()
    for b, n in enumerate(lens_b):
        assert np.all(got[b, n:] == 0.0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bad", ["bf16 matrix past the fp16 range", "NaN in a LayerNorm gain"])
def test_weights_outside_the_compute_type_are_refused(env, bad):
    """A bf16 weight beyond 65504 (it would convert to inf in fp16) or a NaN
    weight: the first call on the ctx returns KIMODO_EWEIGHTS after set-up has
    checked every converted value, and so does every later call."""
    from synthetic.inputs import Dims, make_noise, make_text, make_weights, round_to_bf16_bits, weight_specs

    K = env["K"]
    dims = Dims(layers_root=1, layers_body=1)
    w = make_weights(dims, seed=3)
    names = [n for n, _, _ in weight_specs(dims)]
    if bad.startswith("bf16"):
        w[names.index("body.layer0.ff1.W")][3, 7] = 98304.0  # exactly representable in bf16
    else:
        w[names.index("root.layer0.ln1.g")][11] = np.nan
    bits = [round_to_bf16_bits(a) for a in w]
    sess = env["Session"](bits, 1, 1, 2, 16, 2, K.KIMODO_BF16)
    B, T = 2, 16
    x, text = _to_dev(env, make_noise(B, T, dims)), _to_dev(env, make_text(B, dims))
    for _ in range(2):
        with pytest.raises(K.KimodoError, match="EWEIGHTS"):
            sess.denoise_step(x, text, [T, T], 50, 0.5, 0.6, 2.5)
    sess.close()


@pytest.mark.parametrize("dtype_name,B", [("bf16", 4), ("bf16", 8), ("f32", 4)])
def test_nonfinite_clip_does_not_leak_into_later_calls(env, dtype_name, B):
    """A clip whose noise is NaN leaves NaN in its own activation rows and in
    its key positions of the transposed V buffer. Later calls pack other
    lengths over those rows, and attention reads key positions past each
    sequence's end (with weight 0) from that buffer; the kernels replace those
    positions by zeros, so the later samples are finite, match the oracle and
    have zero padded frames. bf16 with 4 clips: separate QKV projection and
    attention kernel; bf16 with 8 clips: fused QKV + attention kernel; fp32:
    the fp32 attention kernel."""
    from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text, make_weights, round_to_bf16_bits

    K, O = env["K"], env["O"]
    dims = Dims(layers_root=2, layers_body=2)
    T, S = 100, 2
    w = make_weights(dims)
    if dtype_name == "bf16":
        bits = [round_to_bf16_bits(a) for a in w]
        w_dev, w_ref, dtype = bits, [bf16_bits_to_f32(b) for b in bits], K.KIMODO_BF16
    else:
        w_dev, w_ref, dtype = w, w, K.KIMODO_F32
    sess = env["Session"](w_dev, 2, 2, B, T, S, dtype)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    _, abar_ref = O.linear_beta_schedule()
    nets = O.unpack_params(w_ref, dims)
    text = make_text(B, dims)
    bad = make_noise(B, T, dims)
    bad[1] = np.nan
    print(f"{dtype_name} B={B}: a NaN clip, then finite clips at other lengths", flush=True)
    first = sess.sample(_to_dev(env, bad), _to_dev(env, text), [T] * B, ts, ab, 2.5).cpu().numpy()
    assert np.all(np.isnan(first[1]))
    for T_call, lens in ((T, [37 + (23 * b) % 60 for b in range(B)]), (60, [60 - (7 * b) % 50 for b in range(B)])):
        noise = make_noise(B, T_call, dims, seed=3)
        got = sess.sample(_to_dev(env, noise), _to_dev(env, text), lens, ts, ab, 2.5).cpu().numpy()
        assert np.all(np.isfinite(got))
        for b, n in enumerate(lens):
            assert np.all(got[b, n:] == 0.0)
        want = O.sample(nets, dims, noise, text, lens, O.ddim_timesteps(S), abar_ref, 2.5)
        if dtype == K.KIMODO_F32:
            err = max(float(np.abs(got[b, :n] - want[b, :n]).max()) for b, n in enumerate(lens))
            print(f"  T={T_call}: max-abs {err:.3e}", flush=True)
            assert err <= 2e-3
        else:
            r = _rel_l2(got, want, lens)
            print(f"  T={T_call}: rel-L2 {r:.3e}", flush=True)
            assert r <= 1e-2
    sess.close()


# --- full-size workloads against stored oracle outputs --------------------
@pytest.mark.parametrize("B,T,lengths", [
    # two chains of 16 sequences on the fused QKV + attention kernel
    (16, 150, [150, 133, 150, 150, 97, 150, 150, 150, 12, 150, 150, 150, 150, 71, 150, 150]),
    # 32 ragged clips: the 32-query attention kernel, partial last key blocks
    (32, 180, [180, 61, 177, 130, 180, 99, 63, 180, 145, 180, 71, 180, 180, 88, 179, 180,
               64, 180, 123, 180, 180, 75, 180, 180, 160, 180, 180, 93, 180, 180, 118, 180]),
    # one clip: the 16-query attention kernel and split-K with the LayerNorm
    (1, 150, [117]),
])
def test_workspace_contents_do_not_matter(env, B, T, lengths):
    """Two sessions with the same weights, one workspace filled with 0xFF
    bytes (NaN in fp16 and fp32) and one with zeros before the first call,
    give bit for bit the same samples: no kernel reads a workspace byte that
    the set-up or the call itself has not written (key positions past a
    sequence's end, dead packed rows, split-K partials, Vt padding)."""
    from synthetic.inputs import Dims, make_noise, make_text

    K = env["K"]
    dims = Dims(layers_root=2, layers_body=2)
    print(f"workspace contents B={B} T={T}", flush=True)
    out = []
    for fill in (0xFF, 0x00):
        sess, _ = _bf16_session(env, dims, B, T, 3)
        sess.workspace.fill_(fill)
        noise, text = make_noise(B, T, dims), make_text(B, dims)
        ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, 3)
        out.append(sess.sample(_to_dev(env, noise), _to_dev(env, text), lengths, ts, ab, 2.5).cpu().numpy())
        sess.close()
    assert np.all(np.isfinite(out[0]))
    diff = np.abs(out[0] - out[1])
    print(f"  {int((diff > 0).sum())} elements differ", flush=True)
    assert np.array_equal(out[0], out[1])


@pytest.fixture(scope="module")
def full_session(env):
    from synthetic.inputs import Dims

    sess, _ = _bf16_session(env, Dims(), 128, 300, 100)
    yield sess
    sess.close()


def _golden(config, clip):
    path = os.path.join(GOLDEN, f"sample_c{config}_clip{clip}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing oracle output {path}: run tests/golden/make_golden.py")
    z = np.load(path, allow_pickle=False)
    return z["x0"], json.loads(str(z["meta"]))


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_full_size_sample_vs_oracle(env, full_session, config):
    import sys

    sys.path.insert(0, GOLDEN)
    from make_golden import TARGETS, clips_for

    from synthetic.inputs import CONFIGS, make_lengths, make_noise, make_text

    K = env["K"]
    c = CONFIGS[config]
    B, T, S = c["B"], c["T"], c["steps"]
    lengths = make_lengths(B, T, c["lengths"])
    clips = clips_for(*TARGETS[f"c{config}"])
    goldens = {}
    from make_golden import oracle_sha

    sha = oracle_sha()
    for b in clips:
        x0, meta = _golden(config, b)
        # metadata gate before any array comparison: the stored output was made
        # by this oracle source, for this workload, clip and length
        assert meta["oracle_sha256"] == sha, f"clip {b}: stored output made by another oracle source"
        assert (meta["config"], meta["clip"], meta["length"], meta["B"], meta["T"], meta["steps"],
                meta["cfg_scale"], meta["layers"], meta["dtype"]) == (config, b, int(lengths[b]), B, T, S,
                                                                       c["cfg_scale"], 16, "bf16")
        goldens[b] = x0
    print(f"config {config}: B={B} T={T} S={S}, clips {clips}", flush=True)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    out = full_session.sample(_to_dev(env, make_noise(B, T)), _to_dev(env, make_text(B)), lengths, ts, ab,
                              c["cfg_scale"]).cpu().numpy()
    assert np.all(np.isfinite(out))
    for b, want in goldens.items():
        n = int(lengths[b])
        r = _rel_l2(out[b:b + 1, :n], want[None, :n], [n])
        print(f"config {config} clip {b} (length {n}): rel-L2 {r:.3e}", flush=True)
        assert r <= 1e-2
        assert np.all(out[b, n:] == 0.0)
    for b in range(B):
        assert np.all(out[b, int(lengths[b]):] == 0.0)


@pytest.mark.parametrize("dtype_name,schedule,S", [("f32", "cosine", 15), ("bf16", "cosine", 20),
                                                   ("bf16", "linear", 35)])
def test_schedule_and_step_count_variants(env, dtype_name, schedule, S):
    """The sampler under other schedules and step counts (the pages' cosine
    schedule; 15 / 20 / 35 steps), on a 2 + 2 layer model small enough for the
    oracle to run the whole chain: the GPU takes its tables from the library's
    schedule functions, the oracle from its own. fp32: max-abs 2e-3 on the
    final motion; bf16: rel-L2 1e-2. Padded frames are exactly 0."""
    from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text, make_weights, round_to_bf16_bits

    O, K, Session = env["O"], env["K"], env["Session"]
    dims = Dims(layers_root=2, layers_body=2)
    B, T, w_cfg = 2, 60, 2.5
    lengths = np.array([60, 41], np.int32)
    w = make_weights(dims, seed=5)
    dtype = K.KIMODO_F32 if dtype_name == "f32" else K.KIMODO_BF16
    if dtype == K.KIMODO_BF16:
        bits = [round_to_bf16_bits(a) for a in w]
        w_dev, w_ref = bits, [bf16_bits_to_f32(b) for b in bits]
    else:
        w_dev = w_ref = w
    noise, text = make_noise(B, T, dims, seed=11), make_text(B, dims, seed=12)
    print(f"schedule case {dtype_name} {schedule} S={S} B={B} T={T} lengths={lengths.tolist()}", flush=True)

    if schedule == "cosine":
        ts, ab = K.kimodo_make_cosine_schedule(100, 0.008, 0.999, S)
        _, abar_ref = O.cosine_beta_schedule()
    else:
        ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
        _, abar_ref = O.linear_beta_schedule()
    sess = Session(w_dev, 2, 2, B, T, max_steps=S, dtype=dtype)
    try:
        got = sess.sample(_to_dev(env, noise), _to_dev(env, text), lengths, ts, ab, w_cfg).cpu().numpy()
    finally:
        sess.close()
    nets = O.unpack_params(w_ref, dims)
    want = O.sample(nets, dims, noise, text, lengths, O.ddim_timesteps(S), abar_ref, w_cfg)
    assert np.all(np.isfinite(got))
    for b in range(B):
        assert np.all(got[b, lengths[b]:] == 0.0)
    if dtype == K.KIMODO_F32:
        err = max(float(np.max(np.abs(got[b, :n] - want[b, :n]))) for b, n in enumerate(lengths))
        print(f"  max-abs {err:.3e}", flush=True)
        assert err <= 2e-3
    else:
        r = _rel_l2(got, want, lengths)
        print(f"  rel-L2 {r:.3e}", flush=True)
        assert r <= 1e-2
