"""GPU parity of the FK decode (kimodo_fk) against the fp64 oracle
(oracle/kimodo_fk.py), through the C ABI.

Tolerance: positions max-abs 1e-4 m; rotation entries max-abs
1e-5 + 8 u / sin(theta_min). fp32 carries a unit roundoff u = 2^-24; a joint's
transform is at most 9 chained 3x3 products (heading plus depth 8) of
unit-norm factors and positions are O(1) (root N(0, 1), bones <= 0.45 m), so
well-conditioned frames agree to O(1e-6). Gram-Schmidt of the 6D form
amplifies rounding by 1 / sin(theta), theta the angle between the two
3-vectors; among 30,000 random pairs the smallest sin(theta) is ~0.01, so the
rotation bound takes the sample's own smallest value.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    from oracle import kimodo_fk as FK
    from synthetic.inputs import make_skeleton
    from text_motion_diffusion_amd import kimodo as K

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _, parents, offsets = make_skeleton()
    return dict(torch=torch, FK=FK, K=K, parents=parents, offsets=offsets, dev=torch.device("cuda:0"))


def _min_sin(motion):
    """Smallest sin of the angle between the two 3-vectors of any joint's 6D
    rotation in the sample (all-zero frames skipped)."""
    a = motion[:, 5:275].reshape(-1, 30, 9)[..., :6].astype(np.float64)
    a1, a2 = a[..., :3], a[..., 3:6]
    den = np.linalg.norm(a1, axis=-1) * np.linalg.norm(a2, axis=-1)
    keep = den > 0
    return float((np.linalg.norm(np.cross(a1, a2), axis=-1)[keep] / den[keep]).min())


def _run(env, motion, with_rot=True):
    torch = env["torch"]
    n = motion.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(motion, np.float32)).to(env["dev"])
    pos = torch.full((n, 30, 3), np.nan, device=env["dev"])
    rot = torch.full((n, 30, 3, 3), np.nan, device=env["dev"]) if with_rot else None
    env["K"].kimodo_fk(n, x, env["parents"], env["offsets"], pos, rot)
    torch.cuda.synchronize()
    return pos.cpu().numpy(), None if rot is None else rot.cpu().numpy()


@pytest.mark.parametrize("n", [1, 7, 8, 1001])
def test_fk_matches_oracle(env, n):
    """Random frames (N(0, 1) features: arbitrary 6D pairs, headings and root
    positions), frame counts around the 8 frames of a workgroup, one padded
    (all-zero) frame."""
    print(f"fk case n={n}", flush=True)
    motion = np.random.default_rng(n).standard_normal((n, 279)).astype(np.float32)
    if n > 1:
        motion[n // 2] = 0.0
    pos, rot = _run(env, motion)
    want_p, want_R = env["FK"].forward_kinematics(motion, env["parents"], env["offsets"])
    ep, er = float(np.abs(pos - want_p).max()), float(np.abs(rot - want_R).max())
    tol_r = 1e-5 + 8 * 2.0 ** -24 / _min_sin(motion)
    print(f"  positions max-abs {ep:.2e}, rotations max-abs {er:.2e} (bound {tol_r:.2e})", flush=True)
    assert ep <= 1e-4 and er <= tol_r
    if n > 1:
        assert np.all(pos[n // 2] == 0.0) and np.all(rot[n // 2] == 0.0)


def test_fk_without_rotations_and_of_a_sampled_clip(env):
    """The decode of real sampler output (a 1 + 1 layer model, 3 steps, one
    ragged clip whose padded frames decode to zeros), positions only."""
    from synthetic.inputs import Dims, bf16_bits_to_f32, make_noise, make_text, make_weights, round_to_bf16_bits
    from text_motion_diffusion_amd.session import Session

    K, torch = env["K"], env["torch"]
    dims = Dims(layers_root=1, layers_body=1)
    bits = [round_to_bf16_bits(a) for a in make_weights(dims, seed=9)]
    B, T = 2, 50
    lens = np.array([50, 31], np.int32)
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, 3)
    print("fk of a sampled clip", flush=True)
    sess = Session(bits, 1, 1, B, T, 3, K.KIMODO_BF16)
    x = sess.sample(torch.from_numpy(make_noise(B, T, dims)).to(env["dev"]),
                    torch.from_numpy(make_text(B, dims)).to(env["dev"]), lens, ts, ab, 2.5)
    pos = torch.full((B * T, 30, 3), np.nan, device=env["dev"])
    K.kimodo_fk(B * T, x, env["parents"], env["offsets"], pos)
    torch.cuda.synchronize()
    motion = x.cpu().numpy().reshape(B * T, 279)
    sess.close()
    pos = pos.cpu().numpy()
    want, _ = env["FK"].forward_kinematics(motion, env["parents"], env["offsets"])
    assert float(np.abs(pos - want).max()) <= 1e-4
    assert np.all(pos.reshape(B, T, 30, 3)[1, 31:] == 0.0)
