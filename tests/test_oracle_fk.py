"""Pins of the FK oracle (CPU only): library rotations, closed forms, a
hand-worked chain, bone lengths, equivariance under a global yaw and
translation, and agreement of the heading convention with the root
conversion."""
import numpy as np
import pytest
from scipy.spatial.transform import Rotation

from oracle import kimodo_fk as FK
from oracle import kimodo_oracle as O
from synthetic.inputs import make_skeleton

RNG = np.random.default_rng(2024)
_, PARENTS, OFFSETS = make_skeleton()


def _motion(n, rng=RNG):
    x = rng.standard_normal((n, 279))
    return x


def test_6d_of_a_rotation_gives_it_back():
    R = Rotation.random(200, random_state=7).as_matrix()
    a = np.concatenate([R[:, :, 0], R[:, :, 1]], axis=1)
    np.testing.assert_allclose(FK.rotation_from_6d(a), R, atol=1e-14)


def test_6d_gives_proper_rotations_and_ignores_scale_and_a1_component():
    a = RNG.standard_normal((500, 6))
    R = FK.rotation_from_6d(a)
    np.testing.assert_allclose(R @ np.swapaxes(R, 1, 2), np.broadcast_to(np.eye(3), R.shape), atol=1e-12)
    np.testing.assert_allclose(np.linalg.det(R), 1.0, atol=1e-12)
    b = a.copy()
    b[:, 0:3] *= 3.7
    b[:, 3:6] = 0.4 * a[:, 3:6] + 2.5 * a[:, 0:3]
    np.testing.assert_allclose(FK.rotation_from_6d(b), R, atol=1e-12)
    # the first column follows a1
    np.testing.assert_allclose(R[:, :, 0], a[:, 0:3] / np.linalg.norm(a[:, 0:3], axis=1, keepdims=True), atol=1e-14)


def test_identity_pose_is_the_rest_skeleton():
    """Identity local rotations and heading (1, 0): R_j = I and p_j = root +
    the sum of the offsets on the path from the root to j."""
    x = np.zeros((3, 279))
    x[:, 0:3] = RNG.standard_normal((3, 3))
    x[:, 3] = 2.0  # heading (2, 0): unit heading (1, 0)
    for j in range(30):
        x[:, 5 + 9 * j: 5 + 9 * j + 6] = [1, 0, 0, 0, 1, 0]
    p, R = FK.forward_kinematics(x, PARENTS, OFFSETS)
    np.testing.assert_allclose(R, np.broadcast_to(np.eye(3), R.shape), atol=1e-15)
    for j in range(30):
        want = x[:, 0:3].copy()
        k = j
        while PARENTS[k] >= 0:
            want += OFFSETS[k]
            k = PARENTS[k]
        np.testing.assert_allclose(p[:, j], want, atol=1e-12)


def test_hand_worked_chain():
    """Three joints in a line along +y. The root's local rotation is 90 degrees
    about +z (y -> -x); joint 1's is 90 degrees about +x (y -> +z); heading
    psi = 90 degrees maps (x, z) -> (-z, x). Worked by hand:
      root R0 = H Rz: y -> -x -> (0, 0, -1)  (x' = c x - s z = 0, z' = s x = -1)
      p1 = p0 + R0 (0, 1, 0) = p0 + (0, 0, -1)
      R1 = R0 Rx: y -> z -> R0 z = H (Rz z) = H z = (-1, 0, 0)
      p2 = p1 + R1 (0, 1, 0) = p0 + (0, 0, -1) + (-1, 0, 0)"""
    parents = [-1, 0, 1] + list(range(2, 29))  # the rest hangs off joint 2 and is not checked
    offsets = np.zeros((30, 3))
    offsets[1] = offsets[2] = [0, 1, 0]
    x = np.zeros((1, 279))
    x[0, 0:3] = [1.0, 2.0, 3.0]
    x[0, 3:5] = [0.0, 1.0]
    x[0, 5:11] = [0, 1, 0, -1, 0, 0]         # Rz(90): columns R e_x = (0,1,0), R e_y = (-1,0,0)
    x[0, 14:20] = [1, 0, 0, 0, 0, 1]         # Rx(90): columns R e_x = (1,0,0), R e_y = (0,0,1)
    for j in range(2, 30):
        x[0, 5 + 9 * j: 5 + 9 * j + 6] = [1, 0, 0, 0, 1, 0]
    p, _ = FK.forward_kinematics(x, parents, offsets)
    np.testing.assert_allclose(p[0, 0], [1, 2, 3], atol=1e-15)
    np.testing.assert_allclose(p[0, 1], [1, 2, 2], atol=1e-15)
    np.testing.assert_allclose(p[0, 2], [0, 2, 2], atol=1e-15)


def test_bone_lengths_are_kept():
    p, R = FK.forward_kinematics(_motion(50), PARENTS, OFFSETS)
    for j in range(1, 30):
        d = np.linalg.norm(p[:, j] - p[:, PARENTS[j]], axis=-1)
        np.testing.assert_allclose(d, np.linalg.norm(OFFSETS[j].astype(np.float64)), rtol=1e-12)


def test_global_yaw_and_translation_equivariance():
    """Turning the heading by psi0 and moving the root position by that yaw
    plus a translation moves every joint the same way."""
    x = _motion(40)
    psi0 = 0.83
    c0, s0 = np.cos(psi0), np.sin(psi0)
    H0 = FK.heading_rotation(np.array(c0), np.array(s0))
    t = np.array([0.3, -0.2, 1.5])
    y = x.copy()
    y[:, 0:3] = x[:, 0:3] @ H0.T + t
    y[:, 3] = c0 * x[:, 3] - s0 * x[:, 4]   # (c + i s)(c0 + i s0)
    y[:, 4] = s0 * x[:, 3] + c0 * x[:, 4]
    p, R = FK.forward_kinematics(x, PARENTS, OFFSETS)
    q, Q = FK.forward_kinematics(y, PARENTS, OFFSETS)
    np.testing.assert_allclose(q, p @ H0.T + t, atol=1e-12)
    np.testing.assert_allclose(Q, H0 @ R, atol=1e-12)


def test_heading_convention_matches_root_conversion():
    """The root conversion expresses each frame's displacement in that frame's
    heading: v_f = conj(h_f) d_f. The FK heading rotation of frame f must map
    (Re v_f, 0, Im v_f) back to the global displacement."""
    g = RNG.standard_normal((20, 5))
    l = O.global_to_local_root(g)
    H = FK.heading_rotation(g[:, 3], g[:, 4])
    for f in range(1, 20):
        back = H[f] @ np.array([l[f, 0], 0.0, l[f, 2]])
        np.testing.assert_allclose(back, [g[f, 0] - g[f - 1, 0], 0.0, g[f, 2] - g[f - 1, 2]], atol=1e-12)


def test_zero_frame_decodes_to_the_origin():
    p, R = FK.forward_kinematics(np.zeros((2, 279)), PARENTS, OFFSETS)
    assert np.all(p == 0.0) and np.all(R == 0.0)


@pytest.mark.parametrize("lead", [(4,), (2, 3)])
def test_leading_dimensions(lead):
    x = RNG.standard_normal(lead + (279,))
    p, R = FK.forward_kinematics(x, PARENTS, OFFSETS)
    flat_p, flat_R = FK.forward_kinematics(x.reshape(-1, 279), PARENTS, OFFSETS)
    np.testing.assert_array_equal(p.reshape(-1, 30, 3), flat_p)
    np.testing.assert_array_equal(R.reshape(-1, 30, 3, 3), flat_R)
