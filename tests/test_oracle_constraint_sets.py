"""Pins of the constraint-set oracle (CPU only): the waypoint path against
exact rational arithmetic and its closed-form special cases, the covered
features against a brute-force ancestor search over the skeleton, and the
property the end-effector and full-body readings rest on: forward kinematics
of a motion that carries a set's entries puts the constrained joints exactly
where the reference pose puts them, whatever the free entries hold."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import kimodo_constraint_sets as C
from oracle import kimodo_fk as FK
from synthetic.inputs import make_skeleton

_, PARENTS, OFFSETS = make_skeleton()
RNG = np.random.default_rng(31)


def _path_exact(w, n):
    """The same path in exact rationals: waypoint i at frame i (n-1)/(m-1)."""
    m = len(w)
    out = []
    for f in range(n):
        if m == 1 or n == 1:
            out.append(tuple(Fraction(v) for v in w[0]))
            continue
        u = Fraction(f * (m - 1), n - 1)
        s = min(int(u), m - 2)
        a = u - s
        out.append(tuple(Fraction(w[s][k]) + a * (Fraction(w[s + 1][k]) - Fraction(w[s][k])) for k in range(2)))
    return out


@pytest.mark.parametrize("m,n", [(5, 180), (2, 2), (3, 7), (4, 30), (7, 5), (1, 9), (3, 1)])
def test_root_path_against_exact_rationals(m, n):
    w = np.round(RNG.uniform(-4, 4, size=(m, 2)), 3)
    got = C.root_path(w, n)
    want = np.array([[float(v) for v in p] for p in _path_exact(w.tolist(), n)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_root_path_hits_waypoints_and_is_linear_between():
    # the README's square: 5 waypoints over 181 frames, waypoint i at frame 45 i
    w = np.array([(0, 0), (3, 0), (3, 3), (0, 3), (0, 0)], float)
    p = C.root_path(w, 181)
    np.testing.assert_array_equal(p[::45], w)
    for s in range(4):
        seg = p[45 * s:45 * s + 46]
        np.testing.assert_allclose(np.diff(seg, 2, axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(np.abs(np.diff(seg, axis=0)).sum(axis=1), 3.0 / 45, atol=1e-12)


def test_chain_is_the_ancestor_set():
    for j in range(30):
        brute = {k for k in range(30) if _is_ancestor_or_self(k, j)}
        assert set(C.chain_to_root(PARENTS, j)) == brute
    assert C.chain_to_root(PARENTS, 0) == [0]


def _is_ancestor_or_self(k, j):
    while j >= 0:
        if j == k:
            return True
        j = int(PARENTS[j])
    return False


def test_covered_features_counts_and_layout():
    assert np.flatnonzero(C.covered_features(C.ROOT_PATH)).tolist() == [0, 2]
    fb = C.covered_features(C.FULL_BODY)
    assert fb.sum() == 5 + 270 and not fb[275:].any()
    left_hand = 10  # Hips, Spine, Spine1, Spine2, LeftShoulder, LeftArm, LeftForeArm, LeftHand
    ee = C.covered_features(C.END_EFFECTOR, left_hand, PARENTS)
    assert ee.sum() == 5 + 6 * 8
    assert ee[5 + 9 * 10:5 + 9 * 10 + 6].all() and not ee[5 + 9 * 10 + 6:5 + 9 * 11].any()
    assert not ee[5 + 9 * 12:5 + 9 * 13].any()  # RightShoulder is off the chain
    with pytest.raises(ValueError):
        C.covered_features(7)


@pytest.mark.parametrize("joint", [10, 15, 19, 24, 6])
def test_end_effector_pins_the_joint_under_fk(joint):
    T, frames = 12, [0, 5, 11]
    ref = RNG.standard_normal((len(frames), 279))
    known = np.zeros((T, 279))
    mask = np.zeros((T, 279), dtype=bool)
    C.apply_set(known, mask, C.END_EFFECTOR, frames, ref, joint, PARENTS)
    motion = np.where(mask, known, RNG.standard_normal((T, 279)))
    p, R = FK.forward_kinematics(motion, PARENTS, OFFSETS)
    p_ref, R_ref = FK.forward_kinematics(ref, PARENTS, OFFSETS)
    for i, f in enumerate(frames):
        for k in C.chain_to_root(PARENTS, joint):
            np.testing.assert_allclose(p[f, k], p_ref[i, k], rtol=0, atol=1e-12)
            np.testing.assert_allclose(R[f, k], R_ref[i, k], rtol=0, atol=1e-12)
        # joints off the chain stay free
        off = [k for k in range(30) if k not in C.chain_to_root(PARENTS, joint)]
        assert np.abs(p[f, off] - p_ref[i, off]).max() > 1e-3
    # frames without a key are untouched
    assert not mask[1:5].any() and not mask[6:11].any()


def test_full_body_pins_every_joint_and_leaves_contacts_free():
    T, frames = 6, [2, 4]
    ref = RNG.standard_normal((2, 279))
    known = np.zeros((T, 279))
    mask = np.zeros((T, 279), dtype=bool)
    C.apply_set(known, mask, C.FULL_BODY, frames, ref)
    motion = np.where(mask, known, RNG.standard_normal((T, 279)))
    p, R = FK.forward_kinematics(motion, PARENTS, OFFSETS)
    p_ref, R_ref = FK.forward_kinematics(ref, PARENTS, OFFSETS)
    np.testing.assert_allclose(p[frames], p_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(R[frames], R_ref, rtol=0, atol=1e-12)
    assert not mask[:, 275:].any()


def test_sets_combine_and_the_later_one_wins():
    T = 8
    known = np.zeros((T, 279))
    mask = np.zeros((T, 279), dtype=bool)
    a = np.full((1, 279), 1.0)
    b = np.full((1, 279), 2.0)
    C.apply_set(known, mask, C.FULL_BODY, [3], a)
    C.apply_set(known, mask, C.END_EFFECTOR, [3], b, 19, PARENTS)
    ee = C.covered_features(C.END_EFFECTOR, 19, PARENTS)
    fb = C.covered_features(C.FULL_BODY)
    np.testing.assert_array_equal(known[3, ee], 2.0)
    np.testing.assert_array_equal(known[3, fb & ~ee], 1.0)
    np.testing.assert_array_equal(mask[3], fb | ee)
