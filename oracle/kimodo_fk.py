"""Plain CPU oracle of the forward-kinematics decode of sampled motion, in
numpy float64.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module. It shares no code with the
HIP library.

The pages place an FK decode after the sampling loop that turns the motion
into joint positions and rotation matrices on the 30-joint skeleton (Kimodo
WebGPU README: feature list, "Architecture" diagram, "Model details" table:
SOMA30, output "joint positions (3D), rotation matrices, root trajectory,
foot contacts"). They give neither the feature layout nor the skeleton. The
readings, shared with the HIP kernel:

  * a frame is 279 features: the root stream (x, y, z, c, s) = root position
    (y up) and heading (c, s) = (cos psi, sin psi), as in
    ``kimodo_oracle.global_to_local_root``; then 30 joints x 9 features and 4
    foot contacts;
  * joint j's first 6 features are its local rotation (relative to its parent)
    in the continuous 6D form of Zhou et al., "On the Continuity of Rotation
    Representations in Neural Networks" (CVPR 2019): the first two columns of
    the rotation matrix, made orthonormal by Gram-Schmidt (``rotation_from_6d``);
    the other 3 are not used by FK;
  * the root joint's global rotation is the heading rotation about y
    (``heading_rotation``) times its local rotation; it sits at the root
    position; every other joint j has R_j = R_parent L_j and
    p_j = p_parent + R_parent o_j with o_j its offset in the parent's frame;
  * vector lengths below 1e-8 are clamped to 1e-8 before division (as in the
    root conversion), so an all-zero frame (a padded frame) decodes to zero
    rotations and every joint at the origin.

Pinned by tests/test_oracle_fk.py (library rotations, closed forms, a
hand-worked chain, bone lengths, yaw and translation equivariance, agreement
of the heading convention with the root conversion).
"""
from __future__ import annotations

import numpy as np

N_JOINTS = 30
JOINT_FEATS = 9
ROOT_FEATS = 5
EPS = 1e-8


def _normalize(v: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(v * v, axis=-1, keepdims=True))
    return v / np.maximum(n, EPS)


def rotation_from_6d(a: np.ndarray) -> np.ndarray:
    """[..., 6] = (a1, a2), two 3-vectors -> [..., 3, 3] with columns
    b1 = a1/|a1|, b2 = (a2 - (b1.a2) b1)/|...|, b3 = b1 x b2."""
    a = np.asarray(a, np.float64)
    a1, a2 = a[..., 0:3], a[..., 3:6]
    b1 = _normalize(a1)
    b2 = _normalize(a2 - np.sum(b1 * a2, axis=-1, keepdims=True) * b1)
    b3 = np.cross(b1, b2)
    return np.stack([b1, b2, b3], axis=-1)


def heading_rotation(c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Rotation about +y by the heading psi with (cos psi, sin psi) = (c, s) /
    |(c, s)|, in the convention of the root conversion: the ground-plane point
    x + i z is multiplied by cos psi + i sin psi, i.e. x' = c x - s z,
    z' = s x + c z. [...] -> [..., 3, 3]."""
    c = np.asarray(c, np.float64)
    s = np.asarray(s, np.float64)
    n = np.maximum(np.sqrt(c * c + s * s), EPS)
    hc, hs = c / n, s / n
    R = np.zeros(c.shape + (3, 3))
    R[..., 0, 0] = hc
    R[..., 0, 2] = -hs
    R[..., 1, 1] = 1.0
    R[..., 2, 0] = hs
    R[..., 2, 2] = hc
    return R


def forward_kinematics(motion: np.ndarray, parents, offsets):
    """motion [..., 279] -> (positions [..., 30, 3], rotations [..., 30, 3, 3])
    of every joint in the global frame."""
    x = np.asarray(motion, np.float64)
    parents = [int(p) for p in parents]
    offsets = np.asarray(offsets, np.float64)
    lead = x.shape[:-1]
    body = x[..., ROOT_FEATS:ROOT_FEATS + N_JOINTS * JOINT_FEATS].reshape(lead + (N_JOINTS, JOINT_FEATS))
    local = rotation_from_6d(body[..., 0:6])
    R = np.zeros(lead + (N_JOINTS, 3, 3))
    p = np.zeros(lead + (N_JOINTS, 3))
    for j in range(N_JOINTS):
        if parents[j] < 0:
            R[..., j, :, :] = heading_rotation(x[..., 3], x[..., 4]) @ local[..., j, :, :]
            p[..., j, :] = x[..., 0:3]
        else:
            q = parents[j]
            R[..., j, :, :] = R[..., q, :, :] @ local[..., j, :, :]
            p[..., j, :] = p[..., q, :] + R[..., q, :, :] @ offsets[j]
    return p, R
