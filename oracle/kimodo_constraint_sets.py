"""Plain CPU oracle of the constraint sets that fill the known-entry
constraint (``kimodo_oracle.apply_known``), in numpy float64.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module. It shares no code with the
HIP library.

The kimodo-fast README ("Python" section) constrains generation with a pinned
root path built from waypoints and a frame count, and names two more kinds of
constraint set that Kimodo ships: end effectors (hand and foot variants) and
full-body poses. It gives no definition of any of them. The readings here,
shared with the library's builder:

  * every set writes entries of one clip's known values [T, 279] and sets the
    same entries of its mask; entries it does not cover are left as they
    are, so several sets combine, and a later set wins where two overlap;
  * a set covers key frames ``frames`` with one reference pose per key frame
    (a 279-feature frame laid out as in ``kimodo_fk``: the root stream
    (x, y, z, c, s), then 30 joints x 9 features, then 4 foot contacts);
  * root path: the root's ground-plane position (x, z), features 0 and 2;
  * full body: the whole pose, the 5 root features and all 9 features of
    every joint (the 4 foot contacts stay free);
  * end effector (a hand or a foot): the 5 root features and the 6D local
    rotation (the first 6 of the joint's 9 features) of every joint on the
    chain from the root joint to the end-effector joint. Forward kinematics
    of that joint reads nothing else (``kimodo_fk.forward_kinematics``), so a
    motion carrying these entries puts the joint exactly where, and turned
    exactly as, the reference pose does, while the rest of the body stays
    free;
  * the path through n waypoints over T frames reaches waypoint i at the
    real frame position u_i = i (T - 1) / (n - 1) and is linear in between:
    frame f lies on segment s = min(floor(f (n - 1) / (T - 1)), n - 2) at
    a = f (n - 1) / (T - 1) - s, position w_s + a (w_{s+1} - w_s). One
    waypoint, or one frame, gives a constant path at the first waypoint.

Pinned by tests/test_oracle_constraint_sets.py (exact rational arithmetic for
the path, brute-force ancestor sets, and the FK invariance above).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

FEATS = 279
ROOT_FEATS = 5
N_JOINTS = 30
JOINT_FEATS = 9
ROT_FEATS = 6

ROOT_PATH, FULL_BODY, END_EFFECTOR = 0, 1, 2


def root_path(waypoints, n_frames: int) -> np.ndarray:
    """(x, z) per frame [n_frames, 2] of the piecewise-linear path through the
    waypoints [n, 2], waypoint i reached at real frame position
    i (n_frames - 1) / (n - 1)."""
    w = np.asarray(waypoints, np.float64).reshape(-1, 2)
    n = w.shape[0]
    out = np.empty((n_frames, 2))
    for f in range(n_frames):
        if n == 1 or n_frames == 1:
            out[f] = w[0]
            continue
        u = f * (n - 1) / (n_frames - 1)
        s = min(int(np.floor(u)), n - 2)
        a = u - s
        out[f] = w[s] + a * (w[s + 1] - w[s])
    return out


def chain_to_root(parents: Sequence[int], joint: int) -> list:
    """The joints from ``joint`` up to the root joint (parent -1), child first."""
    out, j = [], int(joint)
    while j >= 0:
        out.append(j)
        j = int(parents[j])
    return out


def covered_features(kind: int, joint: Optional[int] = None, parents=None) -> np.ndarray:
    """Boolean [279]: the features of one frame a set of ``kind`` covers."""
    cov = np.zeros(FEATS, dtype=bool)
    if kind == ROOT_PATH:
        cov[[0, 2]] = True
    elif kind == FULL_BODY:
        cov[:ROOT_FEATS + N_JOINTS * JOINT_FEATS] = True
    elif kind == END_EFFECTOR:
        cov[:ROOT_FEATS] = True
        for j in chain_to_root(parents, joint):
            base = ROOT_FEATS + JOINT_FEATS * j
            cov[base:base + ROT_FEATS] = True
    else:
        raise ValueError(f"unknown constraint kind {kind}")
    return cov


def apply_set(known: np.ndarray, mask: np.ndarray, kind: int, frames: Sequence[int], poses: np.ndarray,
              joint: Optional[int] = None, parents=None) -> None:
    """Writes one constraint set into a clip's known values [T, 279] and mask
    [T, 279] (in place): at key frame frames[i] the covered features take
    poses[i]'s values and their mask entries are set."""
    cov = covered_features(kind, joint, parents)
    poses = np.asarray(poses)
    for i, f in enumerate(frames):
        known[f, cov] = poses[i, cov]
        mask[f, cov] = True
