"""CPU tests of the C ABI: the library loads, exports every entry point of
include/kimodo.h, reports the canonical weight table, builds the schedule, and
rejects every invalid argument on the host before touching a device."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from oracle import kimodo_oracle as O
from synthetic.inputs import Dims, weight_specs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "text_motion_diffusion_amd", "libkimodo.so")
if not os.path.exists(LIB):  # build only when nothing is built
    from text_motion_diffusion_amd.build import build

    build()

from text_motion_diffusion_amd import kimodo as K  # noqa: E402

FAKE = 1 << 20  # a 256-byte aligned address that is never dereferenced


def header_functions():
    with open(os.path.join(ROOT, "include", "kimodo.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(kimodo_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) == 20
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(K.EXPORTED)


def _header_struct_fields(name):
    """Field names of `typedef struct { ... } name;` in include/kimodo.h, in order."""
    with open(os.path.join(ROOT, "include", "kimodo.h")) as f:
        text = f.read()
    body = re.search(r"typedef struct \{([^}]*)\}\s*" + name + r"\s*;", text).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    out = []
    for decl in body.split(";"):
        decl = " ".join(decl.split())
        if decl:  # "int32_t a, b" / "float *x" / "char name[32]"
            out += [re.sub(r"\[.*\]", "", v).replace("*", "").strip() for v in decl.partition(" ")[2].split(",")]
    return out


@pytest.mark.parametrize("name,cls", [("kimodo_trace", K.kimodo_trace), ("kimodo_config", K.kimodo_config),
                                      ("kimodo_kernel_time", K.kimodo_kernel_time)])
def test_binding_structs_match_the_header(name, cls):
    """The ctypes structs declare the header's fields in the header's order."""
    assert [f for f, _ in cls._fields_] == _header_struct_fields(name)


@pytest.mark.parametrize("L", [16, 2, 0])
def test_weight_table_matches_canonical_order(L):
    cfg = K.make_config(L, L, 4, 32, 8, K.KIMODO_BF16)
    specs = weight_specs(Dims(layers_root=L, layers_body=L))
    assert K.kimodo_weight_count(cfg) == len(specs)
    for i, (name, shape, _) in enumerate(specs):
        assert K.kimodo_weight_shape(cfg, i) == tuple(shape), name


def test_config_validation():
    good = K.make_config(2, 2, 4, 32, 8, K.KIMODO_F32)
    assert K.kimodo_workspace_bytes(good) > 0
    for field, bad in (("d_model", 512), ("n_heads", 16), ("d_ff", 4096), ("root_feats", 6), ("body_feats", 270),
                       ("text_dim", 1024), ("max_batch", 0), ("max_frames", 0), ("max_steps", 0),
                       ("layers_root", -1), ("dtype", 7), ("max_batch", 513), ("max_frames", 5000)):
        cfg = K.make_config(2, 2, 4, 32, 8, K.KIMODO_F32)
        setattr(cfg, field, bad)
        assert K.kimodo_workspace_bytes(cfg) == 0, field
        assert K.kimodo_weight_count(cfg) == -1, field


def test_workspace_grows_with_capacity_and_dtype():
    ws = lambda B, dt: K.kimodo_workspace_bytes(K.make_config(16, 16, B, 150, 100, dt))
    assert 0 < ws(1, K.KIMODO_F16) < ws(16, K.KIMODO_F16) < ws(16, K.KIMODO_F32)
    # the activations alone: 2B(T+2) rows x (4 x 1024 + 3072 + 2048) x 2 bytes
    assert ws(16, K.KIMODO_F16) >= 2 * 16 * 152 * (4 * 1024 + 3072 + 2048) * 2
    # bf16 weights: the workspace also holds their fp16 matrix copy
    cfg = K.make_config(16, 16, 16, 150, 100, K.KIMODO_BF16)
    mats = sum(int(np.prod(s)) for s in (K.kimodo_weight_shape(cfg, i) for i in range(K.kimodo_weight_count(cfg)))
               if len(s) == 2)
    assert ws(16, K.KIMODO_BF16) - ws(16, K.KIMODO_F16) >= 2 * mats


@pytest.mark.parametrize("S", [1, 15, 35, 50, 100])
def test_schedule_matches_oracle(S):
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    _, abar = O.linear_beta_schedule()
    np.testing.assert_array_equal(ts, O.ddim_timesteps(S))
    np.testing.assert_allclose(ab, abar[ts], rtol=1e-15, atol=0)


@pytest.mark.parametrize("S", [15, 20, 35, 50, 100])
def test_cosine_schedule_matches_oracle(S):
    ts, ab = K.kimodo_make_cosine_schedule(100, 0.008, 0.999, S)
    _, abar = O.cosine_beta_schedule()
    np.testing.assert_array_equal(ts, O.ddim_timesteps(S))
    np.testing.assert_allclose(ab, abar[ts], rtol=1e-13, atol=0)


def test_cosine_schedule_rejects_bad_arguments():
    for args in ((1, 0.008, 0.999, 1), (100, 0.008, 0.999, 0), (100, 0.008, 0.999, 101), (100, -0.1, 0.999, 10),
                 (100, 0.008, 0.0, 10), (100, 0.008, 1.0, 10)):
        with pytest.raises(K.KimodoError):
            K.kimodo_make_cosine_schedule(*args)


def test_schedule_rejects_bad_arguments():
    for args in ((1, 1e-4, 0.02, 1), (100, 1e-4, 0.02, 0), (100, 1e-4, 0.02, 101), (100, 0.0, 0.02, 10),
                 (100, 0.03, 0.02, 10), (100, 1e-4, 1.0, 10)):
        with pytest.raises(K.KimodoError):
            K.kimodo_make_schedule(*args)


def _fake_weights(cfg):
    return [FAKE + 256 * i for i in range(K.kimodo_weight_count(cfg))]


def test_create_rejects_bad_arguments():
    cfg = K.make_config(2, 2, 2, 16, 4, K.KIMODO_BF16)
    ws = K.kimodo_workspace_bytes(cfg)
    w = _fake_weights(cfg)
    cases = [
        (dict(weights=w[:-1]), "EWEIGHTS"),
        (dict(weights=w[:3] + [0] + w[4:]), "EWEIGHTS"),
        (dict(weights=w[:3] + [FAKE + 8] + w[4:]), "EWEIGHTS"),
        (dict(workspace=0), "EWORKSPACE"),
        (dict(workspace=FAKE + 64), "EWORKSPACE"),
        (dict(workspace=FAKE + 128), "EWORKSPACE"),
        (dict(nbytes=ws - 1), "EWORKSPACE"),
    ]
    for over, code in cases:
        a = dict(weights=w, workspace=FAKE, nbytes=ws)
        a.update(over)
        with pytest.raises(K.KimodoError, match=code):
            K.kimodo_create(cfg, a["weights"], a["workspace"], a["nbytes"])
    bad = K.make_config(2, 2, 2, 16, 4, K.KIMODO_BF16)
    bad.d_model = 768
    with pytest.raises(K.KimodoError, match="ECONFIG"):
        K.kimodo_create(bad, w, FAKE, ws)
    bad = K.make_config(2, 2, 2, 16, 4, 5)
    with pytest.raises(K.KimodoError, match="EDTYPE"):
        K.kimodo_create(bad, w, FAKE, ws)


def test_calls_reject_bad_arguments_before_any_device_work():
    cfg = K.make_config(2, 2, 2, 16, 4, K.KIMODO_BF16)
    ctx = K.kimodo_create(cfg, _fake_weights(cfg), FAKE, K.kimodo_workspace_bytes(cfg))
    try:
        step = dict(B=2, T=16, x_t=FAKE, text=FAKE, lengths=None, t=50, abar_t=0.7, abar_prev=0.8, w=2.5, x_prev=FAKE)
        bad_steps = [
            (dict(B=0), "ESHAPE"), (dict(B=3), "ESHAPE"), (dict(T=0), "ESHAPE"), (dict(T=17), "ESHAPE"),
            (dict(lengths=[16, 0]), "ESHAPE"), (dict(lengths=[17, 3]), "ESHAPE"), (dict(t=-1), "ESHAPE"),
            (dict(abar_t=1.0), "EINVAL"), (dict(abar_t=0.0), "EINVAL"), (dict(abar_prev=1.5), "EINVAL"),
            (dict(w=math.nan), "EINVAL"), (dict(w=math.inf), "EINVAL"), (dict(x_t=0), "EINVAL"),
            (dict(text=0), "EINVAL"), (dict(x_prev=0), "EINVAL"),
        ]
        for over, code in bad_steps:
            a = dict(step)
            a.update(over)
            with pytest.raises(K.KimodoError, match=code):
                K.kimodo_denoise_step(ctx, a["B"], a["T"], a["x_t"], a["text"], a["lengths"], a["t"], a["abar_t"],
                                      a["abar_prev"], a["w"], a["x_prev"])
            assert K.kimodo_last_error(ctx)
        ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, 4)
        samp = dict(B=2, T=16, ts=ts, ab=ab)
        bad_samples = [
            (dict(ts=ts[::-1].copy()), "ESHAPE"), (dict(ts=np.array([0, 5, 5, 9])), "ESHAPE"),
            (dict(ts=np.arange(5), ab=np.full(5, 0.5)), "ESHAPE"),
            (dict(ab=np.array([0.9, 0.8, 1.0, 0.5])), "EINVAL"), (dict(ab=np.array([0.9, 0.8, 0.0, 0.5])), "EINVAL"),
            (dict(B=5), "ESHAPE"),
        ]
        for over, code in bad_samples:
            a = dict(samp)
            a.update(over)
            with pytest.raises(K.KimodoError, match=code):
                K.kimodo_sample(ctx, a["B"], a["T"], FAKE, FAKE, None, a["ts"], a["ab"], 2.5, FAKE)
    finally:
        K.kimodo_destroy(ctx)
    K.kimodo_destroy(0)  # NULL is a no-op


def test_constrained_and_timeline_calls_reject_bad_arguments():
    cfg = K.make_config(2, 2, 2, 16, 4, K.KIMODO_BF16)
    ctx = K.kimodo_create(cfg, _fake_weights(cfg), FAKE, K.kimodo_workspace_bytes(cfg))
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, 4)
    try:
        for known, mask in ((FAKE, None), (None, FAKE), (FAKE + 2, FAKE)):
            with pytest.raises(K.KimodoError, match="EINVAL"):
                K.kimodo_denoise_step_constrained(ctx, 2, 16, FAKE, FAKE, None, 50, 0.7, 0.8, 2.5, known, mask, FAKE)
            with pytest.raises(K.KimodoError, match="EINVAL"):
                K.kimodo_sample_constrained(ctx, 2, 16, FAKE, FAKE, None, ts, ab, 2.5, known, mask, FAKE)
        with pytest.raises(K.KimodoError, match="ESHAPE"):  # the step's own checks still apply
            K.kimodo_sample_constrained(ctx, 3, 16, FAKE, FAKE, None, ts, ab, 2.5, FAKE, FAKE, FAKE)
        tl = dict(V=2, frames=[8, 6, 5], n_tr=2, out=FAKE, ts=ts, ab=ab, w=2.5)
        bad = [
            (dict(V=0), "ESHAPE"), (dict(V=3), "ESHAPE"), (dict(frames=[]), "ESHAPE"),
            (dict(frames=[8, 17]), "ESHAPE"), (dict(frames=[8, 0]), "ESHAPE"),
            (dict(frames=[8, 2]), "ESHAPE"),        # n_tr must be < T_k
            (dict(frames=[1, 8]), "ESHAPE"),        # and <= T_{k-1}
            (dict(n_tr=-1), "ESHAPE"), (dict(out=0), "EINVAL"), (dict(w=math.nan), "EINVAL"),
            (dict(ts=ts[::-1].copy()), "ESHAPE"), (dict(ab=np.array([0.9, 0.8, 1.0, 0.5])), "EINVAL"),
        ]
        for over, code in bad:
            a = dict(tl)
            a.update(over)
            with pytest.raises(K.KimodoError, match=code):
                K.kimodo_sample_timeline(ctx, a["V"], a["frames"], FAKE, FAKE, a["n_tr"], a["ts"], a["ab"], a["w"],
                                         a["out"])
            assert K.kimodo_last_error(ctx)
    finally:
        K.kimodo_destroy(ctx)


def test_fk_rejects_bad_arguments_before_any_device_work():
    from synthetic.inputs import make_skeleton

    _, parents, offsets = make_skeleton()
    good = dict(n=10, motion=FAKE, parents=parents, offsets=offsets, pos=FAKE, rot=None)
    bad_parents = parents.copy()
    bad_parents[5] = 7          # a parent after its child
    root_parent = parents.copy()
    root_parent[0] = 0
    bad_offsets = offsets.copy()
    bad_offsets[3, 1] = np.nan
    cases = [
        (dict(n=-1), "ESHAPE"), (dict(n=1 << 27), "ESHAPE"), (dict(motion=0), "EINVAL"), (dict(pos=0), "EINVAL"),
        (dict(motion=FAKE + 2), "EINVAL"), (dict(rot=FAKE + 1), "EINVAL"), (dict(parents=bad_parents), "EINVAL"),
        (dict(parents=root_parent), "EINVAL"), (dict(offsets=bad_offsets), "EINVAL"),
    ]
    for over, code in cases:
        a = dict(good)
        a.update(over)
        with pytest.raises(K.KimodoError, match=code):
            K.kimodo_fk(a["n"], a["motion"], a["parents"], a["offsets"], a["pos"], a["rot"])
    K.kimodo_fk(0, FAKE, parents, offsets, FAKE)  # no frames: nothing is launched
    with pytest.raises(ValueError):
        K.kimodo_fk(1, FAKE, parents[:29], offsets[:29], FAKE)


def test_static_step_rejects_bad_arguments_before_any_device_work():
    """kimodo_denoise_step_static checks everything on the host first: dtype,
    shapes, the weight table, scratch capacity and the step arguments."""
    cfg16 = K.make_config(2, 2, 1, 1, 1, K.KIMODO_F16)
    cfg32 = K.make_config(2, 2, 1, 1, 1, K.KIMODO_F32)
    w = _fake_weights(cfg16)
    bad = K.make_config(2, 2, 1, 1, 1, K.KIMODO_F16)
    bad.d_model = 512
    cases = [
        (dict(cfg=K.make_config(2, 2, 1, 1, 1, K.KIMODO_BF16)), "EDTYPE"),
        (dict(B=0), "ESHAPE"), (dict(T=5000), "ESHAPE"), (dict(cfg=bad), "ECONFIG"),
        (dict(weights=w[:-1]), "EWEIGHTS"), (dict(weights=w[:3] + [FAKE + 8] + w[4:]), "EWEIGHTS"),
        (dict(B=8, T=150), "EWORKSPACE"),  # 2,432 token rows: past the static scratch
        (dict(cfg=cfg32, B=6, T=150), "EWORKSPACE"),
        (dict(x=None), "EINVAL"), (dict(lengths=[11]), "ESHAPE"), (dict(ab_t=1.0), "EINVAL"),
        (dict(cs=float("nan")), "EINVAL"),
    ]
    for over, code in cases:
        a = dict(cfg=cfg16, weights=w, B=1, T=10, x=FAKE, lengths=None, ab_t=0.5, cs=2.5)
        a.update(over)
        with pytest.raises(K.KimodoError, match=code):
            K.kimodo_denoise_step_static(a["cfg"], a["weights"], a["B"], a["T"], a["x"], FAKE, a["lengths"], 5,
                                         a["ab_t"], 0.6, a["cs"], FAKE)


def test_status_strings():
    for s in range(9):
        assert K.kimodo_status_str(s)
    assert K.kimodo_status_str(99) == "unknown status"


# ---- constraint sets (host functions of the library) against the oracle ----

def _skeleton():
    from synthetic.inputs import make_skeleton

    return make_skeleton()[1]


@pytest.mark.parametrize("kind,joint", [(K.KIMODO_CONSTRAINT_ROOT_PATH, -1), (K.KIMODO_CONSTRAINT_FULL_BODY, -1),
                                        (K.KIMODO_CONSTRAINT_END_EFFECTOR, 10), (K.KIMODO_CONSTRAINT_END_EFFECTOR, 24),
                                        (K.KIMODO_CONSTRAINT_END_EFFECTOR, 0)])
def test_constraint_set_matches_oracle(kind, joint):
    from oracle import kimodo_constraint_sets as C

    parents = _skeleton()
    rng = np.random.default_rng(kind * 31 + joint + 1)
    T, frames = 40, [0, 7, 39, 7]  # a repeated key frame: the later pose wins
    poses = rng.standard_normal((len(frames), 279)).astype(np.float32)
    known = rng.standard_normal((T, 279)).astype(np.float32)  # a set leaves other entries as they are
    mask = (rng.random((T, 279)) < 0.1).astype(np.uint8)
    want_k, want_m = known.astype(np.float64), mask.astype(bool)
    C.apply_set(want_k, want_m, kind, frames, poses.astype(np.float64), joint if joint >= 0 else None, parents)
    K.kimodo_constraint_set(kind, frames, poses, known, mask, joint, parents)
    np.testing.assert_array_equal(mask.astype(bool), want_m)
    np.testing.assert_array_equal(known, want_k.astype(np.float32))


def test_constraint_set_refuses_bad_arguments_and_writes_nothing():
    parents = _skeleton()
    known = np.zeros((10, 279), np.float32)
    mask = np.zeros((10, 279), np.uint8)
    pose = np.ones((1, 279), np.float32)
    for kind, frames, joint, par in ((3, [0], -1, None), (K.KIMODO_CONSTRAINT_FULL_BODY, [10], -1, None),
                                     (K.KIMODO_CONSTRAINT_ROOT_PATH, [-1], -1, None),
                                     (K.KIMODO_CONSTRAINT_END_EFFECTOR, [0], 30, parents),
                                     (K.KIMODO_CONSTRAINT_END_EFFECTOR, [0], 5, None),
                                     (K.KIMODO_CONSTRAINT_END_EFFECTOR, [0], 5, parents[::-1].copy())):
        with pytest.raises(K.KimodoError):
            K.kimodo_constraint_set(kind, frames, pose, known, mask, joint, par)
    assert not known.any() and not mask.any()


@pytest.mark.parametrize("m,n", [(5, 180), (5, 181), (2, 2), (3, 7), (1, 9), (4, 1)])
def test_root_path_matches_oracle(m, n):
    from oracle import kimodo_constraint_sets as C

    w = np.random.default_rng(m * 100 + n).uniform(-4, 4, size=(m, 2)).astype(np.float32)
    got = K.kimodo_root_path(w, n)
    want = C.root_path(w.astype(np.float64), n)
    # both evaluate w_s + a (w_{s+1} - w_s) in double; the library then rounds to fp32
    np.testing.assert_allclose(got, want, rtol=0, atol=np.spacing(np.float32(4.0)))
    with pytest.raises(K.KimodoError):
        K.kimodo_root_path(np.array([[0.0, np.nan]]), 3)
