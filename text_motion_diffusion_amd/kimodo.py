"""ctypes binding of libkimodo.so with the entry points of include/kimodo.h.

Argument marshalling only: every stage of the denoiser runs in the library's
HIP kernels. Device tensors may be passed as torch tensors (their data_ptr()
is used) or as raw integer addresses; streams as torch streams, raw hipStream_t
integers, or None for the null stream. A non-OK status raises KimodoError.

Importing this module loads the library and fails loudly when it has not been
built (``python -m text_motion_diffusion_amd.build``). torch is imported first
so the library binds to the HIP runtime torch has loaded (one runtime per
process).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch  # noqa: F401  (loads the process's HIP runtime before the library)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkimodo.so")

KIMODO_F32, KIMODO_BF16, KIMODO_F16 = 0, 1, 2
KIMODO_CONSTRAINT_ROOT_PATH, KIMODO_CONSTRAINT_FULL_BODY, KIMODO_CONSTRAINT_END_EFFECTOR = 0, 1, 2
STATUS = {0: "OK", 1: "EINVAL", 2: "ESHAPE", 3: "EDTYPE", 4: "EWORKSPACE", 5: "EWEIGHTS", 6: "EHIP", 7: "ESTATE",
          8: "ECONFIG"}


class KimodoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class kimodo_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layers_root", "layers_body", "d_model", "n_heads", "d_ff", "root_feats", "body_feats", "text_dim",
        "max_batch", "max_frames", "max_steps", "dtype")]


class kimodo_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("ms", ctypes.c_float)]


class kimodo_trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("layers", "root_out", "local_root", "body_out", "x0_hat", "inputs")]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m text_motion_diffusion_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, D, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double, ctypes.c_float
    cfgp = ctypes.POINTER(kimodo_config)
    sig = {
        "kimodo_workspace_bytes": (SZ, [cfgp]),
        "kimodo_weight_count": (I32, [cfgp]),
        "kimodo_weight_shape": (I32, [cfgp, I32, ctypes.POINTER(I32), ctypes.POINTER(I64)]),
        "kimodo_make_schedule": (I32, [I32, D, D, I32, P, P]),
        "kimodo_make_cosine_schedule": (I32, [I32, D, D, I32, P, P]),
        "kimodo_create": (I32, [cfgp, ctypes.POINTER(P), I32, P, SZ, P, ctypes.POINTER(P)]),
        "kimodo_denoise_step": (I32, [P, I32, I32, P, P, P, I32, D, D, F, P, ctypes.POINTER(kimodo_trace), P]),
        "kimodo_denoise_step_static": (I32, [cfgp, P, I32, I32, I32, P, P, P, I32, D, D, F, P, P]),
        "kimodo_sample": (I32, [P, I32, I32, P, P, P, P, P, I32, F, P, P]),
        "kimodo_denoise_step_constrained": (I32, [P, I32, I32, P, P, P, I32, D, D, F, P, P, P,
                                                  ctypes.POINTER(kimodo_trace), P]),
        "kimodo_sample_constrained": (I32, [P, I32, I32, P, P, P, P, P, I32, F, P, P, P, P]),
        "kimodo_sample_timeline": (I32, [P, I32, I32, P, P, P, I32, P, P, I32, F, P, P]),
        "kimodo_profile_step": (I32, [P, I32, I32, P, P, P, I32, D, D, F, P, ctypes.POINTER(kimodo_kernel_time), I32,
                                      ctypes.POINTER(I32), P]),
        "kimodo_fk": (I32, [I32, P, P, P, P, P, P]),
        "kimodo_constraint_set": (I32, [I32, I32, I32, P, P, I32, P, P, P]),
        "kimodo_root_path": (I32, [I32, P, I32, P]),
        "kimodo_status_str": (ctypes.c_char_p, [I32]),
        "kimodo_last_error": (ctypes.c_char_p, [P]),
        "kimodo_graph_stats": (I32, [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
        "kimodo_destroy": (None, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("kimodo_workspace_bytes", "kimodo_weight_count", "kimodo_weight_shape", "kimodo_make_schedule",
            "kimodo_make_cosine_schedule",
            "kimodo_create", "kimodo_denoise_step", "kimodo_denoise_step_static", "kimodo_sample",
            "kimodo_denoise_step_constrained",
            "kimodo_sample_constrained", "kimodo_sample_timeline", "kimodo_fk", "kimodo_constraint_set",
            "kimodo_root_path", "kimodo_profile_step",
            "kimodo_status_str",
            "kimodo_last_error", "kimodo_graph_stats", "kimodo_destroy")


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _check(status: int, ctx=None) -> None:
    if status != 0:
        msg = _lib.kimodo_status_str(status).decode()
        if ctx is not None:
            detail = _lib.kimodo_last_error(ctx).decode()
            if detail:
                msg += f" ({detail})"
        raise KimodoError(status, msg)


def _host_i32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def make_config(layers_root=16, layers_body=16, max_batch=16, max_frames=150, max_steps=100,
                dtype=KIMODO_BF16) -> kimodo_config:
    return kimodo_config(layers_root, layers_body, 1024, 8, 2048, 5, 274, 4096, max_batch, max_frames, max_steps,
                         dtype)


def kimodo_workspace_bytes(cfg: kimodo_config) -> int:
    return int(_lib.kimodo_workspace_bytes(ctypes.byref(cfg)))


def kimodo_weight_count(cfg: kimodo_config) -> int:
    return int(_lib.kimodo_weight_count(ctypes.byref(cfg)))


def kimodo_weight_shape(cfg: kimodo_config, index: int) -> tuple:
    nd = ctypes.c_int32()
    shape = (ctypes.c_int64 * 2)()
    _check(_lib.kimodo_weight_shape(ctypes.byref(cfg), index, ctypes.byref(nd), shape))
    return tuple(int(shape[i]) for i in range(nd.value))


def kimodo_make_schedule(n_train: int, beta_start: float, beta_end: float, S: int):
    ts = np.zeros(S, np.int32)
    ab = np.zeros(S, np.float64)
    _check(_lib.kimodo_make_schedule(n_train, beta_start, beta_end, S, ts.ctypes.data, ab.ctypes.data))
    return ts, ab


def kimodo_make_cosine_schedule(n_train: int, s: float, max_beta: float, S: int):
    ts = np.zeros(S, np.int32)
    ab = np.zeros(S, np.float64)
    _check(_lib.kimodo_make_cosine_schedule(n_train, s, max_beta, S, ts.ctypes.data, ab.ctypes.data))
    return ts, ab


def kimodo_create(cfg: kimodo_config, weights: Sequence, workspace, workspace_bytes: int, stream=None) -> int:
    arr = (ctypes.c_void_p * len(weights))(*[_ptr(w) for w in weights])
    out = ctypes.c_void_p()
    _check(_lib.kimodo_create(ctypes.byref(cfg), arr, len(weights), _ptr(workspace), workspace_bytes,
                              _stream(stream), ctypes.byref(out)))
    return out.value


def _trace(trace: Optional[dict]):
    if not trace:
        return None
    return kimodo_trace(*[_ptr(trace.get(k)) for k in ("layers", "root_out", "local_root", "body_out", "x0_hat",
                                                          "inputs")])


def _schedule(timesteps, abar):
    ts = _host_i32(timesteps)
    ab = np.ascontiguousarray(np.asarray(abar), dtype=np.float64)
    if ts.shape != ab.shape:
        raise ValueError("timesteps and abar differ in length")
    return ts, ab


def kimodo_denoise_step(ctx: int, B: int, T: int, x_t, text_emb, lengths, t: int, abar_t: float, abar_prev: float,
                        cfg_scale: float, x_prev, trace: Optional[dict] = None, stream=None) -> None:
    lens = _host_i32(lengths)
    tr = _trace(trace)
    _check(_lib.kimodo_denoise_step(ctx, B, T, _ptr(x_t), _ptr(text_emb), None if lens is None else lens.ctypes.data,
                                    t, abar_t, abar_prev, cfg_scale, _ptr(x_prev),
                                    None if tr is None else ctypes.byref(tr), _stream(stream)), ctx)


def kimodo_denoise_step_static(cfg: kimodo_config, weights: Sequence, B: int, T: int, x_t, text_emb, lengths, t: int,
                               abar_t: float, abar_prev: float, cfg_scale: float, x_prev, stream=None) -> None:
    """kimodo_denoise_step without a ctx or workspace (the library's static scratch)."""
    lens = _host_i32(lengths)
    arr = (ctypes.c_void_p * len(weights))(*[_ptr(w) for w in weights])
    _check(_lib.kimodo_denoise_step_static(ctypes.byref(cfg), arr, len(weights), B, T, _ptr(x_t), _ptr(text_emb),
                                           None if lens is None else lens.ctypes.data, t, abar_t, abar_prev,
                                           cfg_scale, _ptr(x_prev), _stream(stream)))


def kimodo_denoise_step_constrained(ctx: int, B: int, T: int, x_t, text_emb, lengths, t: int, abar_t: float,
                                    abar_prev: float, cfg_scale: float, known_values, known_mask, x_prev,
                                    trace: Optional[dict] = None, stream=None) -> None:
    lens = _host_i32(lengths)
    tr = _trace(trace)
    _check(_lib.kimodo_denoise_step_constrained(
        ctx, B, T, _ptr(x_t), _ptr(text_emb), None if lens is None else lens.ctypes.data, t, abar_t, abar_prev,
        cfg_scale, _ptr(known_values), _ptr(known_mask), _ptr(x_prev), None if tr is None else ctypes.byref(tr),
        _stream(stream)), ctx)


def kimodo_sample(ctx: int, B: int, T: int, noise, text_emb, lengths, timesteps, abar, cfg_scale: float, out,
                  stream=None) -> None:
    lens = _host_i32(lengths)
    ts, ab = _schedule(timesteps, abar)
    _check(_lib.kimodo_sample(ctx, B, T, _ptr(noise), _ptr(text_emb), None if lens is None else lens.ctypes.data,
                              ts.ctypes.data, ab.ctypes.data, len(ts), cfg_scale, _ptr(out), _stream(stream)), ctx)


def kimodo_sample_constrained(ctx: int, B: int, T: int, noise, text_emb, lengths, timesteps, abar,
                              cfg_scale: float, known_values, known_mask, out, stream=None) -> None:
    lens = _host_i32(lengths)
    ts, ab = _schedule(timesteps, abar)
    _check(_lib.kimodo_sample_constrained(
        ctx, B, T, _ptr(noise), _ptr(text_emb), None if lens is None else lens.ctypes.data, ts.ctypes.data,
        ab.ctypes.data, len(ts), cfg_scale, _ptr(known_values), _ptr(known_mask), _ptr(out), _stream(stream)), ctx)


def kimodo_sample_timeline(ctx: int, V: int, seg_frames, seg_text, noise, n_transition: int, timesteps, abar,
                           cfg_scale: float, out, stream=None) -> None:
    frames = _host_i32(seg_frames)
    ts, ab = _schedule(timesteps, abar)
    _check(_lib.kimodo_sample_timeline(ctx, V, len(frames), frames.ctypes.data, _ptr(seg_text), _ptr(noise),
                                       n_transition, ts.ctypes.data, ab.ctypes.data, len(ts), cfg_scale, _ptr(out),
                                       _stream(stream)), ctx)


def kimodo_profile_step(ctx: int, B: int, T: int, x_t, text_emb, lengths, t: int, abar_t: float, abar_prev: float,
                        cfg_scale: float, x_prev, max_records: int = 1024, stream=None) -> list:
    """Returns [(kernel name, ms), ...] in launch order."""
    lens = _host_i32(lengths)
    recs = (kimodo_kernel_time * max_records)()
    n = ctypes.c_int32()
    _check(_lib.kimodo_profile_step(ctx, B, T, _ptr(x_t), _ptr(text_emb), None if lens is None else lens.ctypes.data,
                                    t, abar_t, abar_prev, cfg_scale, _ptr(x_prev), recs, max_records,
                                    ctypes.byref(n), _stream(stream)), ctx)
    return [(recs[i].name.decode(), float(recs[i].ms)) for i in range(min(n.value, max_records))]


def kimodo_fk(n_frames: int, motion, parents, offsets, positions, rotations=None, stream=None) -> None:
    """parents: int32 [30] and offsets: fp32 [30, 3] host arrays; motion,
    positions, rotations: device tensors or addresses."""
    par = _host_i32(parents)
    off = np.ascontiguousarray(np.asarray(offsets), dtype=np.float32)
    if par.shape != (30,) or off.shape != (30, 3):
        raise ValueError("parents must be [30] and offsets [30, 3]")
    _check(_lib.kimodo_fk(n_frames, _ptr(motion), par.ctypes.data, off.ctypes.data, _ptr(positions),
                          _ptr(rotations), _stream(stream)))


def kimodo_constraint_set(kind: int, frames, poses, known_values: np.ndarray, known_mask: np.ndarray, joint: int = -1,
                          parents=None) -> None:
    """One constraint set into one clip's host arrays known_values fp32 [T,
    279] and known_mask u8 [T, 279] (C-contiguous, updated in place); frames
    int [n_keys], poses fp32 [n_keys, 279]."""
    fr = _host_i32(frames).reshape(-1)
    po = np.ascontiguousarray(np.asarray(poses), dtype=np.float32).reshape(-1, 279)
    if po.shape[0] != fr.shape[0]:
        raise ValueError("one pose per key frame")
    if known_values.dtype != np.float32 or known_mask.dtype != np.uint8 or known_values.ndim != 2 \
            or known_values.shape != known_mask.shape or known_values.shape[1] != 279 \
            or not known_values.flags.c_contiguous or not known_mask.flags.c_contiguous:
        raise ValueError("known_values fp32 and known_mask u8, both C-contiguous [T, 279]")
    par = _host_i32(parents)
    _check(_lib.kimodo_constraint_set(kind, known_values.shape[0], fr.shape[0], fr.ctypes.data, po.ctypes.data, joint,
                                      None if par is None else par.ctypes.data, known_values.ctypes.data,
                                      known_mask.ctypes.data))


def kimodo_root_path(waypoints, n_frames: int) -> np.ndarray:
    """waypoints [n, 2] (x, z) -> fp32 [n_frames, 2]."""
    w = np.ascontiguousarray(np.asarray(waypoints), dtype=np.float32).reshape(-1, 2)
    out = np.empty((n_frames, 2), np.float32)
    _check(_lib.kimodo_root_path(w.shape[0], w.ctypes.data, n_frames, out.ctypes.data))
    return out


def kimodo_status_str(status: int) -> str:
    return _lib.kimodo_status_str(status).decode()


def kimodo_last_error(ctx: int) -> str:
    return _lib.kimodo_last_error(ctx).decode()


def kimodo_graph_stats(ctx: int) -> tuple:
    """(step graphs instantiated, step graphs updated in place) over the ctx's life."""
    inst, upd = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib.kimodo_graph_stats(ctx, ctypes.byref(inst), ctypes.byref(upd)))
    return inst.value, upd.value


def kimodo_destroy(ctx: int) -> None:
    _lib.kimodo_destroy(ctx)
