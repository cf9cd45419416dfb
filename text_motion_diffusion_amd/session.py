"""Device-memory plumbing around the C ABI: torch allocates the weight table,
the workspace and the output tensors; every computation happens in
libkimodo.so through the binding in ``kimodo.py``."""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import kimodo as K


def _check_known(known, known_mask, shape) -> None:
    if (known is None) != (known_mask is None):
        raise ValueError("known and known_mask go together")
    if known is None:
        return
    if tuple(known.shape) != tuple(shape) or known.dtype != torch.float32 or not known.is_contiguous():
        raise ValueError("known must be contiguous fp32 of the state's shape")
    if tuple(known_mask.shape) != tuple(shape) or known_mask.dtype != torch.uint8 or not known_mask.is_contiguous():
        raise ValueError("known_mask must be contiguous uint8 of the state's shape")


class Session:
    """Weights resident on one GPU plus a ctx and its workspace.

    weights in canonical order (kimodo_weight_shape): fp32 arrays for
    KIMODO_F32, bf16 bit patterns (uint16) for KIMODO_BF16, float16 arrays for
    KIMODO_F16.
    """

    def __init__(self, weights: Sequence[np.ndarray], layers_root: int, layers_body: int, max_batch: int,
                 max_frames: int, max_steps: int = 100, dtype: int = K.KIMODO_BF16, device: str = "cuda:0"):
        self.device = torch.device(device)
        self.cfg = K.make_config(layers_root, layers_body, max_batch, max_frames, max_steps, dtype)
        n = K.kimodo_weight_count(self.cfg)
        if n != len(weights):
            raise ValueError(f"expected {n} weight tensors, got {len(weights)}")
        self.weights = []
        for i, w in enumerate(weights):
            shape = K.kimodo_weight_shape(self.cfg, i)
            a = np.ascontiguousarray(w)
            if tuple(a.shape) != shape:
                raise ValueError(f"weight {i}: shape {a.shape} != {shape}")
            if dtype == K.KIMODO_BF16:
                if a.dtype != np.uint16:
                    raise TypeError("bf16 sessions take bf16 bit patterns (uint16)")
                t = torch.from_numpy(a.view(np.int16)).to(self.device).view(torch.bfloat16)
            elif dtype == K.KIMODO_F16:
                t = torch.from_numpy(a.astype(np.float16, copy=False)).to(self.device)
            else:
                t = torch.from_numpy(a.astype(np.float32, copy=False)).to(self.device)
            self.weights.append(t)
        self.ws_bytes = K.kimodo_workspace_bytes(self.cfg)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.ctx = K.kimodo_create(self.cfg, self.weights, self.workspace, self.ws_bytes,
                                   torch.cuda.current_stream(self.device))

    @property
    def act_dtype(self):
        return torch.float32 if self.cfg.dtype == K.KIMODO_F32 else torch.float16

    def denoise_step(self, x_t: torch.Tensor, text: torch.Tensor, lengths, t: int, abar_t: float, abar_prev: float,
                     cfg_scale: float, x_prev: Optional[torch.Tensor] = None, trace: bool = False,
                     known: Optional[torch.Tensor] = None, known_mask: Optional[torch.Tensor] = None):
        """One DDIM step; known / known_mask (fp32 and uint8 [B, T, 279]) fix
        entries of the clean motion (kimodo_denoise_step_constrained)."""
        B, T, _ = x_t.shape
        if x_prev is None:
            x_prev = torch.empty_like(x_t)
        tr = None
        if trace:
            L = self.cfg.layers_root + self.cfg.layers_body
            tr = {
                "layers": torch.empty((L, 2 * B, T + 2, 1024), dtype=self.act_dtype, device=self.device),
                "inputs": torch.empty((2, 2 * B, T + 2, 1024), dtype=self.act_dtype, device=self.device),
                "root_out": torch.empty((2 * B, T, 5), device=self.device),
                "local_root": torch.empty((2 * B, T, 5), device=self.device),
                "body_out": torch.empty((2 * B, T, 274), device=self.device),
                "x0_hat": torch.empty((B, T, 279), device=self.device),
            }
        _check_known(known, known_mask, x_t.shape)
        K.kimodo_denoise_step_constrained(self.ctx, B, T, x_t, text, lengths, t, abar_t, abar_prev, cfg_scale, known,
                                          known_mask, x_prev, tr, torch.cuda.current_stream(self.device))
        return (x_prev, tr) if trace else x_prev

    def sample(self, noise: torch.Tensor, text: torch.Tensor, lengths, timesteps, abar, cfg_scale: float,
               out: Optional[torch.Tensor] = None, known: Optional[torch.Tensor] = None,
               known_mask: Optional[torch.Tensor] = None) -> torch.Tensor:
        B, T, _ = noise.shape
        if out is None:
            out = torch.empty_like(noise)
        _check_known(known, known_mask, noise.shape)
        K.kimodo_sample_constrained(self.ctx, B, T, noise, text, lengths, timesteps, abar, cfg_scale, known,
                                    known_mask, out, torch.cuda.current_stream(self.device))
        return out

    def sample_timeline(self, seg_frames: Sequence[int], seg_text: torch.Tensor, noise: Sequence[torch.Tensor],
                        n_transition: int, timesteps, abar, cfg_scale: float) -> torch.Tensor:
        """seg_text [n_seg, V, 4096]; noise[k] [V, T_k, 279]. Returns the
        timeline [V, T_0 + sum_{k>0} (T_k - n_transition), 279]."""
        V = seg_text.shape[1]
        frames = [int(f) for f in seg_frames]
        if seg_text.shape != (len(frames), V, 4096) or seg_text.dtype != torch.float32:
            raise ValueError("seg_text must be fp32 [n_seg, V, 4096]")
        for k, (n, Tk) in enumerate(zip(noise, frames)):
            if tuple(n.shape) != (V, Tk, 279):
                raise ValueError(f"noise[{k}] must be [V, {Tk}, 279]")
        flat = torch.cat([n.reshape(-1) for n in noise]).to(self.device, torch.float32).contiguous()
        total = frames[0] + sum(f - n_transition for f in frames[1:])
        out = torch.empty((V, total, 279), dtype=torch.float32, device=self.device)
        K.kimodo_sample_timeline(self.ctx, V, frames, seg_text.contiguous(), flat, n_transition, timesteps, abar,
                                 cfg_scale, out, torch.cuda.current_stream(self.device))
        return out

    def graph_stats(self) -> tuple:
        """(step graphs instantiated, step graphs updated in place) so far."""
        return K.kimodo_graph_stats(self.ctx)

    def close(self):
        if getattr(self, "ctx", None):
            K.kimodo_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
