"""Device buffers for one MoE layer call (torch owns the memory; libmoe.so computes).

``MoELayer`` keeps the weight pointers, a workspace sized by
``moe_workspace_bytes`` and the per-call outputs, so a forward is one C call
with no allocation.  Only torch tensors that already live on the GPU are
accepted.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib


def _dev(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("MoELayer needs device tensors")
    return t.contiguous()


class MoELayer:
    """One layer: x [T,d] -> y [T,d] for a fixed shape.

    weights: dict with w_gate/w_up/w_down (+ s_* for int4, + sh_* for a shared
    expert) laid out [E][N][K] as moe.h describes; w_router [E,d] fp32;
    b_router [E] fp32 or None.
    """

    def __init__(self, T, d, E, k, F, act, wt, weights, w_router, b_router=None, n_shared=0,
                 tau=0, device=None):
        self.shape = _lib.make_shape(T, d, E, k, F, act, wt, n_shared, tau)
        self.device = device or weights["w_gate"].device
        self.t = {n: _dev(weights.get(n)) for n in (
            "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
            "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down")}
        self.w_router = _dev(w_router)
        self.b_router = _dev(b_router)
        self.weights = _lib.make_weights(**self.t)
        nbytes = _lib.moe_workspace_bytes(self.shape)
        if nbytes == 0:
            raise ValueError("invalid MoE shape")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        act_dt = torch.float32 if act == "f32" else torch.bfloat16
        self.y = torch.empty(T, d, dtype=act_dt, device=self.device)
        self.counts = torch.empty(E, dtype=torch.int32, device=self.device)
        self.topk_idx = torch.empty(T, k, dtype=torch.int32, device=self.device)

    def forward(self, x: torch.Tensor, residual: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        y = self.y if out is None else out
        _lib.moe_layer_forward(self.shape, x, self.w_router, self.b_router, self.weights, residual,
                               y, self.counts, self.topk_idx, self.ws, stream=stream)
        return y


def pack_int4_tiled(weights: dict, stream=None) -> dict:
    """Copy of an int4 or MXFP4 weight dict with every code tensor (w_*, sh_* of
    shape [..., N, K/2], uint8, row-major) rewritten by moe_pack_int4_tiled into
    the tiled layout; scales and other entries are passed through.  Done once
    per weight set, before the layer runs with wt="int4_tiled" or
    "mxfp4_tiled"."""
    return _pack_tiled(weights, 2, _lib.moe_pack_int4_tiled, stream)


def pack_mxfp8_tiled(weights: dict, stream=None) -> dict:
    """Copy of an MXFP8 weight dict with every code tensor (w_*, sh_* of shape
    [..., N, K], uint8, row-major) rewritten by moe_pack_mxfp8_tiled into the
    tiled layout; scales and other entries are passed through.  Done once per
    weight set, before the layer runs with wt="mxfp8_tiled"."""
    return _pack_tiled(weights, 1, _lib.moe_pack_mxfp8_tiled, stream)


def _pack_tiled(weights: dict, per_byte: int, pack, stream) -> dict:
    out = dict(weights)
    for n in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down"):
        t = weights.get(n)
        if t is None:
            continue
        t = _dev(t)
        if t.dtype != torch.uint8 or t.dim() < 2:
            raise ValueError(f"{n}: codes must be a uint8 tensor [..., N, K/{per_byte}]")
        N, K = t.shape[-2], t.shape[-1] * per_byte
        dst = torch.empty_like(t)
        pack(t, dst, t.numel() // (N * (K // per_byte)), N, K, stream=stream)
        out[n] = dst
    return out
