"""ctypes binding of libmoe.so (declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are passed as device pointers (``tensor.data_ptr()``) and the
stream as torch's current HIP stream.  If the shared library is missing the
import of this module raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EHIP, MOE_EUNSUPPORTED = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_INT4_G128, MOE_INT4_G128_TILED = 0, 1, 2, 3
MOE_INT4_G64, MOE_MXFP4, MOE_MXFP8, MOE_MXFP4_TILED, MOE_MXFP8_TILED = 4, 5, 6, 7, 8
DTYPE_CODES = {"f32": MOE_F32, "bf16": MOE_BF16, "int4": MOE_INT4_G128, "int4_tiled": MOE_INT4_G128_TILED,
               "int4g64": MOE_INT4_G64, "mxfp4": MOE_MXFP4, "mxfp8": MOE_MXFP8,
               "mxfp4_tiled": MOE_MXFP4_TILED, "mxfp8_tiled": MOE_MXFP8_TILED}

EXPORTS = ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
           "moe_layer_forward_noalloc", "moe_workspace_bytes", "moe_rmsnorm", "moe_pack_int4_tiled",
           "moe_pack_mxfp8_tiled", "moe_topk_overlap", "moe_strerror")


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("F", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("act", ctypes.c_int32), ("wt", ctypes.c_int32), ("tau", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
        "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down")]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (run python -m moe_layer_forward_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p, sz, cp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_char_p
        sp = ctypes.POINTER(Shape)
        wp = ctypes.POINTER(Weights)
        L.moe_route.argtypes = [sp, vp, vp, vp, vp, i32p, vp, vp, cp, sz]
        L.moe_dispatch.argtypes = [sp, i32p, i32p, i32p, i32p, i32p, vp, cp, sz]
        L.moe_expert_ffn.argtypes = [sp, vp, wp, i32p, i32p, i32p, vp, vp, vp, sz, vp, cp, sz]
        L.moe_combine.argtypes = [sp, vp, i32p, vp, vp, vp, vp, vp, cp, sz]
        L.moe_layer_forward.argtypes = [sp, vp, vp, vp, wp, vp, vp, i32p, i32p, vp, sz, vp, cp, sz]
        L.moe_layer_forward_noalloc.argtypes = [sp, vp, vp, vp, wp, vp, vp, i32p, i32p, vp, cp, sz]
        L.moe_workspace_bytes.argtypes = [sp]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_rmsnorm.argtypes = [sp, vp, vp, ctypes.c_float, vp, vp, cp, sz]
        L.moe_pack_int4_tiled.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, cp, sz]
        L.moe_pack_mxfp8_tiled.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, cp, sz]
        L.moe_topk_overlap.argtypes = [sp, i32p, i32p, i32p, vp, cp, sz]
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
                  "moe_layer_forward", "moe_layer_forward_noalloc", "moe_rmsnorm", "moe_pack_int4_tiled",
                  "moe_pack_mxfp8_tiled", "moe_topk_overlap"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _call(name, *args):
    buf = ctypes.create_string_buffer(512)
    rc = getattr(lib(), name)(*args, buf, len(buf))
    if rc != MOE_OK:
        raise MoEError(name, rc, buf.value.decode(errors="replace"))
    return rc


def make_shape(T, d, E, k, F, act="bf16", wt="bf16", n_shared=0, tau=0) -> Shape:
    return Shape(T, d, E, k, F, n_shared, DTYPE_CODES[act] if isinstance(act, str) else act,
                 DTYPE_CODES[wt] if isinstance(wt, str) else wt, tau)


def make_weights(w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None, sh_gate=None,
                 sh_up=None, sh_down=None, sh_s_gate=None, sh_s_up=None, sh_s_down=None) -> Weights:
    return Weights(*[_ptr(t) for t in (w_gate, w_up, w_down, s_gate, s_up, s_down, sh_gate,
                                       sh_up, sh_down, sh_s_gate, sh_s_up, sh_s_down)])


def moe_workspace_bytes(shape: Shape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape)))


def moe_strerror(status: int) -> str:
    return lib().moe_strerror(status).decode()


def moe_route(shape, x, w_router, b_router, logits, topk_idx, topk_w, stream=None):
    return _call("moe_route", ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(b_router),
                 _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _stream(stream))


def moe_dispatch(shape, topk_idx, counts, offsets, perm, inv, stream=None):
    return _call("moe_dispatch", ctypes.byref(shape), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                 _ptr(perm), _ptr(inv), _stream(stream))


def moe_expert_ffn(shape, x, weights, counts, offsets, perm, y_perm, y_shared, ws, ws_bytes=None,
                   stream=None):
    nbytes = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    return _call("moe_expert_ffn", ctypes.byref(shape), _ptr(x), ctypes.byref(weights),
                 _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(y_perm), _ptr(y_shared), _ptr(ws),
                 nbytes, _stream(stream))


def moe_combine(shape, y_perm, inv, topk_w, y_shared, residual, y, stream=None):
    return _call("moe_combine", ctypes.byref(shape), _ptr(y_perm), _ptr(inv), _ptr(topk_w),
                 _ptr(y_shared), _ptr(residual), _ptr(y), _stream(stream))


def moe_layer_forward(shape, x, w_router, b_router, weights, residual, y, counts_out, topk_idx_out,
                      ws, ws_bytes=None, stream=None):
    nbytes = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    return _call("moe_layer_forward", ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(b_router),
                 ctypes.byref(weights), _ptr(residual), _ptr(y), _ptr(counts_out),
                 _ptr(topk_idx_out), _ptr(ws), nbytes, _stream(stream))


def moe_layer_forward_noalloc(shape, x, w_router, b_router, weights, residual, y, counts_out,
                              topk_idx_out, stream=None):
    """moe_layer_forward on the library's fixed device workspace (no allocation)."""
    return _call("moe_layer_forward_noalloc", ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(b_router),
                 ctypes.byref(weights), _ptr(residual), _ptr(y), _ptr(counts_out), _ptr(topk_idx_out),
                 _stream(stream))


def moe_pack_int4_tiled(src, dst, n_mats, N, K, stream=None):
    """Row-major int4 codes (n_mats x [N][K/2] bytes) -> the tiled layout."""
    return _call("moe_pack_int4_tiled", _ptr(src), _ptr(dst), int(n_mats), int(N), int(K), _stream(stream))


def moe_pack_mxfp8_tiled(src, dst, n_mats, N, K, stream=None):
    """Row-major MXFP8 codes (n_mats x [N][K] bytes) -> the tiled layout."""
    return _call("moe_pack_mxfp8_tiled", _ptr(src), _ptr(dst), int(n_mats), int(N), int(K), _stream(stream))


def moe_topk_overlap(shape, pred_idx, actual_idx, hist, stream=None):
    """hist[j] = tokens whose two top-k selections share j experts."""
    return _call("moe_topk_overlap", ctypes.byref(shape), _ptr(pred_idx), _ptr(actual_idx), _ptr(hist),
                 _stream(stream))


def moe_rmsnorm(shape, h, gamma, eps, out, stream=None):
    return _call("moe_rmsnorm", ctypes.byref(shape), _ptr(h), _ptr(gamma), float(eps), _ptr(out),
                 _stream(stream))
