"""fp64 CPU oracle of the MoE layer forward (ctypes over ``liboracle.so``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
bench's CPU-baseline leg, never by the product package.  It shares no code with
the HIP library.  Inputs are NumPy arrays in storage form: fp32 arrays, bf16 and
fp16 codes as ``uint16``, packed int4 codes as ``uint8``.  Outputs are float64.

The arithmetic lives in ``oracle.c``; each function there cites the passage of
the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, INT4_G128, INT4_G64, MXFP4, MXFP8 = 0, 1, 2, 3, 4, 5
DTYPES = {"f32": F32, "bf16": BF16, "int4": INT4_G128, "int4g64": INT4_G64, "mxfp4": MXFP4,
          "mxfp8": MXFP8}
MF_IEEE, MF_FN, MF_FINITE = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        L.orc_dec_bf16.restype = ctypes.c_double
        L.orc_dec_bf16.argtypes = [ctypes.c_uint16]
        L.orc_dec_f16.restype = ctypes.c_double
        L.orc_dec_f16.argtypes = [ctypes.c_uint16]
        L.orc_dec_int4.restype = ctypes.c_int
        L.orc_dec_int4.argtypes = [ctypes.c_uint8, ctypes.c_int]
        L.orc_dec_minifloat.restype = ctypes.c_double
        L.orc_dec_minifloat.argtypes = [ctypes.c_uint32, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.orc_dec_e8m0.restype = ctypes.c_double
        L.orc_dec_e8m0.argtypes = [ctypes.c_uint8]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "need C-contiguous ndarray"
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (rc={rc})")


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of later oracle calls (timing only; results do not depend on it)."""
    lib().orc_set_num_threads(ctypes.c_int(int(n)))


def dec_bf16(h: int) -> float:
    return lib().orc_dec_bf16(h)


def dec_f16(h: int) -> float:
    return lib().orc_dec_f16(h)


def dec_int4(byte: int, hi: int) -> int:
    return lib().orc_dec_int4(byte, hi)


def dec_minifloat(code: int, ebits: int, mbits: int, bias: int, special: int) -> float:
    return lib().orc_dec_minifloat(code, ebits, mbits, bias, special)


def dec_e8m0(code: int) -> float:
    return lib().orc_dec_e8m0(code)


def router_logits(x, act, w_router, b_router=None):
    T, d = x.shape
    E = w_router.shape[0]
    out = np.empty((T, E), np.float64)
    _check(lib().orc_router_logits(T, d, E, DTYPES[act], _p(x), _p(w_router), _p(b_router),
                                   _p(out)), "router_logits")
    return out


def softmax(logits):
    logits = np.ascontiguousarray(logits, np.float64)
    T, E = logits.shape
    out = np.empty_like(logits)
    _check(lib().orc_softmax(T, E, _p(logits), _p(out)), "softmax")
    return out


def topk(logits, k):
    logits = np.ascontiguousarray(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _check(lib().orc_topk(T, E, k, _p(logits), _p(idx), _p(w)), "topk")
    return idx, w


def gate_weights(logits, idx):
    logits = np.ascontiguousarray(logits, np.float64)
    idx = np.ascontiguousarray(idx, np.int32)
    T, E = logits.shape
    k = idx.shape[1]
    w = np.empty((T, k), np.float64)
    _check(lib().orc_gate_weights(T, E, k, _p(logits), _p(idx), _p(w)), "gate_weights")
    return w


def dispatch(idx, E):
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    _check(lib().orc_dispatch(T, k, E, _p(idx), _p(counts), _p(offsets), _p(perm), _p(inv)),
           "dispatch")
    return counts, offsets, perm, inv


def _wargs(W):
    return [_p(W["w_gate"]), _p(W["w_up"]), _p(W["w_down"]),
            _p(W.get("s_gate")), _p(W.get("s_up")), _p(W.get("s_down"))]


def expert_ffn(x, act, wt, W, counts, offsets, perm, k):
    T, d = x.shape
    E, F = W["w_gate"].shape[0], W["w_gate"].shape[1]
    yp = np.empty((T * k, d), np.float64)
    _check(lib().orc_expert_ffn(T, d, E, k, F, DTYPES[act], DTYPES[wt], _p(x), *_wargs(W),
                                _p(counts), _p(offsets), _p(perm), _p(yp)), "expert_ffn")
    return yp


def shared_ffn(x, act, wt, S):
    """S: dict with w_gate/w_up/w_down [1,...] and optional s_* scales."""
    T, d = x.shape
    F = S["w_gate"].shape[1]
    ys = np.empty((T, d), np.float64)
    _check(lib().orc_shared_ffn(T, d, F, DTYPES[act], DTYPES[wt], _p(x), *_wargs(S), _p(ys)),
           "shared_ffn")
    return ys


def combine(y_perm, inv, w, k, ys=None, residual=None, res_act="f32"):
    y_perm = np.ascontiguousarray(y_perm, np.float64)
    w = np.ascontiguousarray(w, np.float64)
    d = y_perm.shape[1]
    T = w.shape[0]
    y = np.empty((T, d), np.float64)
    _check(lib().orc_combine(T, d, k, _p(y_perm), _p(np.ascontiguousarray(inv, np.int32)),
                             _p(w), _p(ys), _p(residual), DTYPES[res_act], _p(y)), "combine")
    return y


def layer_forward(x, act, wt, k, w_router, b_router, W, S=None, residual=None,
                  forced_idx=None, sel=None):
    """Returns (y [n_sel or T, d] f64, idx, w, logits) for the selected tokens."""
    T, d = x.shape
    E, F = W["w_gate"].shape[0], W["w_gate"].shape[1]
    sel_a = None if sel is None else np.ascontiguousarray(sel, np.int32)
    n = T if sel_a is None else len(sel_a)
    y = np.empty((n, d), np.float64)
    idx = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    lg = np.empty((n, E), np.float64)
    S = S or {}
    fi = None if forced_idx is None else np.ascontiguousarray(forced_idx, np.int32)
    _check(lib().orc_layer_forward(
        T, d, E, k, F, DTYPES[act], DTYPES[wt], _p(x), _p(w_router), _p(b_router), *_wargs(W),
        _p(S.get("w_gate")), _p(S.get("w_up")), _p(S.get("w_down")),
        _p(S.get("s_gate")), _p(S.get("s_up")), _p(S.get("s_down")),
        _p(residual), _p(fi), n, _p(sel_a), _p(y), _p(idx), _p(w), _p(lg)), "layer_forward")
    return y, idx, w, lg


def topk_overlap(pred, actual):
    """hist[j] = tokens whose two top-k lists share j experts (j = 0..k)."""
    pred = np.ascontiguousarray(pred, np.int32)
    actual = np.ascontiguousarray(actual, np.int32)
    T, k = pred.shape
    hist = np.empty(k + 1, np.int32)
    _check(lib().orc_topk_overlap(T, k, _p(pred), _p(actual), _p(hist)), "topk_overlap")
    return hist


def rmsnorm(h, act, gamma, eps):
    T, d = h.shape
    out = np.empty((T, d), np.float64)
    _check(lib().orc_rmsnorm(T, d, DTYPES[act], _p(h), _p(gamma), ctypes.c_double(eps), _p(out)),
           "rmsnorm")
    return out
