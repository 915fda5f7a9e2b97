"""ctypes binding of libmoe_measure.so (declared in include/moe_measure.h).

Measurement helpers beside the layer, not part of it: the HBM read ceiling and
the bf16 matrix-core ceiling of the GPU, against which the bench reads its
roofline fractions next to the published peaks.  Argument marshalling only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

from ._lib import MoEError, _ptr, _stream

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_measure.so")
EXPORTS = ("moe_mfma_ceiling", "moe_read_ceiling")

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (run python -m moe_layer_forward_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, cp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_char_p
        L.moe_read_ceiling.argtypes = [vp, sz, vp, vp, cp, sz]
        L.moe_mfma_ceiling.argtypes = [ctypes.c_int32, vp, sz, vp, ctypes.POINTER(ctypes.c_int64), vp, cp, sz]
        for n in EXPORTS:
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def _call(name, *args):
    buf = ctypes.create_string_buffer(512)
    rc = getattr(lib(), name)(*args, buf, len(buf))
    if rc != 0:
        raise MoEError(name, rc, buf.value.decode(errors="replace"))
    return rc


def moe_mfma_ceiling(iters, sink, sink_bytes, clock=None, stream=None):
    """Independent bf16 MFMAs on every CU; returns the launch's flop count.
    clock: device uint64[2] (shader cycles, 100 MHz ticks) or None."""
    flops = ctypes.c_int64(0)
    _call("moe_mfma_ceiling", int(iters), _ptr(sink), int(sink_bytes), _ptr(clock), ctypes.byref(flops),
          _stream(stream))
    return flops.value


def moe_read_ceiling(buf, nbytes, sink, stream=None):
    """Streaming read of nbytes at buf, every 32-bit word XORed into sink."""
    return _call("moe_read_ceiling", _ptr(buf), int(nbytes), _ptr(sink), _stream(stream))
