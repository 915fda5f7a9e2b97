"""MI355X (gfx950) MoE layer forward: hand-written HIP kernels behind a C ABI.

The layer (router -> softmax -> top-k -> dispatch -> SwiGLU experts -> combine)
runs entirely in ``libmoe.so``; this package is its ctypes binding plus a
small helper that owns device buffers for one layer.
"""
from . import layer, measure  # noqa: F401
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, MOE_BF16, MOE_EHIP, MOE_EINVAL, MOE_ENOMEM, MOE_EUNSUPPORTED, MOE_F32,
    MOE_INT4_G128, MOE_INT4_G128_TILED, MOE_INT4_G64, MOE_MXFP4, MOE_MXFP4_TILED, MOE_MXFP8, MOE_MXFP8_TILED, MOE_OK, MoEError, Shape, Weights, lib, make_shape,
    make_weights, moe_combine, moe_dispatch, moe_expert_ffn, moe_layer_forward,
    moe_layer_forward_noalloc,
    moe_pack_int4_tiled, moe_pack_mxfp8_tiled, moe_rmsnorm, moe_route, moe_topk_overlap,
    moe_strerror,
    moe_workspace_bytes)
