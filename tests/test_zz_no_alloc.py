"""moe_layer_forward_noalloc (the layer on the library's fixed device
workspace, for callers that cannot allocate) against moe_layer_forward with a
caller workspace: same kernels, so the outputs, expert choices and usage
counts must be identical bit for bit, on two calls in a row, the second with
fewer tokens (the fixed array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import moe_inputs
import moe_layer_forward_amd as moe
from gpu_common import DEV, act_dtype, device_inputs, run_layer, say, shape_of, weights_struct

pytestmark = pytest.mark.gpu

SCRATCH = 128 << 20

CASES = [
    # the Mixtral-shaped decode layer (GEMV), then 3 tokens
    (moe_inputs.CONFIGS["mixtral_decode"], 3),
    # 64-row MFMA tiles, skinny kernel and a bf16 shared expert, then 17 tokens
    (moe_inputs.MoEConfig("noalloc_mid", T=120, d=1024, E=4, k=2, F=1536, act="bf16", wt="bf16",
                          model="s_noalloc", n_shared=1, w_std=0.05), 17),
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _noalloc(cfg, d, T):
    x = d["x"][:T].contiguous()
    shape = shape_of(cfg, T=T)
    assert moe.moe_workspace_bytes(shape) <= SCRATCH
    y = torch.full((T, cfg.d), float("nan"), dtype=act_dtype(cfg), device=DEV)
    counts = torch.full((cfg.E,), -1, dtype=torch.int32, device=DEV)
    idx = torch.full((T, cfg.k), -1, dtype=torch.int32, device=DEV)
    moe.moe_layer_forward_noalloc(shape, x, d["w_router"], d["b_router"], weights_struct(d), None, y,
                                  counts, idx)
    torch.cuda.synchronize()
    return y, counts, idx


@pytest.mark.parametrize("cfg,T2", CASES, ids=[c[0].name for c in CASES])
def test_noalloc_matches_layer_forward(cfg, T2):
    say(f"no-alloc layer {cfg.name}: T={cfg.T} then T={T2}")
    d = device_inputs(cfg)
    for T in (cfg.T, T2):
        y, counts, idx = _noalloc(cfg, d, T)
        y_r, counts_r, idx_r = run_layer(cfg, d, x=d["x"][:T].contiguous())
        assert torch.equal(idx, idx_r)
        assert torch.equal(counts, counts_r)
        assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                           y_r.view(torch.int16) if y_r.dtype == torch.bfloat16 else y_r)
        say(f"  T={T}: identical (counts {counts.cpu().tolist()})")


def test_noalloc_rejects_shapes_beyond_its_array():
    cfg = moe_inputs.CONFIGS["mixtral_prefill"]
    shape = shape_of(cfg)
    assert moe.moe_workspace_bytes(shape) > SCRATCH
    p = 1 << 20
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_layer_forward_noalloc(shape, p, p, None, moe.make_weights(p, p, p), None, p, None, None)
    assert ei.value.status == moe.MOE_ENOMEM and "fixed device array" in str(ei.value)
