"""The layer captured in a HIP graph (torch.cuda.CUDAGraph over the C-ABI
call) and replayed: every replay, with eager layer calls on other inputs and
device synchronisations between replays, must reproduce the eager output bit
for bit (same kernels, same inputs)."""
import pytest
import torch

import moe_inputs
import moe_layer_forward_amd as moe
from gpu_common import DEV, act_dtype, device_inputs, run_layer, say, shape_of, weights_struct

pytestmark = pytest.mark.gpu

CASES = [
    # decode batch: fused routing kernel, GEMV experts
    moe_inputs.MoEConfig("graph_decode", T=8, d=512, E=8, k=2, F=1024, act="bf16", wt="bf16",
                         model="s_graph_dec", w_std=0.05),
    # 256-row MFMA tiles with a split tail round and a bf16 shared expert
    moe_inputs.MoEConfig("graph_prefill", T=600, d=256, E=6, k=2, F=384, act="bf16", wt="bf16",
                         model="s_graph_pre", n_shared=1, w_std=0.05),
    # int4 experts on the matrix cores
    moe_inputs.MoEConfig("graph_int4", T=16, d=1024, E=16, k=4, F=1024, act="bf16", wt="int4",
                         model="s_graph_i4", n_shared=1, w_std=0.05),
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_graph_replay_matches_eager(cfg):
    say(f"graph replay {cfg.name}")
    d = device_inputs(cfg)
    y_ref, c_ref, i_ref = run_layer(cfg, d)
    shape = shape_of(cfg)
    W = weights_struct(d)
    ws = torch.empty(moe.moe_workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    y = torch.empty(cfg.T, cfg.d, dtype=act_dtype(cfg), device=DEV)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_layer_forward(shape, d["x"], d["w_router"], d["b_router"], W, None, y, counts, idx, ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer_forward(shape, d["x"], d["w_router"], d["b_router"], W, None, y, counts, idx, ws,
                              stream=torch.cuda.current_stream())
    other = (d["x"].float() * -0.5).to(d["x"].dtype).contiguous()
    for r in range(4):
        y.fill_(0)
        counts.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_ref)), f"replay {r}"
        assert torch.equal(counts, c_ref) and torch.equal(idx, i_ref), f"replay {r}"
        # eager work between replays, on other inputs and the graph's own workspace
        run_layer(cfg, dict(d, x=other))
        moe.moe_layer_forward(shape, other, d["w_router"], d["b_router"], W, None, y, counts, idx, ws)
        torch.cuda.synchronize()
    say(f"  {cfg.name}: 4 replays identical to the eager call")
