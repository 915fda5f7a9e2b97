"""Concurrent callers: the library keeps no state between calls beyond
per-device attribute caches set once, so host threads calling
moe_layer_forward at the same time on their own streams and workspaces must
each get the output a lone sequential call gets, bit for bit.  The threaded
calls run first in the process, so they also race on those caches being set."""
import threading

import pytest
import torch

import moe_inputs
import moe_layer_forward_amd as moe
from gpu_common import DEV, act_dtype, device_inputs, run_layer, say, shape_of, weights_struct

pytestmark = pytest.mark.gpu

CASES = [
    # fused decode routing + GEMV experts
    moe_inputs.MoEConfig("conc_decode", T=8, d=512, E=8, k=2, F=1024, act="bf16", wt="bf16",
                         model="s_conc_dec", w_std=0.05),
    # 64-row and 256-row MFMA tiles, a bf16 shared expert
    moe_inputs.MoEConfig("conc_prefill", T=600, d=256, E=6, k=2, F=384, act="bf16", wt="bf16",
                         model="s_conc_pre", n_shared=1, w_std=0.05),
    # int4 experts on the matrix cores with a shared expert in the same launch
    moe_inputs.MoEConfig("conc_int4", T=16, d=1024, E=16, k=4, F=1024, act="bf16", wt="int4",
                         model="s_conc_i4", n_shared=1, w_std=0.05),
    # int4 groups on the dequantising GEMM, short last tiles on the skinny kernel
    moe_inputs.MoEConfig("conc_int4_dq", T=300, d=1024, E=4, k=2, F=1024, act="bf16", wt="int4",
                         model="s_conc_i4dq", n_shared=1, w_std=0.05),
]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_threads_on_own_streams_match_sequential():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    say("concurrent callers on their own streams")
    inputs = [device_inputs(c) for c in CASES]
    torch.cuda.synchronize()
    reps = 4
    outs = [[None] * reps for _ in CASES]
    errors = []
    start = threading.Barrier(len(CASES))

    def worker(i):
        try:
            cfg, d = CASES[i], inputs[i]
            shape = shape_of(cfg)
            W = weights_struct(d)
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                ws = torch.empty(moe.moe_workspace_bytes(shape), dtype=torch.uint8, device=DEV)
                ys = [torch.empty(cfg.T, cfg.d, dtype=act_dtype(cfg), device=DEV) for _ in range(reps)]
                counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
                idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=DEV)
            start.wait()
            for r in range(reps):
                moe.moe_layer_forward(shape, d["x"], d["w_router"], d["b_router"], W, None, ys[r], counts, idx,
                                      ws, stream=st)
            st.synchronize()
            for r in range(reps):
                outs[i][r] = ys[r]
        except Exception as e:   # reported after the join
            errors.append((CASES[i].name, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i, cfg in enumerate(CASES):
        y_ref, _, _ = run_layer(cfg, inputs[i])
        for r in range(reps):
            assert torch.equal(_bits(outs[i][r]), _bits(y_ref)), f"{cfg.name} call {r}"
        say(f"  {cfg.name}: {reps} concurrent calls identical to a sequential one")
