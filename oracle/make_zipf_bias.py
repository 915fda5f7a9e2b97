"""Calibrate the router bias of the Mixtral-shaped prefill workload (T=4096).

The workload asks for a router bias under which the experts' top-2 selection
frequencies follow Zipf(s=1.1) over the 8 experts (expert 0 most frequent).
Reading taken: start from b = 0 and iterate b <- b + 0.5*(ln p - ln f) for 200
steps, where p are the Zipf targets and f the achieved top-2 assignment
frequencies on the workload's own activations, with the oracle's fp64 logits
and top-k.  The bias is frozen as fp32 and stored beside the input generator.

Run:  python -m oracle.make_zipf_bias
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
import moe_inputs  # noqa: E402


def storage(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def calibrate(cfg, seed=0, iters=200, step=0.5):
    x = storage(moe_inputs.activations(cfg, seed))
    wg = storage(moe_inputs.router_weights(cfg, seed, 0))
    L0 = oracle.router_logits(x, cfg.act, wg, None)
    p = np.array(moe_inputs.zipf_targets(cfg.E))
    b = np.zeros(cfg.E)
    for _ in range(iters):
        b32 = b.astype(np.float32).astype(np.float64)
        idx, _ = oracle.topk(L0 + b32[None, :], cfg.k)
        f = np.bincount(idx.ravel(), minlength=cfg.E) / idx.size
        f = np.maximum(f, 0.5 / idx.size)
        b = b + step * (np.log(p) - np.log(f))
        b = b - b.mean()
    b32 = b.astype(np.float32)
    idx, _ = oracle.topk(L0 + b32.astype(np.float64)[None, :], cfg.k)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    return b32, counts


def main():
    oracle.build(force=False)
    cfg = moe_inputs.CONFIGS["mixtral_prefill"]
    b, counts = calibrate(cfg)
    data = {
        "workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "seed": 0,
        "zipf_s": moe_inputs.ZIPF_S, "targets": moe_inputs.zipf_targets(cfg.E),
        "bias": [float(v) for v in b],
        "achieved_counts": [int(c) for c in counts],
        "written_by": "oracle/make_zipf_bias.py (oracle router logits + top-k only)",
    }
    with open(moe_inputs.ZIPF_BIAS_FILE, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps(data))
    assert all(math.isfinite(v) for v in data["bias"])


if __name__ == "__main__":
    main()
