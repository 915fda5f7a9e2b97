"""Shared pieces of the GPU parity tests: device inputs, the C-ABI calls in the
layer's order, and the comparisons against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import moe_inputs
import moe_layer_forward_amd as moe
from helpers import np_store

DEV = "cuda"
TOL = {"f32": 1e-5, "bf16": 2e-2, "int4": 2e-2, "int4_tiled": 2e-2, "int4g64": 2e-2, "mxfp4": 2e-2,
       "mxfp8": 2e-2}
FLIP_MARGIN = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(cfg, seed=0, layer=0, experts=None):
    """Inputs of one layer on the GPU: small tensors drawn on the CPU and copied,
    expert weights drawn on the GPU."""
    inp = moe_inputs.generate(cfg, seed=seed, device=DEV, experts=experts)
    L = inp["layers"][layer]
    out = {"x": inp["x"].to(DEV), "w_router": L["w_router"].to(DEV),
           "b_router": None if L["b_router"] is None else L["b_router"].to(DEV)}
    for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
              "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down"):
        t = L.get(n)
        out[n] = None if t is None else t.to(DEV).contiguous()
    return out


def weights_struct(d):
    return moe.make_weights(d["w_gate"], d["w_up"], d["w_down"], d["s_gate"], d["s_up"],
                            d["s_down"], d["sh_gate"], d["sh_up"], d["sh_down"], d["sh_s_gate"],
                            d["sh_s_up"], d["sh_s_down"])


def oracle_weights(d):
    W = {n: np_store(d[n]) for n in ("w_gate", "w_up", "w_down")}
    for n in ("s_gate", "s_up", "s_down"):
        W[n] = np_store(d[n]) if d[n] is not None else None
    S = None
    if d["sh_gate"] is not None:
        S = {"w_gate": np_store(d["sh_gate"]), "w_up": np_store(d["sh_up"]),
             "w_down": np_store(d["sh_down"]),
             "s_gate": np_store(d["sh_s_gate"]), "s_up": np_store(d["sh_s_up"]),
             "s_down": np_store(d["sh_s_down"])}
    return W, S


def shape_of(cfg, tau=0, T=None, wt=None):
    return moe.make_shape(cfg.T if T is None else T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.act,
                          cfg.wt if wt is None else wt, cfg.n_shared, tau)


def tiled_inputs(d, wt="int4"):
    """The same inputs with every code tensor packed into the tiled layout
    (moe_pack_int4_tiled, or moe_pack_mxfp8_tiled for MXFP8 codes, through the
    C ABI); the oracle keeps reading d."""
    t = moe.layer.pack_mxfp8_tiled(d) if wt == "mxfp8" else moe.layer.pack_int4_tiled(d)
    torch.cuda.synchronize()
    return t


def act_dtype(cfg):
    return torch.float32 if cfg.act == "f32" else torch.bfloat16


def run_layer(cfg, d, tau=0, residual=None, x=None, wt=None):
    """moe_layer_forward through the C ABI; returns (y, counts, topk_idx).
    wt overrides the weight dtype code (e.g. "int4_tiled" with packed codes)."""
    x = d["x"] if x is None else x
    T = x.shape[0]
    shape = shape_of(cfg, tau, T, wt)
    ws = torch.empty(moe.moe_workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    y = torch.empty(T, cfg.d, dtype=act_dtype(cfg), device=DEV)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    idx = torch.empty(T, cfg.k, dtype=torch.int32, device=DEV)
    moe.moe_layer_forward(shape, x, d["w_router"], d["b_router"], weights_struct(d), residual, y,
                          counts, idx, ws)
    torch.cuda.synchronize()
    return y, counts, idx


def topk_margins(logits, k):
    """fp64 margins: gap between the k-th and (k+1)-th logit, and the smallest gap
    between consecutive selected logits (a near-tie inside the selection)."""
    s = -np.sort(-logits, axis=1)
    kth = s[:, k - 1] - (s[:, k] if logits.shape[1] > k else -np.inf)
    inner = np.min(s[:, :k - 1] - s[:, 1:k], axis=1) if k > 1 else np.full(len(s), np.inf)
    return kth, inner


def check_routing_with_flips(gpu_idx, orc_idx, orc_logits, k):
    """End-to-end routing rule: indices equal the oracle's except at tokens whose
    fp64 margin is below FLIP_MARGIN (set flip) or whose selected logits are
    within FLIP_MARGIN (slot swap).  Returns the number of flipped tokens."""
    bad = np.where((gpu_idx != orc_idx).any(axis=1))[0]
    if len(bad) == 0:
        return 0
    kth, inner = topk_margins(orc_logits[bad], k)
    for i, t in enumerate(bad):
        same_set = set(gpu_idx[t].tolist()) == set(orc_idx[t].tolist())
        ok = kth[i] < FLIP_MARGIN or (same_set and inner[i] < FLIP_MARGIN)
        assert ok, (f"token {t}: gpu {gpu_idx[t].tolist()} oracle {orc_idx[t].tolist()} "
                    f"margins kth={kth[i]:.3g} inner={inner[i]:.3g}")
    return len(bad)


def tokenwise_rel(y, r):
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    num = np.abs(y - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return num / den
