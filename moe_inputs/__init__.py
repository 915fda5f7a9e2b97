"""Seeded synthetic inputs for the MoE layer forward.

This module is shared by the oracle side (tests, CPU baseline) and the GPU
side (tests, bench).  It holds none of the layer's arithmetic: it only draws
random tensors, rounds them to their storage dtype and packs int4 codes.  The
one data file it reads (the calibrated router bias of the prefill workload) is
written by ``oracle/make_zipf_bias.py``.

Recipe (every tensor has its own torch generator, seeded from a SHA-256 of
``(seed, model, layer, tensor, expert)``, so any single expert can be redrawn
alone and the decode and prefill workloads of one model share their weights):

* activations ``x ~ N(0, 1)`` drawn in fp32 on the CPU, rounded to the
  activation dtype (bf16 round-to-nearest-even);
* router ``W_g`` drawn in fp32 with std ``w_std`` (or ``1/sqrt(d)``), kept fp32;
* expert weights drawn in fp32 with std ``w_std`` (or ``1/sqrt(fan_in)``) on the
  requested device, then rounded to bf16, kept fp32, or quantised to
  symmetric int4 with one fp16 scale per 128 (or 64) consecutive K elements:
  ``s = fp16(absmax/7)``, ``q = clamp(round_half_even(w/s), -8, 7)``, two codes
  per byte, the even K index in the low nibble; or to an OCP MX format (E2M1
  or E4M3 elements, one E8M0 power-of-two scale per 32 K elements,
  ``X = 2^(floor(log2 absmax) - emax)``, elements rounded to nearest even and
  saturated);
* the stacked workload's routers follow ``W_{l+1} = 0.7 W_l + 0.3 N(0, 0.02)``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import json
import os
from typing import Dict, List, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
ZIPF_BIAS_FILE = os.path.join(_HERE, "zipf_bias_mixtral_prefill.json")


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    act: str            # "f32" | "bf16"
    wt: str             # "f32" | "bf16" | "int4" | "int4g64" | "mxfp4" | "mxfp8"
    model: str          # weight family; workloads of one model share weights
    n_shared: int = 0
    layers: int = 1
    w_std: Optional[float] = None   # None: 1/sqrt(fan_in)
    router_bias: Optional[str] = None  # None | "zipf"
    description: str = ""

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, MoEConfig] = {
    "tiny_f32": MoEConfig(
        "tiny_f32", T=16, d=64, E=8, k=2, F=128, act="f32", wt="f32",
        model="tiny", description="tiny fp32 layer, T=16 d=64 E=8 top-2 F=128"),
    "mixtral_decode": MoEConfig(
        "mixtral_decode", T=8, d=4096, E=8, k=2, F=14336, act="bf16", wt="bf16",
        model="mixtral", w_std=0.02,
        description="Mixtral-8x7B-shaped layer, decode T=8, bf16"),
    "mixtral_prefill": MoEConfig(
        "mixtral_prefill", T=4096, d=4096, E=8, k=2, F=14336, act="bf16", wt="bf16",
        model="mixtral", w_std=0.02, router_bias="zipf",
        description="Mixtral-8x7B-shaped layer, prefill T=4096, bf16, Zipf(1.1) expert load"),
    "fine_int4_decode": MoEConfig(
        "fine_int4_decode", T=64, d=7168, E=256, k=8, F=2048, act="bf16", wt="int4",
        model="fine256", n_shared=1, w_std=0.02,
        description="fine-grained layer, T=64 d=7168 E=256 top-8 + 1 shared, int4-g128"),
    "fine_int4_prefill": MoEConfig(
        "fine_int4_prefill", T=4096, d=7168, E=256, k=8, F=2048, act="bf16", wt="int4",
        model="fine256", n_shared=1, w_std=0.02,
        description="the fine-grained int4-g128 layer at prefill, T=4096"),
    "fine_mxfp4_prefill": MoEConfig(
        "fine_mxfp4_prefill", T=4096, d=7168, E=256, k=8, F=2048, act="bf16", wt="mxfp4",
        model="fine256", n_shared=1, w_std=0.02,
        description="the fine-grained layer with MXFP4 experts (E2M1, E8M0 per 32) at prefill"),
    "mixtral_mxfp8_prefill": MoEConfig(
        "mixtral_mxfp8_prefill", T=4096, d=4096, E=8, k=2, F=14336, act="bf16", wt="mxfp8",
        model="mixtral", w_std=0.02,
        description="the Mixtral-shaped layer with MXFP8 experts (E4M3, E8M0 per 32) at prefill"),
    "stack4": MoEConfig(
        "stack4", T=512, d=2048, E=64, k=6, F=1408, act="bf16", wt="bf16",
        model="stack64", layers=4, w_std=0.02,
        description="4 pre-norm MoE layers with residual, T=512 d=2048 E=64 top-6 F=1408"),
}

ZIPF_S = 1.1


def zipf_targets(E: int, s: float = ZIPF_S) -> List[float]:
    """Target selection frequencies p_r proportional to r^-s, expert 0 most frequent."""
    raw = [(r + 1) ** (-s) for r in range(E)]
    tot = sum(raw)
    return [v / tot for v in raw]


def tensor_seed(seed: int, model: str, layer: int, tensor: str, expert: int = -1) -> int:
    h = hashlib.sha256(f"{seed}/{model}/{layer}/{tensor}/{expert}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def randn(shape, std: float, s: int, device="cpu") -> torch.Tensor:
    g = _gen(device, s)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std)


def quantise_int4_g128(w: torch.Tensor, gs: int = 128):
    """Symmetric int4, gs-element groups along the last (K) axis, fp16 scales.

    Returns (packed uint8 [..., K/2], scales fp16 [..., K/gs]).  Low nibble of
    each byte holds the even K index.
    """
    *lead, K = w.shape
    assert K % gs == 0
    g = w.reshape(*lead, K // gs, gs)
    s16 = (g.abs().amax(dim=-1) / 7.0).to(torch.float16)
    s32 = s16.to(torch.float32).unsqueeze(-1)
    safe = torch.where(s32 > 0, s32, torch.ones_like(s32))
    q = torch.round(g / safe).clamp_(-8, 7)
    q = torch.where(s32 > 0, q, torch.zeros_like(q)).to(torch.int16).reshape(*lead, K)
    u = (q & 0xF).to(torch.uint8)
    packed = u[..., 0::2] | (u[..., 1::2] << 4)
    return packed.contiguous(), s16.contiguous()


# OCP MX element formats: E2M1 (fp4, 2 exponent bits, bias 1, no inf/nan,
# largest 6 = 1.5 * 2^2) and E4M3 (fp8 "fn": bias 7, largest 448 = 1.75 * 2^8)
_E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_MX_EMAX = {"e2m1": 2, "e4m3": 8}


def quantise_mx(w: torch.Tensor, elem: str, block: int = 32):
    """MX quantisation along the last (K) axis: blocks of 32 elements share an
    E8M0 scale X = 2^(floor(log2(amax)) - emax_elem); each element is v / X
    rounded to the nearest element value (ties to the even mantissa),
    saturating at the element format's largest magnitude.

    Returns (codes, scales): codes uint8 [..., K/2] (E2M1, two per byte, the
    even K index in the low nibble) or [..., K] (E4M3); scales uint8 E8M0
    codes (2^(code - 127)) [..., K/32]."""
    *lead, K = w.shape
    assert K % block == 0
    g = w.reshape(*lead, K // block, block).to(torch.float32)
    amax = g.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                       # amax = m * 2^ex, m in [0.5, 1)
    shared = torch.where(amax > 0, ex - 1 - _MX_EMAX[elem], torch.zeros_like(ex))
    shared = shared.clamp(-127, 127)
    scale_code = (shared + 127).to(torch.uint8)
    # dividing by a power of two is exact in fp32 (the weights are far from
    # the subnormal range)
    v = torch.ldexp(g, (-shared).unsqueeze(-1).to(torch.float32))
    if elem == "e4m3":
        q = v.clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        codes = q.view(torch.uint8).reshape(*lead, K)
    else:
        # nearest E2M1 magnitude code: count the midpoints below |v|; a value
        # on a midpoint goes to the neighbour with the even mantissa (code 0,
        # 2, 4 or 6), i.e. down at 0.25, 1.25, 2.5, 5 and up at 0.75, 1.75, 3.5
        a = v.abs()
        mag = torch.zeros_like(a, dtype=torch.uint8)
        for b, up in ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True),
                      (5.0, False)):
            mag += (a >= b if up else a > b).to(torch.uint8)
        sign = ((v < 0) & (mag > 0)).to(torch.uint8) << 3
        nib = (mag | sign).reshape(*lead, K)
        codes = (nib[..., 0::2] | (nib[..., 1::2] << 4)).contiguous()
    return codes.contiguous(), scale_code.reshape(*lead, K // block).contiguous()


def _store(w32: torch.Tensor, wt: str):
    if wt == "f32":
        return {"w": w32.contiguous(), "s": None}
    if wt == "bf16":
        return {"w": w32.to(torch.bfloat16).contiguous(), "s": None}
    if wt == "int4":
        p, s = quantise_int4_g128(w32)
        return {"w": p, "s": s}
    if wt == "int4g64":
        p, s = quantise_int4_g128(w32, gs=64)
        return {"w": p, "s": s}
    if wt in ("mxfp4", "mxfp8"):
        c, s = quantise_mx(w32, "e2m1" if wt == "mxfp4" else "e4m3")
        return {"w": c, "s": s}
    raise ValueError(wt)


def _act_dtype(act: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[act]


def expert_matrix(cfg: MoEConfig, seed: int, layer: int, name: str, e: int,
                  device="cpu", shared: bool = False):
    """One expert's weight matrix in storage form: dict(w=..., s=...).

    gate/up are [F, d] (K = d contiguous), down is [d, F] (K = F contiguous).
    """
    d, F = cfg.d, cfg.F
    N, K = (F, d) if name in ("gate", "up") else (d, F)
    std = cfg.w_std if cfg.w_std is not None else 1.0 / (K ** 0.5)
    tname = ("sh_" if shared else "") + name
    w32 = randn((N, K), std, tensor_seed(seed, cfg.model, layer, tname, e), device)
    return _store(w32, cfg.wt)


def _stack_experts(cfg, seed, layer, name, device, n, shared=False, experts=None):
    ws, ss = [], []
    for e in range(n):
        if experts is not None and e not in experts:
            ws.append(None)
            ss.append(None)
            continue
        m = expert_matrix(cfg, seed, layer, name, e, device, shared)
        ws.append(m["w"])
        ss.append(m["s"])
    if experts is not None:
        # fill unrequested experts with zeros of the right shape (tests only)
        ref = next(w for w in ws if w is not None)
        refs = next((s for s in ss if s is not None), None)
        ws = [w if w is not None else torch.zeros_like(ref) for w in ws]
        if refs is not None:
            ss = [s if s is not None else torch.zeros_like(refs) for s in ss]
    w = torch.stack(ws).contiguous()
    s = torch.stack(ss).contiguous() if ss[0] is not None else None
    return w, s


def router_weights(cfg: MoEConfig, seed: int, layer: int) -> torch.Tensor:
    """Router W_g [E, d] fp32 (CPU).  Layers of a stack are correlated."""
    std = cfg.w_std if cfg.w_std is not None else 1.0 / (cfg.d ** 0.5)
    w = randn((cfg.E, cfg.d), std, tensor_seed(seed, cfg.model, 0, "router"))
    for l in range(1, layer + 1):
        fresh = randn((cfg.E, cfg.d), 0.02, tensor_seed(seed, cfg.model, l, "router_fresh"))
        w = 0.7 * w + 0.3 * fresh
    return w.contiguous()


def router_bias(cfg: MoEConfig) -> Optional[torch.Tensor]:
    if cfg.router_bias is None:
        return None
    if cfg.router_bias == "zipf":
        with open(ZIPF_BIAS_FILE) as f:
            data = json.load(f)
        if data["T"] != cfg.T or data["E"] != cfg.E or data["d"] != cfg.d:
            raise ValueError("stored Zipf bias was calibrated for another shape")
        return torch.tensor(data["bias"], dtype=torch.float32)
    raise ValueError(cfg.router_bias)


def activations(cfg: MoEConfig, seed: int) -> torch.Tensor:
    x = randn((cfg.T, cfg.d), 1.0, tensor_seed(seed, cfg.name, 0, "x"))
    return x.to(_act_dtype(cfg.act)).contiguous()


def generate(cfg: MoEConfig, seed: int = 0, device="cpu", experts=None) -> dict:
    """All inputs of one workload.  Small tensors are drawn on the CPU; expert
    weights are drawn on ``device`` (CUDA and CPU generators give different
    streams, so a run that compares both sides copies one side's tensors to
    the other).  ``experts`` (a set) restricts which routed experts are drawn;
    the others are zero (used only by CPU tests that need one expert).
    """
    out = {"cfg": cfg, "seed": seed, "x": activations(cfg, seed), "layers": []}
    for l in range(cfg.layers):
        L = {"w_router": router_weights(cfg, seed, l), "b_router": router_bias(cfg)}
        for name in ("gate", "up", "down"):
            w, s = _stack_experts(cfg, seed, l, name, device, cfg.E, experts=experts)
            L["w_" + name] = w
            L["s_" + name] = s
            if cfg.n_shared:
                w, s = _stack_experts(cfg, seed, l, name, device, cfg.n_shared, shared=True)
                L["sh_" + name] = w
                L["sh_s_" + name] = s
            else:
                L["sh_" + name] = None
                L["sh_s_" + name] = None
        out["layers"].append(L)
    if cfg.layers > 1:
        out["gamma"] = [torch.ones(cfg.d, dtype=torch.float32) for _ in range(cfg.layers)]
        out["eps"] = 1e-6
    return out
