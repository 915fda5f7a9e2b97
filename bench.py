"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole layer (router, softmax, top-k, dispatch,
expert SwiGLU FFN, combine) over one batch: one moe_layer_forward call through
the C ABI.  The timed region is K back-to-back calls after W warm-up calls,
bracketed by device synchronisation; a HIP event between calls gives the
per-step median and p99.  A second loop of the same length (after its own
warm-up) calls the four steps one by one (route -> dispatch -> expert_ffn ->
combine, the same kernels) with HIP events around moe_expert_ffn.  Inputs and
weights are resident in HBM before the timed region.

The headline is the Mixtral-8x7B-shaped decode layer (T=8).  The same JSON
line carries the prefill layer (T=4096, Zipf-loaded experts, same weights; at
least 20 warm-ups and 50 steps whatever the flags), the fine-grained int4
decode layer (T=64, E=256 + 1 shared expert, tiled int4 codes) and the 4-layer
pre-norm stack (T=512, E=64, top-6) with its per-layer usage histogram.

Roofline: the dominant step is the expert FFN (the GEMV or skinny MFMA gate/up
and down kernels at decode, the MFMA gate/up and down kernels at prefill; the
bench line names the kernels the group sizes select).  Its time is measured
live with HIP events recorded on the library's stream around the
moe_expert_ffn call; its algorithmic bytes are the weight bytes of the experts
actually hit (batch union) plus the activation traffic, its algorithmic flops
2*3*T*k*d*F.

CPU baseline: the fp64 oracle (oracle/, test infrastructure) timed on the
host's cores: the full decode layer repeated to ~10 s, and a seeded sample of
the prefill tokens (one token per thread per call) for ~10 s; each with a
one-thread run, the threads that worked and the CPU model.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_inputs  # noqa: E402
import moe_layer_forward_amd as moe  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s at decode T=8 and prefill T=4096; % of HBM/MFMA roofline"
DEV = "cuda"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def device_layer(cfg, seed=0, layer=0, shared_weights=None):
    inp = moe_inputs.generate(cfg, seed=seed, device=DEV) if shared_weights is None else None
    x = moe_inputs.activations(cfg, seed).to(DEV)
    wr = moe_inputs.router_weights(cfg, seed, layer).to(DEV)
    br = moe_inputs.router_bias(cfg)
    br = None if br is None else br.to(DEV)
    if shared_weights is not None:
        W = shared_weights
    else:
        L = inp["layers"][layer]
        W = {n: (None if L.get(n) is None else L[n].to(DEV)) for n in (
            "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
            "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down")}
    return x, wr, br, W


class Runner:
    """Buffers for one workload and the four C-ABI steps of the layer."""

    def __init__(self, cfg, x, wr, br, W, tau=0, wt=None):
        self.cfg, self.x, self.wr, self.br, self.W = cfg, x, wr, br, W
        T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
        self.wt = cfg.wt if wt is None else wt
        self.shape = moe.make_shape(T, d, E, k, cfg.F, cfg.act, self.wt, cfg.n_shared, tau)
        self.wstruct = moe.make_weights(**W)
        self.ws = torch.empty(moe.moe_workspace_bytes(self.shape), dtype=torch.uint8, device=DEV)
        act = torch.float32 if cfg.act == "f32" else torch.bfloat16
        self.logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
        self.idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        self.w = torch.empty(T, k, dtype=torch.float32, device=DEV)
        self.counts = torch.empty(E, dtype=torch.int32, device=DEV)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        self.perm = torch.empty(T * k, dtype=torch.int32, device=DEV)
        self.inv = torch.empty(T * k, dtype=torch.int32, device=DEV)
        self.yp = torch.empty(T * k, d, dtype=torch.float32, device=DEV)
        self.ys = torch.empty(T, d, dtype=torch.float32, device=DEV) if cfg.n_shared else None
        self.y = torch.empty(T, d, dtype=act, device=DEV)
        self.stream = torch.cuda.current_stream()

    def step(self, ev=None):
        """route -> dispatch -> expert_ffn -> combine, events around the FFN."""
        s = self.stream
        moe.moe_route(self.shape, self.x, self.wr, self.br, self.logits, self.idx, self.w, stream=s)
        moe.moe_dispatch(self.shape, self.idx, self.counts, self.offsets, self.perm, self.inv, stream=s)
        if ev is not None:
            ev[0].record(s)
        moe.moe_expert_ffn(self.shape, self.x, self.wstruct, self.counts, self.offsets, self.perm,
                           self.yp, self.ys, self.ws, stream=s)
        if ev is not None:
            ev[1].record(s)
        moe.moe_combine(self.shape, self.yp, self.inv, self.w, self.ys, None, self.y, stream=s)

    def layer_call(self):
        moe.moe_layer_forward(self.shape, self.x, self.wr, self.br, self.wstruct, None, self.y,
                              self.counts, self.idx, self.ws, stream=self.stream)

    def time_layer(self, steps, warmup):
        """The timed region: `steps` back-to-back moe_layer_forward calls,
        bracketed by device synchronisation (host wall clock), with a HIP event
        recorded on the library's stream between consecutive calls for the
        per-step median and p99."""
        for _ in range(warmup):
            self.layer_call()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        for i in range(steps):
            evs[i].record(self.stream)
            self.layer_call()
        evs[steps].record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        return {"wall_s": wall, "ms_per_step": wall * 1e3 / steps, "median": float(np.median(per)),
                "p99": float(np.percentile(per, 99)), "mean": float(np.mean(per))}

    def time_ffn(self, steps, warmup):
        """The same layer as four calls with HIP events around moe_expert_ffn
        (the dominant step), after its own warm-up of the same length."""
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ffn = [a.elapsed_time(b) for a, b in evs]
        return {"four_call_ms_per_step": wall * 1e3 / steps, "mean": float(np.mean(ffn)),
                "median": float(np.median(ffn)), "p99": float(np.percentile(ffn, 99))}

    def ffn_algorithmic(self):
        """Experts hit, bytes and flops of one moe_expert_ffn call."""
        c = self.counts.cpu().numpy()
        U = int((c > 0).sum())
        return (U,) + ffn_work(self.cfg, U)


def ffn_work(cfg, U):
    """Algorithmic bytes and flops of one expert-FFN step with U experts hit:
    each hit expert's three matrices read once (batch union, plus the shared
    expert's), gathered x rows read, h written and read back, y_perm written."""
    tk = cfg.T * cfg.k
    if cfg.wt in ("int4", "int4g64"):
        mat = cfg.F * cfg.d // 2 + cfg.F * (cfg.d // (128 if cfg.wt == "int4" else 64)) * 2
    elif cfg.wt in ("mxfp4", "mxfp8"):
        mat = cfg.F * cfg.d // (2 if cfg.wt == "mxfp4" else 1) + cfg.F * (cfg.d // 32)
    else:
        mat = cfg.F * cfg.d * (4 if cfg.wt == "f32" else 2)
    ab = 4 if cfg.act == "f32" else 2
    w_bytes = (U + cfg.n_shared) * 3 * mat
    act_bytes = (tk * cfg.d * ab              # gathered x rows
                 + 2 * tk * cfg.F * ab         # h written then read
                 + tk * cfg.d * 4)             # y_perm written
    if cfg.n_shared:
        act_bytes += cfg.T * cfg.d * ab + 2 * cfg.T * cfg.F * ab + cfg.T * cfg.d * 4
    flops = 2 * 3 * (tk + cfg.n_shared * cfg.T) * cfg.d * cfg.F
    return w_bytes + act_bytes, flops


def _np_store(t):
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class OracleTimer:
    """The fp64 oracle (oracle/, test infrastructure) timed on the host's cores.
    It parallelises over the tokens of a call (one token per thread), so a
    call over n tokens keeps at most n threads busy: `cores` states the
    threads that actually worked."""

    def __init__(self, cfg, runner, Wd):
        import oracle
        oracle.build(force=False)
        self.oracle = oracle
        self.cfg = cfg
        self.threads = oracle.num_threads()
        self.W = {n: _np_store(Wd[n]) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")}
        self.S = None
        if cfg.n_shared:
            self.S = {"w_gate": _np_store(Wd["sh_gate"]), "w_up": _np_store(Wd["sh_up"]),
                      "w_down": _np_store(Wd["sh_down"]), "s_gate": _np_store(Wd["sh_s_gate"]),
                      "s_up": _np_store(Wd["sh_s_up"]), "s_down": _np_store(Wd["sh_s_down"])}
        self.set_tokens(cfg, runner)

    def set_tokens(self, cfg, runner):
        """Another workload on the same weights (the prefill batch)."""
        self.cfg = cfg
        self.x, self.wr, self.br = _np_store(runner.x), _np_store(runner.wr), _np_store(runner.br)

    def rate(self, order, chunk, target_s, threads, max_calls=50):
        """Tokens/s of oracle layer_forward calls over consecutive chunks of
        `order` (wrapping around) until target_s has elapsed."""
        cfg = self.cfg
        self.oracle.set_num_threads(threads)
        done, calls, i, t0 = 0, 0, 0, time.perf_counter()
        while True:
            sel = np.array([order[(i + j) % len(order)] for j in range(chunk)], np.int32)
            i += chunk
            self.oracle.layer_forward(self.x, cfg.act, cfg.wt, cfg.k, self.wr, self.br, self.W, self.S,
                                      sel=sel)
            done += chunk
            calls += 1
            el = time.perf_counter() - t0
            if el >= target_s or calls >= max_calls:
                break
        self.oracle.set_num_threads(self.threads)
        return done / el, done, calls, el

    def baseline(self, target_s=10.0, sample=False, single_thread_tokens=2):
        """All T tokens per call (sample=False), or a fixed seeded random order
        of the tokens in calls of one token per thread (sample=True), repeated
        until target_s; plus a one-thread run on a few tokens."""
        cfg = self.cfg
        if not sample:
            busy = min(self.threads, cfg.T)
            value, done, calls, el = self.rate(list(range(cfg.T)), cfg.T, target_s, busy)
            desc = (f"{cfg.name}: the full layer on all {cfg.T} tokens per call, fp64, {calls} calls "
                    f"({el:.1f} s)")
        else:
            busy = self.threads
            order = np.random.default_rng(0).permutation(cfg.T).tolist()
            value, done, calls, el = self.rate(order, busy, target_s, busy)
            which = (f"{done} of its {cfg.T} tokens" if done <= cfg.T else
                     f"{done} tokens (its {cfg.T}, then again from the start)")
            desc = (f"{cfg.name}: {which} in a fixed seeded random order, {busy} per call, the whole "
                    f"layer per token (router, top-{cfg.k}, SwiGLU experts, weighted sum), fp64 "
                    f"({el:.1f} s)")
        v1, d1, _, e1 = self.rate(list(range(cfg.T)), single_thread_tokens, 0.0, 1, max_calls=1)
        return {"value": round(value, 3), "unit": "tokens/s", "cores": busy, "kind": "oracle",
                "sample": desc, "threads_available": self.threads, "cpu_model": cpu_model(),
                "single_thread_value": round(v1, 3),
                "single_thread_sample": f"{d1} token{'s' if d1 > 1 else ''} on one thread ({e1:.1f} s)"}


# kernel sources of each workload's expert-FFN step: the committed counter
# summary is only valid for the sources it was taken on
TRAFFIC_SOURCES = {"mixtral_decode": ["ffn_gemv.hip", "ffn_skinny.hip", "common.h"], "fine_int4_decode": ["ffn_i4mfma.hip", "common.h"],
                   "fine_mxfp4_decode": ["ffn_i4mfma.hip", "common.h"], "mixtral_mxfp8_decode": ["ffn_i4mfma.hip", "common.h"]}

# the MX layers at decode: the first T tokens of the prefill workload's inputs,
# the same weights with their codes in the tiled layout
MX_DECODE = {"fine_mxfp4_decode": ("fine_mxfp4_prefill", 64), "mixtral_mxfp8_decode": ("mixtral_mxfp8_prefill", 8)}


def source_digest(key):
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[key]:
        h.update(open(os.path.join(ROOT, "moe_layer_forward_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch of the dominant step, from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known
    size).  None when the kernel source changed since the counters were taken."""
    import re
    if key not in TRAFFIC_SOURCES:
        return None
    path = os.path.join(ROOT, "profiles", f"{key}_ffn_traffic.md")
    try:
        text = open(path).read()
        digest = source_digest(key)
    except OSError:
        return None
    m = re.search(r"^%s: source=([0-9a-f]{16}) traffic_bytes=([0-9]+)" % re.escape(key), text, re.M)
    if not m or m.group(1) != digest:
        return None
    return int(m.group(2))


def read_ceiling_gbs(nbytes=4 << 30, reps=5):
    """Measured HBM read ceiling: the library's plain streaming-read kernel over
    a 4 GiB buffer (far beyond the caches), timed with HIP events."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for _ in range(2):
        moe.measure.moe_read_ceiling(buf, nbytes, sink)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        moe.measure.moe_read_ceiling(buf, nbytes, sink)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def mfma_ceiling(iters=40000, reps=3):
    """Measured matrix-core ceiling: the library's loop of independent bf16
    MFMAs on every CU, timed with HIP events; also the shader clock (GHz) that
    block 0 ran at, from its cycle and 100 MHz counters."""
    n_sink = 4096
    sink = torch.empty(n_sink, dtype=torch.float32, device=DEV)
    clk = torch.zeros(2, dtype=torch.int64, device=DEV)
    for _ in range(2):
        moe.measure.moe_mfma_ceiling(iters, sink, n_sink * 4)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        flops = moe.measure.moe_mfma_ceiling(iters, sink, n_sink * 4, clk)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    cyc, ticks = clk.cpu().tolist()
    return flops / (ms * 1e-3) / 1e12, cyc / (ticks / 100e6) / 1e9


def ffn_paths(cfg, counts, tau):
    """Which kernels the layer's FFN step runs, from the group sizes (the same
    rule the library applies on the device): bf16 groups above tau take the
    MFMA tiles; below it, when the largest group exceeds one GEMV pass, the
    skinny MFMA kernel (ceil(rows / 16) 16-token tiles, up to 64 rows) takes
    them all, else the GEMV."""
    if cfg.wt in ("int4", "mxfp4", "mxfp8"):
        # groups of at most dqt rows on the skinny kernel (matrix cores when d
        # and F are multiples of 1024, int4 also at most 8192; else the int4
        # GEMV), larger ones on the dequantising GEMM; dqt = 0 (every group on
        # the GEMM; int4: short last tiles on the skinny kernel) once the mean
        # group reaches 64 rows
        sk_mfma = cfg.d % 1024 == 0 and cfg.F % 1024 == 0 and (cfg.wt != "int4" or max(cfg.d, cfg.F) <= 8192)
        if cfg.wt != "int4" and not sk_mfma:
            return f"{cfg.wt} dequantising MFMA GEMM"
        skinny = f"{cfg.wt} skinny MFMA" if sk_mfma else "int4 GEMV"
        if tau < 0:
            return skinny
        dqt = tau if tau > 0 else (0 if cfg.T * cfg.k >= 64 * cfg.E else 32)
        c = [int(v) for v in counts if int(v) > 0]
        small = any(v <= dqt for v in c)
        big = any(v > dqt for v in c)
        gemm = f"{cfg.wt} dequantising MFMA GEMM" + (" (short last tiles on the skinny kernel)"
                                                    if dqt == 0 and sk_mfma and cfg.wt == "int4" else "")
        return " + ".join(([skinny] if small else []) + ([gemm] if big else []))
    if cfg.wt in ("int4g64",):
        return f"{cfg.wt} dequantising MFMA GEMM"
    if cfg.wt != "bf16" or tau < 0:
        return "GEMV"
    skinny = cfg.act == "bf16" and cfg.d % 64 == 0 and cfg.F % 64 == 0
    t = tau if tau > 0 else (64 if skinny and min(cfg.d, cfg.F) >= 4096 else 16)
    c = [int(v) for v in counts if v > 0]
    small = [v for v in c if v <= t]
    parts = []
    for name, K in (("gate/up", cfg.d), ("down", cfg.F)):
        npass = 8 if K <= 8192 else (2 if name == "gate/up" else 4)   # GEMV tokens per pass
        p = []
        if small:
            m = max(small)
            if skinny and t <= 64 and m > npass:
                tt = (m + 15) // 16
                p.append("skinny MFMA, %d token tile%s" % (tt, "" if tt == 1 else "s"))
            else:
                p.append("GEMV")
        if any(v > t for v in c):
            p.append("MFMA tiles")
        parts.append(f"{name}: " + " + ".join(p))
    return "; ".join(parts)


def roofline_obj(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def workload_leg(run, steps, warmup, tau, ceilings, traffic_key=None, layer_first=True):
    """Time one workload: the layer loop (the timed region) and the four-call
    loop that times the expert-FFN step, each after its own warm-up; the
    roofline object of that step (MFMA-bound when the groups are prefill
    sized, else HBM-bound)."""
    lay = run.time_layer(steps, warmup)
    ffn = run.time_ffn(steps, warmup)
    cfg = run.cfg
    U, nbytes, flops = run.ffn_algorithmic()
    common = dict(launch_ms=round(ffn["mean"], 5), launch_ms_median=round(ffn["median"], 5),
                  launch_ms_p99=round(ffn["p99"], 5),
                  ffn_within_layer=bool(ffn["median"] <= lay["median"]))
    if cfg.T * cfg.k / max(U, 1) > 64:      # prefill-sized groups: MFMA-bound
        tf = flops / (ffn["mean"] * 1e-3) / 1e12
        mceil, mclk = ceilings("mfma")
        roof = dict(roofline_obj("mfma", tf, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"),
                    kernel=f"expert FFN step ({ffn_paths(cfg, run.counts.cpu().tolist(), tau)})",
                    flops_per_launch=flops, **common,
                    measured_mfma_ceiling=round(mceil, 1), mfma_ceiling_clock_ghz=round(mclk, 3),
                    frac_of_measured_ceiling=round(tf / mceil, 4))
    else:
        gbs = nbytes / (ffn["mean"] * 1e-3) / 1e9
        ceil = ceilings("hbm")
        roof = dict(roofline_obj("hbm", gbs, HBM_PEAK_GBS, "GB/s",
                                 measured_traffic(traffic_key) if traffic_key else None),
                    kernel=f"expert FFN step ({ffn_paths(cfg, run.counts.cpu().tolist(), tau)}; "
                           f"weights {run.wt})",
                    bytes_per_launch=nbytes, **common,
                    measured_read_ceiling=round(ceil, 1),
                    frac_of_measured_ceiling=round(gbs / ceil, 4))
    if not common["ffn_within_layer"]:
        log(f"warning: {cfg.name}: expert-FFN step median {ffn['median']:.4f} ms exceeds the layer's "
            f"{lay['median']:.4f} ms")
    return {"layer": lay, "ffn": ffn, "U": U, "roofline": roof}


def leg_summary(cfg, leg, steps, warmup):
    lay = leg["layer"]
    return {"workload": cfg.name, "T": cfg.T, "value": round(cfg.T / (lay["ms_per_step"] * 1e-3), 1),
            "unit": "tokens/s", "ms_per_step": round(lay["ms_per_step"], 5),
            "ms_per_step_median": round(lay["median"], 5), "ms_per_step_p99": round(lay["p99"], 5),
            "steps": steps, "warmup": warmup, "active_experts": leg["U"],
            "roofline": leg["roofline"],
            "four_call_ms_per_step": round(leg["ffn"]["four_call_ms_per_step"], 5)}


class Ceilings:
    """Measured ceilings, taken once per process on first use."""

    def __init__(self):
        self.v = {}

    def __call__(self, kind):
        if kind not in self.v:
            self.v[kind] = read_ceiling_gbs() if kind == "hbm" else mfma_ceiling()
        return self.v[kind]


def stack_oracle_baseline(cfg, inp, hs, nrms, target_s=10.0):
    """The oracle (oracle/, test infrastructure) through the stack's layers on a
    fixed seeded random order of its tokens, one token per thread per call:
    per layer the RMSNorm and the layer (router, top-k, SwiGLU experts,
    weighted sum, residual), each layer on the GPU's own input to it (the
    norm's input h_l and the normed rows of the last timed step), so the calls
    need no GPU-side state.  Plus one token through the layers on one thread."""
    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads()
    H = [_np_store(h) for h in hs[:cfg.layers]]
    N = [_np_store(n) for n in nrms]
    Ls = []
    for l in range(cfg.layers):
        L = inp["layers"][l]
        Ls.append(({n: _np_store(L[n]) for n in ("w_gate", "w_up", "w_down")} | {"s_gate": None, "s_up": None,
                                                                              "s_down": None},
                   _np_store(L["w_router"]), inp["gamma"][l].numpy().astype(np.float32)))

    def run(sel):
        for l, (W, wr, g) in enumerate(Ls):
            oracle.rmsnorm(H[l][sel], cfg.act, g, inp["eps"])
            oracle.layer_forward(N[l], cfg.act, cfg.wt, cfg.k, wr, None, W, None, residual=H[l], sel=sel)

    order = np.random.default_rng(0).permutation(cfg.T).astype(np.int32)
    oracle.set_num_threads(threads)
    done, calls, i, t0 = 0, 0, 0, time.perf_counter()
    while True:
        sel = np.array([order[(i + j) % cfg.T] for j in range(threads)], np.int32)
        i += threads
        run(sel)
        done += threads
        calls += 1
        el = time.perf_counter() - t0
        if el >= target_s or calls >= 50:
            break
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    run(order[:1].copy())
    e1 = time.perf_counter() - t1
    oracle.set_num_threads(threads)
    return {"value": round(done / el, 3), "unit": "tokens/s through the 4-layer stack", "cores": threads,
            "kind": "oracle",
            "sample": (f"stack4: {done} of its {cfg.T} tokens (a fixed seeded random order, {threads} per call) "
                       f"through {cfg.layers} layers (RMSNorm, then router, top-{cfg.k}, SwiGLU experts, "
                       f"weighted sum and residual), each layer on the GPU's input to it, fp64 ({el:.1f} s)"),
            "threads_available": threads, "cpu_model": cpu_model(),
            "single_thread_value": round(1.0 / e1, 3),
            "single_thread_sample": f"1 token through {cfg.layers} layers on one thread ({e1:.1f} s)"}


def stack_leg(steps, warmup, cpu=False):
    """The 4-layer pre-norm stack (T=512, d=2048, E=64, top-6, F=1408, bf16):
    per layer h_{l+1} = h_l + MoE_l(rmsnorm(h_l)), as moe_rmsnorm then
    moe_layer_forward with the residual.  Times the whole stack (a step is the
    4 layers) with a HIP event between layers, and returns the per-layer usage
    histogram (layer, expert, count) of the last step; with cpu, the oracle
    timed beside it on the host."""
    cfg = moe_inputs.CONFIGS["stack4"]
    log("generating the 4-layer stack on the GPU")
    inp = moe_inputs.generate(cfg, seed=0, device=DEV)
    layers = []
    for l in range(cfg.layers):
        L = inp["layers"][l]
        W = {n: (None if L.get(n) is None else L[n].to(DEV)) for n in ("w_gate", "w_up", "w_down")}
        layers.append(moe.layer.MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.act, cfg.wt, W,
                                         L["w_router"].to(DEV), None))
    gammas = [g.to(DEV) for g in inp["gamma"]]
    hs = [inp["x"].to(DEV)] + [torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device=DEV)
                               for _ in range(cfg.layers)]
    nrm = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device=DEV)
    st = torch.cuda.current_stream()
    nshape = moe.make_shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.act, cfg.wt)

    def one(evs=None):
        for l, lay in enumerate(layers):
            if evs is not None:
                evs[l].record(st)
            moe.moe_rmsnorm(nshape, hs[l], gammas[l], inp["eps"], nrm, stream=st)
            lay.forward(nrm, residual=hs[l], out=hs[l + 1], stream=st)
        if evs is not None:
            evs[cfg.layers].record(st)

    # one-layer-ahead expert prediction (outside the timed loop): layer l+1's
    # router on layer l's normed input, scored against layer l+1's choice
    wrs = [inp["layers"][l]["w_router"].to(DEV) for l in range(cfg.layers)]
    pilot = []
    one()
    for l in range(cfg.layers - 1):
        moe.moe_rmsnorm(nshape, hs[l], gammas[l], inp["eps"], nrm, stream=st)
        lg = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=DEV)
        pred = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=DEV)
        pw = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=DEV)
        moe.moe_route(nshape, nrm, wrs[l + 1], None, lg, pred, pw, stream=st)
        ov = torch.empty(cfg.k + 1, dtype=torch.int32, device=DEV)
        moe.moe_topk_overlap(nshape, pred, layers[l + 1].topk_idx, ov, stream=st)
        h = ov.cpu().numpy()
        pilot.append({"from_layer": l, "to_layer": l + 1, "tokens_by_shared_experts": h.tolist(),
                      "hit_rate": round(float((np.arange(cfg.k + 1) * h).sum()) / (cfg.T * cfg.k), 4)})

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(cfg.layers + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        one(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_layer = np.array([[e[l].elapsed_time(e[l + 1]) for l in range(cfg.layers)] for e in ev])
    stack = per_layer.sum(axis=1)
    counts = [lay.counts.cpu().tolist() for lay in layers]
    lines = [(l, e, c) for l, cs in enumerate(counts) for e, c in enumerate(cs) if c > 0]
    for l, e, c in lines:
        log(f"usage {l} {e} {c}")
    med = np.median(per_layer, axis=0)
    layer_objs = []
    for l in range(cfg.layers):
        U = sum(1 for c in counts[l] if c > 0)
        nbytes, _ = ffn_work(cfg, U)
        gbs = nbytes / (med[l] * 1e-3) / 1e9
        layer_objs.append({"layer": l, "ms_median": round(float(med[l]), 5),
                           "ms_p99": round(float(np.percentile(per_layer[:, l], 99)), 5),
                           "tokens_per_s": round(cfg.T / (med[l] * 1e-3), 1), "active_experts": U,
                           "expert_ffn_bytes": nbytes, "GBps_over_layer": round(gbs, 1),
                           "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4)})
    ms = wall * 1e3 / steps
    cpu_obj = None
    if cpu:
        log("cpu baseline: oracle through the stack's layers")
        nrms = []
        for l in range(cfg.layers):
            n_l = torch.empty_like(nrm)
            moe.moe_rmsnorm(nshape, hs[l], gammas[l], inp["eps"], n_l, stream=st)
            nrms.append(n_l)
        torch.cuda.synchronize()
        cpu_obj = stack_oracle_baseline(cfg, inp, hs, nrms)
    out = {"workload": "stack4", "T": cfg.T, "layers": cfg.layers,
            "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s through the 4-layer stack",
            "ms_per_step": round(ms, 5), "ms_per_step_median": round(float(np.median(stack)), 5),
            "ms_per_step_p99": round(float(np.percentile(stack, 99)), 5), "steps": steps, "warmup": warmup,
            "per_layer": layer_objs, "usage_histogram": counts, "usage_lines": len(lines),
            "next_layer_prediction": pilot}
    if cpu_obj is not None:
        out["cpu_baseline"] = cpu_obj
    return out


def low_latency_leg(dcfg, wr, W, orc=None, steps=200, warmup=20):
    """Small decode batches of the Mixtral-shaped layer (T = 1, 2, 4, 8): the
    layer as eager moe_layer_forward calls and as one HIP graph replayed
    (captured once, so a step pays no per-kernel launch from the host);
    microseconds per layer, median and p99 over `steps` events; next to it the
    oracle's time for the same call on the host."""
    out = []
    for T in (1, 2, 4, 8):
        cfg = dcfg.replace(name=f"mixtral_decode_t{T}", T=T)
        x = moe_inputs.activations(cfg, 0).to(DEV)
        run = Runner(cfg, x, wr, None, W)
        eager = run.time_layer(steps, warmup)
        # capture one layer call on a side stream, then replay it
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                moe.moe_layer_forward(run.shape, run.x, run.wr, run.br, run.wstruct, None, run.y, run.counts,
                                      run.idx, run.ws, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            moe.moe_layer_forward(run.shape, run.x, run.wr, run.br, run.wstruct, None, run.y, run.counts,
                                  run.idx, run.ws, stream=torch.cuda.current_stream())
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        cur = torch.cuda.current_stream()
        for i in range(steps):
            ev[i].record(cur)
            g.replay()
        ev[steps].record(cur)
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]) * 1e3
        row = {"T": T, "active_experts": int((run.counts > 0).sum()),
               "graph_us_median": round(float(np.median(per)), 2),
               "graph_us_p99": round(float(np.percentile(per, 99)), 2),
               "eager_us_median": round(eager["median"] * 1e3, 2),
               "eager_us_p99": round(eager["p99"] * 1e3, 2),
               "graph_tokens_per_s": round(T / (np.median(per) * 1e-6), 1)}
        if orc is not None:
            orc.set_tokens(cfg, run)
            v, done, calls, el = orc.rate(list(range(T)), T, 0.0, min(orc.threads, T), max_calls=1)
            row["oracle_ms_per_call"] = round(el * 1e3, 1)
            row["oracle_threads"] = min(orc.threads, T)
        out.append(row)
        log(json.dumps(row))
        del g, run
    return out


def extras():
    """Decode-side sweeps printed as JSON lines (not the bench line): the GEMV /
    MFMA crossover that sets tau (one expert holding c rows, Mixtral weights,
    top-1 with the router biased onto expert 0), and the Mixtral layer at
    decode batch sizes T = 8 ... 64."""
    dcfg = moe_inputs.CONFIGS["mixtral_decode"]
    _, wr, _, W = device_layer(dcfg)
    bias = torch.zeros(dcfg.E, dtype=torch.float32, device=DEV)
    bias[0] = 1000.0
    wbytes = 3 * dcfg.d * dcfg.F * 2
    for c in (1, 2, 4, 8, 12, 16, 20, 24, 32, 48, 64):
        cfg = dcfg.replace(name=f"tau_sweep_c{c}", T=c, k=1)
        x = moe_inputs.activations(cfg, 0).to(DEV)
        for tau, path in ((-1, "gemv"), (1, "mfma")):
            if tau == 1 and c < 2:
                continue
            run = Runner(cfg, x, wr, bias, W, tau=tau)
            ffn = run.time_ffn(20, 5)
            assert int(run.counts[0]) == c
            print(json.dumps({"sweep": "tau", "rows": c, "path": path, "ffn_ms": round(ffn["mean"], 4),
                              "ffn_ms_median": round(ffn["median"], 4),
                              "weight_GBps": round(wbytes / (ffn["mean"] * 1e-3) / 1e9, 1)}), flush=True)
            del run
    for T in (8, 16, 32, 64):
        cfg = dcfg.replace(name=f"mixtral_decode_t{T}", T=T)
        x = moe_inputs.activations(cfg, 0).to(DEV)
        run = Runner(cfg, x, wr, None, W)
        lay = run.time_layer(20, 5)
        ffn = run.time_ffn(20, 5)
        U, nbytes, _ = run.ffn_algorithmic()
        print(json.dumps({"sweep": "decode_T", "T": T, "active_experts": U,
                          "ms_per_step": round(lay["ms_per_step"], 4),
                          "tokens_per_s": round(T / (lay["ms_per_step"] * 1e-3), 1),
                          "ffn_ms": round(ffn["mean"], 4),
                          "ffn_GBps": round(nbytes / (ffn["mean"] * 1e-3) / 1e9, 1),
                          "frac_of_8TBps": round(nbytes / (ffn["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}),
              flush=True)
        del run


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixtral_decode",
                    choices=["mixtral_decode", "mixtral_prefill", "fine_int4_decode",
                             "stack4_layer0", "stack4", "fine_int4_prefill", "fine_mxfp4_prefill",
                             "mixtral_mxfp8_prefill", "fine_mxfp4_decode", "mixtral_mxfp8_decode"])
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the int4 decode and 4-layer stack legs of the default run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tau", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload with this many tokens instead of its own T "
                         "(the config is named <workload>_t<tokens>)")
    ap.add_argument("--int4-layout", choices=["tiled", "row-major"], default="tiled",
                    help="code layout the layer streams (tiled: packed once with "
                         "moe_pack_int4_tiled / moe_pack_mxfp8_tiled before timing; needs d, F "
                         "multiples of 1024; int4 up to 8192, MXFP4 and MXFP8 at decode-sized groups)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--extras", action="store_true",
                    help="print the decode sweeps (tau crossover, decode batch sizes) instead of the bench line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the layer is built "
              "and measured on a single MI355X (expert-parallel sharding over several GPUs is designed "
              "but not built)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    moe.lib()   # fail loudly if the HIP library is not built
    if args.extras:
        extras()
        return
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=DEV).fill_(1.0)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ceilings = Ceilings()
    steps, warmup = args.steps, args.warmup

    if args.workload == "stack4":
        out = stack_leg(steps, warmup, cpu=not args.no_cpu_baseline)
        print(json.dumps(out), flush=True)
        return

    name = "stack4" if args.workload == "stack4_layer0" else MX_DECODE.get(args.workload, (args.workload,))[0]
    cfg = moe_inputs.CONFIGS[name]
    if cfg.layers > 1:
        cfg = cfg.replace(layers=1, name="stack4_layer0")
    if args.tokens > 0 and args.workload not in MX_DECODE:
        cfg = cfg.replace(name=f"{cfg.name}_t{args.tokens}", T=args.tokens)
    log(f"generating {cfg.name} inputs on the GPU")
    x, wr, br, W = device_layer(cfg)
    if args.workload in MX_DECODE:
        # the default run's MX decode leg: the prefill inputs' first T tokens
        cfg = cfg.replace(name=args.workload, T=MX_DECODE[args.workload][1])
        x = x[:cfg.T].contiguous()
    wt = cfg.wt
    Wrun = W
    if cfg.wt == "int4" and args.int4_layout == "tiled" and cfg.d % 1024 == 0 and cfg.F % 1024 == 0 \
            and max(cfg.d, cfg.F) <= 8192:
        # weight preparation, once and outside the timed region (weights are static)
        log("packing int4 codes into the tiled layout")
        Wrun = moe.layer.pack_int4_tiled(W)
        torch.cuda.synchronize()
        wt = "int4_tiled"
    elif cfg.wt in ("mxfp4", "mxfp8") and args.int4_layout == "tiled" and cfg.d % 1024 == 0 \
            and cfg.F % 1024 == 0 and cfg.T * cfg.k < 64 * cfg.E:
        # decode-sized groups: every group runs the skinny kernel, which reads
        # the tiled layout (prefill-sized groups keep row-major codes for the
        # dequantising GEMM)
        log(f"packing {cfg.wt.upper()} codes into the tiled layout")
        Wrun = moe.layer.pack_int4_tiled(W) if cfg.wt == "mxfp4" else moe.layer.pack_mxfp8_tiled(W)
        torch.cuda.synchronize()
        wt = f"{cfg.wt}_tiled"
    run = Runner(cfg, x, wr, br, Wrun, tau=args.tau, wt=wt)
    if cfg.name == "mixtral_prefill":   # the prefill protocol, whatever the flags
        steps, warmup = max(steps, 50), max(warmup, 20)
    log(f"timing {cfg.name}: warmup {warmup}, steps {steps}")
    key = cfg.name if args.tau == 0 and (cfg.wt != "int4" or wt == "int4_tiled") else None
    leg = workload_leg(run, steps, warmup, args.tau, ceilings, key)
    lay = leg["layer"]
    out = {
        "metric": METRIC, "value": round(cfg.T / (lay["ms_per_step"] * 1e-3), 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(lay["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" and cfg.wt == "bf16" else
                 ("f32" if cfg.wt == "f32" else f"bf16/{cfg.wt}"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
                   "F": cfg.F, "weights": wt, "shared_experts": cfg.n_shared,
                   "active_experts": leg["U"], "tau": args.tau, "seed": 0},
        "ms_per_step_median": round(lay["median"], 5), "ms_per_step_p99": round(lay["p99"], 5),
        "roofline": leg["roofline"],
        "four_call_ms_per_step": round(leg["ffn"]["four_call_ms_per_step"], 5),
    }
    log(json.dumps(out))
    orc = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the host")
        orc = OracleTimer(cfg, run, W)
        out["cpu_baseline"] = orc.baseline(sample=cfg.T > 64)

    if not args.no_prefill and cfg.name == "mixtral_decode":
        pcfg = moe_inputs.CONFIGS["mixtral_prefill"]
        log("prefill T=4096 on the same weights")
        px, pwr, pbr, _ = device_layer(pcfg, shared_weights=W)
        prun = Runner(pcfg, px, pwr, pbr, W, tau=args.tau)
        psteps, pwarm = max(50, steps), max(20, warmup)
        pleg = workload_leg(prun, psteps, pwarm, args.tau, ceilings)
        out["prefill"] = dict(leg_summary(pcfg, pleg, psteps, pwarm), counts=prun.counts.cpu().tolist())
        log(json.dumps(out["prefill"]))
        if orc is not None:
            log("cpu baseline: oracle on a sample of the prefill tokens")
            orc.set_tokens(pcfg, prun)
            out["prefill"]["cpu_baseline"] = orc.baseline(sample=True)
        del prun, px

    if not args.no_legs and cfg.name == "mixtral_decode":
        log("low-latency decode: T = 1, 2, 4, 8, eager and graph-replayed")
        out["low_latency_decode"] = low_latency_leg(cfg, wr, W, orc)
    del orc

    if not args.no_legs and cfg.name == "mixtral_decode":
        icfg = moe_inputs.CONFIGS["fine_int4_decode"]
        log("int4 decode leg (tiled codes)")
        ix, iwr, ibr, iW = device_layer(icfg)
        iWt = moe.layer.pack_int4_tiled(iW)
        torch.cuda.synchronize()
        irun = Runner(icfg, ix, iwr, ibr, iWt, tau=args.tau, wt="int4_tiled")
        ileg = workload_leg(irun, steps, warmup, args.tau, ceilings, icfg.name if args.tau == 0 else None)
        out["int4_decode"] = leg_summary(icfg, ileg, steps, warmup)
        if not args.no_cpu_baseline:
            log("cpu baseline: oracle on the int4 decode layer (row-major codes)")
            iorc = OracleTimer(icfg, irun, iW)
            out["int4_decode"]["cpu_baseline"] = iorc.baseline(sample=True, single_thread_tokens=1)
            del iorc
        log(json.dumps(out["int4_decode"]))
        del irun, iWt
        torch.cuda.empty_cache()
        # the same int4 layer at prefill (row-major codes: the dequantising
        # grouped GEMM), then MXFP4 experts of that shape and MXFP8 experts of
        # the Mixtral shape
        psteps, pwarm = max(50, steps), max(20, warmup)
        # and the MX layers at decode (the skinny matrix-core kernel), on the
        # same weights: the fine-grained MXFP4 layer at T = 64, the
        # Mixtral-shaped MXFP8 layer at T = 8
        for name, Wq, dec in (("fine_int4_prefill", iW, None),
                              ("fine_mxfp4_prefill", None, ("fine_mxfp4_decode", MX_DECODE["fine_mxfp4_decode"][1])),
                              ("mixtral_mxfp8_prefill", None, ("mixtral_mxfp8_decode", MX_DECODE["mixtral_mxfp8_decode"][1]))):
            qcfg = moe_inputs.CONFIGS[name]
            log(f"{name}: quantised experts at prefill")
            qx, qwr, qbr, qW = device_layer(qcfg, shared_weights=Wq)
            qrun = Runner(qcfg, qx, qwr, qbr, qW, tau=args.tau)
            qleg = workload_leg(qrun, psteps, pwarm, args.tau, ceilings)
            out[name] = leg_summary(qcfg, qleg, psteps, pwarm)
            log(json.dumps(out[name]))
            del qrun
            if dec is not None:
                dname, dT = dec
                dcfg = qcfg.replace(name=dname, T=dT)
                log(f"{dname}: the same experts at decode, T={dT}")
                dW, dwt = qW, None
                if qcfg.wt in ("mxfp4", "mxfp8"):
                    # MX codes packed once into the tiled layout the skinny kernel streams
                    pack = moe.layer.pack_int4_tiled if qcfg.wt == "mxfp4" else moe.layer.pack_mxfp8_tiled
                    dW, dwt = pack(qW), f"{qcfg.wt}_tiled"
                    torch.cuda.synchronize()
                drun = Runner(dcfg, qx[:dT].contiguous(), qwr, qbr, dW, tau=args.tau, wt=dwt)
                dleg = workload_leg(drun, steps, warmup, args.tau, ceilings, dname if args.tau == 0 else None)
                out[dname] = leg_summary(dcfg, dleg, steps, warmup)
                log(json.dumps(out[dname]))
                del drun, dW
            del qW, qx
            torch.cuda.empty_cache()
        del iW
        out["stack4"] = stack_leg(steps, warmup, cpu=not args.no_cpu_baseline)
        log(json.dumps(out["stack4"]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
