"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole layer (router, softmax, top-k, dispatch,
expert SwiGLU FFN, combine) over one batch: one moe_layer_forward call through
the C ABI.  A second timed loop of the same length calls the four steps one
by one (route -> dispatch -> expert_ffn -> combine on one stream, the same
kernels) with HIP events around the expert FFN.  Inputs and weights are resident in HBM before the
timed region.  The headline is the Mixtral-8x7B-shaped decode layer (T=8); the
prefill layer (T=4096, Zipf-loaded experts) runs on the same weights and is
reported in the same JSON line.

Roofline: the dominant step is the expert FFN (the GEMV or skinny MFMA gate/up
and down kernels at decode, the MFMA gate/up and down kernels at prefill; the
bench line names the kernels the group sizes select).  Its time is
measured live with HIP events recorded on the library's stream around the
moe_expert_ffn call; its algorithmic bytes are the weight bytes of the experts
actually hit (batch union) plus the activation traffic, its algorithmic flops
2*3*T*k*d*F.

CPU baseline: the fp64 oracle (oracle/, test infrastructure) timed on the
host's cores on the full decode layer, repeated to ~10 s.
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

    def timed(self, steps, warmup):
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
        ffn_ms = [a.elapsed_time(b) for a, b in evs]
        self.last_ffn_p99 = float(np.percentile(ffn_ms, 99))
        # the single-call path, timed the same way (same kernels)
        t1 = time.perf_counter()
        for _ in range(steps):
            self.layer_call()
        torch.cuda.synchronize()
        wall_layer = time.perf_counter() - t1
        return wall, float(np.mean(ffn_ms)), float(np.median(ffn_ms)), wall_layer

    def ffn_algorithmic(self):
        """Bytes and flops of one moe_expert_ffn call (batch union of weights)."""
        cfg = self.cfg
        c = self.counts.cpu().numpy()
        U = int((c > 0).sum())
        tk = cfg.T * cfg.k
        if cfg.wt == "int4":
            mat = cfg.F * cfg.d // 2 + cfg.F * (cfg.d // 128) * 2
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
        return U, w_bytes + act_bytes, flops


def cpu_baseline(cfg, runner, Wd, target_s=10.0):
    """The oracle timed on the host's cores on the full layer (all T tokens);
    Wd: the device weights in the row-major layout the oracle reads."""
    import oracle
    oracle.build(force=False)

    def st(t):
        if t is None:
            return None
        t = t.detach().cpu().contiguous()
        if t.dtype in (torch.bfloat16, torch.float16):
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    W = {n: st(Wd[n]) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")}
    S = None
    if cfg.n_shared:
        S = {"w_gate": st(Wd["sh_gate"]), "w_up": st(Wd["sh_up"]),
             "w_down": st(Wd["sh_down"]), "s_gate": st(Wd["sh_s_gate"]),
             "s_up": st(Wd["sh_s_up"]), "s_down": st(Wd["sh_s_down"])}
    x, wr, br = st(runner.x), st(runner.wr), st(runner.br)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.layer_forward(x, cfg.act, cfg.wt, cfg.k, wr, br, W, S)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 50:
            break
    return {"value": reps * cfg.T / el, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{cfg.name}: full layer, all {cfg.T} tokens, fp64, repeated {reps}x "
                      f"({el:.1f} s)"}


# kernel sources of each workload's expert-FFN step: the committed counter
# summary is only valid for the sources it was taken on
TRAFFIC_SOURCES = {"mixtral_decode": ["ffn_gemv.hip", "ffn_skinny.hip", "common.h"], "fine_int4_decode": ["ffn_i4mfma.hip", "common.h"]}


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
        moe.moe_read_ceiling(buf, nbytes, sink)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        moe.moe_read_ceiling(buf, nbytes, sink)
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
        moe.moe_mfma_ceiling(iters, sink, n_sink * 4)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        flops = moe.moe_mfma_ceiling(iters, sink, n_sink * 4, clk)
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
    if cfg.wt == "int4":
        return "int4 skinny MFMA" if cfg.d % 1024 == 0 and cfg.F % 1024 == 0 else "int4 GEMV"
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
            _, ffn_mean, ffn_med, _ = run.timed(20, 5)
            assert int(run.counts[0]) == c
            print(json.dumps({"sweep": "tau", "rows": c, "path": path, "ffn_ms": round(ffn_mean, 4),
                              "ffn_ms_median": round(ffn_med, 4),
                              "weight_GBps": round(wbytes / (ffn_mean * 1e-3) / 1e9, 1)}), flush=True)
            del run
    for T in (8, 16, 32, 64):
        cfg = dcfg.replace(name=f"mixtral_decode_t{T}", T=T)
        x = moe_inputs.activations(cfg, 0).to(DEV)
        run = Runner(cfg, x, wr, None, W)
        wall, ffn_mean, _, _ = run.timed(20, 5)
        U, nbytes, _ = run.ffn_algorithmic()
        print(json.dumps({"sweep": "decode_T", "T": T, "active_experts": U,
                          "ms_per_step": round(wall * 1e3 / 20, 4), "tokens_per_s": round(T * 20 / wall, 1),
                          "ffn_ms": round(ffn_mean, 4),
                          "ffn_GBps": round(nbytes / (ffn_mean * 1e-3) / 1e9, 1),
                          "frac_of_8TBps": round(nbytes / (ffn_mean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
        del run


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_decode",
                    choices=["mixtral_decode", "mixtral_prefill", "fine_int4_decode",
                             "stack4_layer0"])
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tau", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload with this many tokens instead of its own T "
                         "(the config is named <workload>_t<tokens>)")
    ap.add_argument("--int4-layout", choices=["tiled", "row-major"], default="tiled",
                    help="int4 code layout the layer streams (tiled: packed once with "
                         "moe_pack_int4_tiled before timing; needs d, F multiples of 1024)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--extras", action="store_true",
                    help="print the decode sweeps (tau crossover, decode batch sizes) instead of the bench line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built for a single MI355X; see the sharding notes in DESIGN.md)",
              file=sys.stderr)
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

    name = "stack4" if args.workload == "stack4_layer0" else args.workload
    cfg = moe_inputs.CONFIGS[name]
    if cfg.layers > 1:
        cfg = cfg.replace(layers=1)
    if args.tokens > 0:
        cfg = cfg.replace(name=f"{cfg.name}_t{args.tokens}", T=args.tokens)
    log(f"generating {cfg.name} inputs on the GPU")
    x, wr, br, W = device_layer(cfg)
    wt = cfg.wt
    Wrun = W
    if cfg.wt == "int4" and args.int4_layout == "tiled" and cfg.d % 1024 == 0 and cfg.F % 1024 == 0 \
            and max(cfg.d, cfg.F) <= 8192:
        # weight preparation, once and outside the timed region (weights are static)
        log("packing int4 codes into the tiled layout")
        Wrun = moe.layer.pack_int4_tiled(W)
        torch.cuda.synchronize()
        wt = "int4_tiled"
    run = Runner(cfg, x, wr, br, Wrun, tau=args.tau, wt=wt)
    log(f"timing {cfg.name}: warmup {args.warmup}, steps {args.steps}")
    wall, ffn_mean, ffn_med, wall_layer = run.timed(args.steps, args.warmup)
    U, ffn_bytes, ffn_flops = run.ffn_algorithmic()
    ms = wall_layer * 1e3 / args.steps
    value = cfg.T * args.steps / wall_layer
    achieved = ffn_bytes / (ffn_mean * 1e-3) / 1e9
    if cfg.T * cfg.k / max(U, 1) > 64:      # prefill-sized groups: MFMA-bound
        tf = ffn_flops / (ffn_mean * 1e-3) / 1e12
        mceil, mclk = mfma_ceiling()
        roof = dict(roofline_obj("mfma", tf, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"),
                    kernel="expert FFN step (MFMA gate/up + down)", flops_per_launch=ffn_flops,
                    launch_ms=round(ffn_mean, 5), launch_ms_median=round(ffn_med, 5),
                    launch_ms_p99=round(run.last_ffn_p99, 5),
                    measured_mfma_ceiling=round(mceil, 1), mfma_ceiling_clock_ghz=round(mclk, 3),
                    frac_of_measured_ceiling=round(tf / mceil, 4))
    else:
        ceil = read_ceiling_gbs()
        roof = dict(roofline_obj("hbm", achieved, HBM_PEAK_GBS, "GB/s",
                                 # counters were taken on the default run (tiled int4 codes)
                                 measured_traffic(cfg.name)
                                 if args.tau == 0 and (cfg.wt != "int4" or wt == "int4_tiled") else None),
                    kernel=f"expert FFN step ({ffn_paths(cfg, run.counts.cpu().tolist(), args.tau)}; weights {wt})",
                    bytes_per_launch=ffn_bytes,
                    launch_ms=round(ffn_mean, 5), launch_ms_median=round(ffn_med, 5),
                    launch_ms_p99=round(run.last_ffn_p99, 5),
                    measured_read_ceiling=round(ceil, 1),
                    frac_of_measured_ceiling=round(achieved / ceil, 4))
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" and cfg.wt == "bf16" else
                 ("bf16/int4" if cfg.wt == "int4" else "f32"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
                   "F": cfg.F, "weights": wt, "shared_experts": cfg.n_shared,
                   "active_experts": U, "tau": args.tau, "seed": 0},
        "roofline": roof,
        "four_call_ms_per_step": round(wall * 1e3 / args.steps, 4),
    }
    log(json.dumps(out))

    if not args.no_prefill and cfg.name == "mixtral_decode":
        pcfg = moe_inputs.CONFIGS["mixtral_prefill"]
        log("prefill T=4096 on the same weights")
        px, pwr, pbr, _ = device_layer(pcfg, shared_weights=W)
        prun = Runner(pcfg, px, pwr, pbr, W, tau=args.tau)
        psteps = max(5, args.steps // 5)
        pwall, pffn_mean, pffn_med, pwall_layer = prun.timed(psteps, max(2, args.warmup // 2))
        _, pbytes, pflops = prun.ffn_algorithmic()
        ptf = pflops / (pffn_mean * 1e-3) / 1e12
        mceil, mclk = mfma_ceiling()
        out["prefill"] = {
            "workload": pcfg.name, "T": pcfg.T, "value": round(pcfg.T * psteps / pwall_layer, 1),
            "unit": "tokens/s", "ms_per_step": round(pwall_layer * 1e3 / psteps, 4), "steps": psteps,
            "counts": prun.counts.cpu().tolist(),
            "roofline": dict(roofline_obj("mfma", ptf, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"),
                             kernel="expert FFN step (MFMA gate/up + down)",
                             flops_per_launch=pflops, launch_ms=round(pffn_mean, 4),
                             launch_ms_median=round(pffn_med, 4),
                             launch_ms_p99=round(prun.last_ffn_p99, 4),
                             measured_mfma_ceiling=round(mceil, 1),
                             mfma_ceiling_clock_ghz=round(mclk, 3),
                             frac_of_measured_ceiling=round(ptf / mceil, 4)),
            "four_call_ms_per_step": round(pwall * 1e3 / psteps, 4),
        }
        log(json.dumps(out["prefill"]))
        del prun, px

    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the host")
        out["cpu_baseline"] = cpu_baseline(cfg, run, W)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
