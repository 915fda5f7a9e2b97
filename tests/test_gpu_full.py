"""GPU parity at the workloads' full sizes, in the launch configuration the bench
times (moe_layer_forward, default tau).  Routing is checked on every token
(bit-exact indices on the GPU's own logits, flip rule against the oracle's fp64
logits); outputs are checked on tokens the oracle computes one by one."""
import numpy as np
import pytest
import torch

import moe_inputs
import moe_layer_forward_amd as moe
from gpu_common import (DEV, TOL, check_routing_with_flips, device_inputs, oracle_weights, run_layer,
                        say, shape_of, tiled_inputs, tokenwise_rel)
from helpers import np_f64, np_store

pytestmark = pytest.mark.gpu
C = moe_inputs.CONFIGS


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _sample_tokens(orc, idx, E, slice_rows=64, extra=8, seed=0):
    """Tokens whose rows cover every slice of `slice_rows` rows of every expert
    group (one random row per slice, plus each group's first and last row):
    with 64-row slices every M-tile of either MFMA kernel (64 or 256 rows) is
    checked, with 16-row slices every token tile of the skinny kernel; plus a
    few random tokens."""
    T, k = idx.shape
    counts, offsets, perm, _ = orc.dispatch(idx, E)
    rng = np.random.default_rng(seed)
    rows = set()
    for e in range(E):
        o, c = int(offsets[e]), int(counts[e])
        if c == 0:
            continue
        rows.update((o, o + c - 1))
        for s0 in range(0, c, slice_rows):
            rows.add(o + s0 + int(rng.integers(min(slice_rows, c - s0))))
    sel = {int(perm[p]) // k for p in rows}
    sel.update(rng.choice(T, min(extra, T), replace=False).tolist())
    return np.array(sorted(sel), np.int32)


def _elementwise_rel(y, r):
    """R12's element-wise relative error with a floor of 1e-3 of the token's
    largest reference magnitude (reported beside the per-token bar)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    floor = 1e-3 * np.abs(r).max(axis=1, keepdims=True)
    return float((np.abs(y - r) / np.maximum(np.abs(r), np.maximum(floor, 1e-30))).max())


def _check_layer(orc, cfg, d, y, counts, idx, sel=None, residual=None):
    gi = idx.cpu().numpy()
    x = np_store(d["x"])
    wr, br = np_store(d["w_router"]), np_store(d["b_router"])
    # routing on every token: the oracle's own fp64 logits and top-k
    lg = orc.router_logits(x, cfg.act, wr, br)
    oi, _ = orc.topk(lg, cfg.k)
    flips = check_routing_with_flips(gi, oi, lg, cfg.k)
    assert np.array_equal(counts.cpu().numpy(), np.bincount(gi.ravel(), minlength=cfg.E))
    # outputs of the sampled tokens with the GPU's expert choice
    if sel is None:
        sel = _sample_tokens(orc, gi, cfg.E)
    W, S = oracle_weights(d)
    say(f"  oracle on {len(sel)} tokens")
    y_f, _, _, _ = orc.layer_forward(x, cfg.act, cfg.wt, cfg.k, wr, br, W, S,
                                     residual=None if residual is None else np_store(residual),
                                     forced_idx=gi, sel=sel)
    yg = np_f64(y)[sel]
    err = tokenwise_rel(yg, y_f)
    say(f"  per-token max rel {err.max():.3g} (mean {err.mean():.3g}), element-wise with floor "
        f"{_elementwise_rel(yg, y_f):.3g}, flips {flips}")
    assert err.max() < TOL[cfg.wt]
    return flips


def test_mixtral_decode_full(orc):
    cfg = C["mixtral_decode"]
    say("full mixtral decode T=8")
    d = device_inputs(cfg)
    y, counts, idx = run_layer(cfg, d)
    _check_layer(orc, cfg, d, y, counts, idx, sel=np.arange(cfg.T, dtype=np.int32))


@pytest.mark.parametrize("T", [32, 96])
def test_mixtral_decode_skinny_full(orc, T):
    """The page's 32 x 4096 x 14336 top-2 shape (groups of 6-11 rows: the
    one-tile skinny MFMA kernel) and 96 tokens (17-33 rows: three token tiles)."""
    cfg = C["mixtral_decode"].replace(name=f"mixtral_decode_t{T}", T=T)
    say(f"full mixtral decode T={T}")
    d = device_inputs(cfg)
    y, counts, idx = run_layer(cfg, d)
    say(f"  counts {counts.cpu().tolist()}")
    _check_layer(orc, cfg, d, y, counts, idx, sel=_sample_tokens(orc, idx.cpu().numpy(), cfg.E, slice_rows=16))


def test_mixtral_prefill_full(orc):
    cfg = C["mixtral_prefill"]
    say("full mixtral prefill T=4096 (Zipf-loaded experts)")
    d = device_inputs(cfg)
    y, counts, idx = run_layer(cfg, d)
    c = counts.cpu().numpy()
    say(f"  counts {c.tolist()}")
    assert c[0] > 2 * c[-1]       # skewed as calibrated
    _check_layer(orc, cfg, d, y, counts, idx)
    # bitwise run-to-run determinism at full size
    y2, counts2, idx2 = run_layer(cfg, d)
    assert torch.equal(y, y2) and torch.equal(idx, idx2)


@pytest.mark.parametrize("wt", ["int4", "int4_tiled"])
def test_fine_int4_decode_full(orc, wt):
    """Row-major codes and the tiled codes the bench streams."""
    cfg = C["fine_int4_decode"]
    say(f"full fine-grained int4 decode T=64 E=256 + shared, {wt}")
    d = device_inputs(cfg)
    y, counts, idx = run_layer(cfg, tiled_inputs(d) if wt == "int4_tiled" else d, wt=wt)
    say(f"  active experts {(counts > 0).sum().item()}")
    _check_layer(orc, cfg, d, y, counts, idx, sel=np.arange(0, cfg.T, 2, dtype=np.int32))


@pytest.mark.parametrize("name", ["fine_int4_prefill", "fine_mxfp4_prefill", "mixtral_mxfp8_prefill"])
def test_quantised_prefill_full(orc, name):
    """Prefill-sized groups of quantised experts on the dequantising grouped
    GEMM: the fine-grained int4-g128 layer (E=256, top-8, shared expert) and
    MXFP4 experts at T=4096, and the Mixtral-shaped layer with MXFP8 experts.
    Routing on every token; outputs on 16 seeded random tokens (the oracle
    decodes every weight element per use, so larger samples take minutes)."""
    cfg = C[name]
    say(f"full {name} T={cfg.T}")
    d = device_inputs(cfg)
    y, counts, idx = run_layer(cfg, d)
    c = counts.cpu().numpy()
    say(f"  active experts {(c > 0).sum()}, largest group {c.max()}")
    sel = np.sort(np.random.default_rng(7).choice(cfg.T, 16, replace=False)).astype(np.int32)
    _check_layer(orc, cfg, d, y, counts, idx, sel=sel)


@pytest.mark.parametrize("name,T", [("fine_mxfp4_prefill", 64), ("mixtral_mxfp8_prefill", 8)])
def test_mx_decode_full(orc, name, T):
    """The MX layers at decode as the bench times them: the first T tokens of
    the prefill inputs, the codes packed once into the tiled layout, every
    group on the skinny matrix-core kernel.  Routing on every token, outputs
    on every token."""
    cfg = C[name].replace(name=f"{name}_t{T}", T=T)
    say(f"full {name} at decode T={T}, tiled codes")
    d = dict(device_inputs(C[name]))
    d["x"] = d["x"][:T].contiguous()
    t = tiled_inputs(d, cfg.wt)
    y, counts, idx = run_layer(cfg, t, wt=f"{cfg.wt}_tiled")
    say(f"  active experts {(counts > 0).sum().item()}")
    _check_layer(orc, cfg, d, y, counts, idx, sel=np.arange(T, dtype=np.int32))


def test_stack4_full_teacher_forced(orc):
    """Four pre-norm layers with residual; each layer checked on the GPU's own
    input (teacher forcing), plus the per-layer usage histogram."""
    cfg = C["stack4"]
    say("full 4-layer stack T=512 E=64 top-6")
    inp = moe_inputs.generate(cfg, seed=0, device=DEV)
    h = inp["x"].to(DEV)
    hist = []
    pred = None          # layer l+1's experts predicted from layer l's input
    for l in range(cfg.layers):
        L = inp["layers"][l]
        d = {"w_router": L["w_router"].to(DEV), "b_router": None}
        for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                  "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down"):
            d[n] = None if L.get(n) is None else L[n].to(DEV)
        gamma = inp["gamma"][l].to(DEV)
        n_ = torch.empty_like(h)
        moe.moe_rmsnorm(shape_of(cfg), h, gamma, inp["eps"], n_)
        torch.cuda.synchronize()
        ref_n = orc.rmsnorm(np_store(h), "bf16", inp["gamma"][l].numpy(), inp["eps"])
        assert tokenwise_rel(np_f64(n_), ref_n).max() < 8e-3
        d["x"] = n_
        y, counts, idx = run_layer(cfg, d, residual=h)
        say(f"  layer {l}")
        _check_layer(orc, cfg, d, y, counts, idx, residual=h)
        if pred is not None:
            # one-layer-ahead prediction scored on the GPU, against the
            # oracle's count on the same selections (bit-exact)
            ov = torch.empty(cfg.k + 1, dtype=torch.int32, device=DEV)
            moe.moe_topk_overlap(shape_of(cfg), pred, idx, ov)
            torch.cuda.synchronize()
            ref = orc.topk_overlap(pred.cpu().numpy(), idx.cpu().numpy())
            assert ov.cpu().numpy().tolist() == ref.tolist()
            hit = float((np.arange(cfg.k + 1) * ref).sum()) / (cfg.T * cfg.k)
            say(f"  layer {l}: experts predicted one layer ahead {hit:.3f}")
        if l + 1 < cfg.layers:
            # the next layer's router on this layer's normed input (PILOT), a
            # moe_route call whose selection is checked bit-exact on its logits
            wr_next = inp["layers"][l + 1]["w_router"]
            lg = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=DEV)
            pred = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=DEV)
            pw = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=DEV)
            moe.moe_route(shape_of(cfg), n_, wr_next.to(DEV), None, lg, pred, pw)
            torch.cuda.synchronize()
            oi, _ = orc.topk(lg.cpu().numpy().astype(np.float64), cfg.k)
            assert np.array_equal(pred.cpu().numpy(), oi)
        c = counts.cpu().numpy()
        hist += [(l, e, int(c[e])) for e in range(cfg.E) if c[e] > 0]
        h = y.clone()
    assert sum(c for (_, _, c) in hist) == cfg.layers * cfg.T * cfg.k
    # consecutive layers' routers are correlated, so expert choices overlap
    say(f"  histogram lines {len(hist)}")
