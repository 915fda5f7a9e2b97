"""Pins of the fp64 oracle against things other than itself.

Each test compares the oracle with a library routine (NumPy/SciPy), a closed
form, a brute-force enumeration, an invariant the pages fix, or a worked
example printed on the pages.  All run on the CPU.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs
from helpers import layer_np, np_store, shared_np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- decoders

def test_fp16_decoder_exhaustive(orc):
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([orc.dec_f16(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decoder_exhaustive(orc):
    codes = np.arange(65536, dtype=np.uint32)
    ref = (codes << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([orc.dec_bf16(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_int4_decoder_exhaustive(orc):
    table = [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]
    for b in range(256):
        assert orc.dec_int4(b, 0) == table[b & 15]
        assert orc.dec_int4(b, 1) == table[b >> 4]


def test_generator_int4_roundtrip_matches_numpy_quantiser():
    """The generator's packing equals an independent NumPy quantiser."""
    g = torch.Generator().manual_seed(3)
    w = torch.randn(5, 256, generator=g) * 0.02
    packed, s16 = moe_inputs.quantise_int4_g128(w)
    wn = w.numpy().reshape(5, 2, 128)
    s = (np.abs(wn).max(-1) / np.float32(7)).astype(np.float16)
    q = np.clip(np.round(wn / s.astype(np.float32)[..., None]), -8, 7).astype(np.int8).reshape(5, 256)
    u = (q & 15).astype(np.uint8)
    assert np.array_equal(s16.numpy(), s)
    assert np.array_equal(packed.numpy(), u[:, 0::2] | (u[:, 1::2] << 4))


# ------------------------------------------------------------------- router

def test_router_logits_vs_numpy(orc):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 48)).astype(np.float32)
    wg = rng.standard_normal((5, 48)).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    ref = x.astype(np.float64) @ wg.astype(np.float64).T + b
    got = orc.router_logits(x, "f32", wg, b)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    got_b = orc.router_logits(np_store(xb), "bf16", wg, None)
    ref_b = xb.double().numpy() @ wg.astype(np.float64).T
    np.testing.assert_allclose(got_b, ref_b, rtol=1e-13, atol=1e-13)


def test_softmax_vs_scipy(orc):
    rng = np.random.default_rng(2)
    L = rng.standard_normal((9, 13)) * 5
    np.testing.assert_allclose(orc.softmax(L), scipy.special.softmax(L, axis=1), rtol=1e-13)


# -------------------------------------------------------------------- top-k

def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-row[e], e))
    return order[:k]


def test_topk_exhaustive_small(orc):
    """Brute-force full sort on every logit vector in {0,1,2}^E, E <= 5, all k."""
    for E in range(1, 6):
        rows = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=E)))
        for k in range(1, E + 1):
            idx, w = orc.topk(rows, k)
            ref = np.array([_brute_topk(r, k) for r in rows])
            assert np.array_equal(idx, ref), (E, k)
            np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)


def test_topk_random_vs_sort(orc):
    rng = np.random.default_rng(3)
    for E, k in [(8, 2), (64, 6), (256, 8), (16, 16)]:
        L = rng.standard_normal((200, E))
        L[::7, 1] = L[::7, 0]          # planted exact ties
        idx, _ = orc.topk(L, k)
        ref = np.array([_brute_topk(r, k) for r in L])
        assert np.array_equal(idx, ref)


def test_topk_all_equal_gives_lowest_indices(orc):
    idx, w = orc.topk(np.zeros((3, 8)), 3)
    assert (idx == [0, 1, 2]).all()
    np.testing.assert_allclose(w, 1 / 3, rtol=1e-15)


def test_renormalised_weights(orc):
    """w_j = P[idx_j] / sum_m P[idx_m] with P a library softmax; sum_j w_j = 1."""
    rng = np.random.default_rng(4)
    L = rng.standard_normal((100, 64)) * 3
    idx, w = orc.topk(L, 6)
    P = scipy.special.softmax(L, axis=1)
    sel = np.take_along_axis(P, idx, axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-12)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-14)
    assert (np.diff(w, axis=1) <= 0).all()   # descending slots


# ----------------------------------------------------------------- dispatch

def test_dispatch_pages_example(orc):
    with open(os.path.join(GOLDEN, "p2_routing_pattern.json")) as f:
        g = json.load(f)
    idx = np.array(g["idx"], np.int32)
    counts, offsets, perm, inv = orc.dispatch(idx, g["E"])
    assert counts.tolist() == g["expected_counts"]
    for e, toks in g["expected_segments"].items():
        e = int(e)
        seg = perm[offsets[e]:offsets[e + 1]] // g["k"]
        assert seg.tolist() == toks


@pytest.mark.parametrize("T,k,E", [(16, 2, 8), (512, 6, 64), (64, 8, 256), (33, 3, 5), (1, 4, 4)])
def test_dispatch_is_stable_bijection(orc, T, k, E):
    rng = np.random.default_rng(T * 1000 + E)
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
    counts, offsets, perm, inv = orc.dispatch(idx, E)
    flat = idx.ravel()
    assert counts.sum() == T * k
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(perm[inv], np.arange(T * k))
    assert np.array_equal(inv[perm], np.arange(T * k))
    assert offsets[0] == 0 and offsets[-1] == T * k
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


def test_dispatch_rejects_bad_index(orc):
    with pytest.raises(ValueError):
        orc.dispatch(np.array([[0, 9]], np.int32), 8)


# --------------------------------------------------------------- SwiGLU FFN

def _np_swiglu(x, wg, wu, wd):
    g = x @ wg.T
    return ((g / (1 + np.exp(-g))) * (x @ wu.T)) @ wd.T


def _rand_layer(rng, E, d, F, scale=0.2):
    return {"w_gate": (rng.standard_normal((E, F, d)) * scale).astype(np.float32),
            "w_up": (rng.standard_normal((E, F, d)) * scale).astype(np.float32),
            "w_down": (rng.standard_normal((E, d, F)) * scale).astype(np.float32)}


def test_single_expert_is_textbook_swiglu(orc):
    """E = 1, k = 1: the layer reduces to a plain SwiGLU MLP (NumPy matmuls)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 32)).astype(np.float32)
    W = _rand_layer(rng, 1, 32, 24)
    wr = rng.standard_normal((1, 32)).astype(np.float32)
    y, idx, w, _ = orc.layer_forward(x, "f32", "f32", 1, wr, None, W)
    ref = _np_swiglu(x.astype(np.float64), W["w_gate"][0].astype(np.float64),
                     W["w_up"][0].astype(np.float64), W["w_down"][0].astype(np.float64))
    assert (idx == 0).all() and (w == 1.0).all()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("E", [4, 8])
def test_k_equals_E_is_dense_softmax_mixture(orc, E):
    """With k = E the routed layer equals sum_e softmax(L)_e * FFN_e(x)."""
    rng = np.random.default_rng(6 + E)
    d, F, T = 32, 40, 9
    x = rng.standard_normal((T, d)).astype(np.float32)
    W = _rand_layer(rng, E, d, F)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    y, _, _, _ = orc.layer_forward(x, "f32", "f32", E, wr, b, W)
    x64 = x.astype(np.float64)
    P = scipy.special.softmax(x64 @ wr.astype(np.float64).T + b, axis=1)
    ref = np.zeros((T, d))
    for e in range(E):
        ref += P[:, e:e + 1] * _np_swiglu(x64, W["w_gate"][e].astype(np.float64),
                                          W["w_up"][e].astype(np.float64),
                                          W["w_down"][e].astype(np.float64))
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_k1_picks_argmax_expert(orc):
    rng = np.random.default_rng(8)
    E, d, F, T = 6, 16, 8, 20
    x = rng.standard_normal((T, d)).astype(np.float32)
    W = _rand_layer(rng, E, d, F)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    y, idx, _, _ = orc.layer_forward(x, "f32", "f32", 1, wr, None, W)
    L = x.astype(np.float64) @ wr.astype(np.float64).T
    assert np.array_equal(idx[:, 0], L.argmax(1))
    for t in range(T):
        e = idx[t, 0]
        ref = _np_swiglu(x[t:t + 1].astype(np.float64), W["w_gate"][e].astype(np.float64),
                         W["w_up"][e].astype(np.float64), W["w_down"][e].astype(np.float64))
        np.testing.assert_allclose(y[t], ref[0], rtol=1e-12, atol=1e-12)


def test_linearity_in_down_projection(orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 16)).astype(np.float32)
    W = _rand_layer(rng, 4, 16, 12)
    wr = rng.standard_normal((4, 16)).astype(np.float32)
    y1, _, _, _ = orc.layer_forward(x, "f32", "f32", 2, wr, None, W)
    W2 = dict(W, w_down=(W["w_down"] * 2).astype(np.float32))
    y2, _, _, _ = orc.layer_forward(x, "f32", "f32", 2, wr, None, W2)
    assert np.array_equal(y2, 2 * y1)


def test_token_permutation_equivariance(orc):
    rng = np.random.default_rng(10)
    x = rng.standard_normal((11, 16)).astype(np.float32)
    W = _rand_layer(rng, 5, 16, 12)
    wr = rng.standard_normal((5, 16)).astype(np.float32)
    y, _, _, _ = orc.layer_forward(x, "f32", "f32", 2, wr, None, W)
    pi = rng.permutation(11)
    yp, _, _, _ = orc.layer_forward(np.ascontiguousarray(x[pi]), "f32", "f32", 2, wr, None, W)
    assert np.array_equal(yp, y[pi])


def test_token_subset_matches_full(orc):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((12, 16)).astype(np.float32)
    W = _rand_layer(rng, 5, 16, 12)
    wr = rng.standard_normal((5, 16)).astype(np.float32)
    y, idx, w, lg = orc.layer_forward(x, "f32", "f32", 2, wr, None, W)
    sel = np.array([11, 0, 5], np.int32)
    ys, idxs, ws, lgs = orc.layer_forward(x, "f32", "f32", 2, wr, None, W, sel=sel)
    assert np.array_equal(ys, y[sel]) and np.array_equal(idxs, idx[sel])


def test_int4_layer_equals_dequantised_fp32(orc):
    """An int4 layer equals the fp32 layer whose weights are q*s (exact in fp32);
    pins nibble order, group indexing and scale decoding."""
    cfg = moe_inputs.MoEConfig("t", T=5, d=256, E=3, k=2, F=128, act="bf16", wt="int4",
                               model="pin_int4", n_shared=1, w_std=0.02)
    inp = moe_inputs.generate(cfg, seed=1)
    L = inp["layers"][0]
    x = np_store(inp["x"])
    W = layer_np(L)
    S = shared_np(L)

    def deq(p, s):
        lo = (p & 15).astype(np.int8)
        hi = (p >> 4).astype(np.int8)
        q = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int8)
        q[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
        q[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
        sc = np.repeat(s.view(np.float16).astype(np.float32), 128, axis=-1)
        return (q.astype(np.float32) * sc).astype(np.float32)

    Wf = {n: np.ascontiguousarray(deq(W["w_" + n[2:]], W["s_" + n[2:]]))
          for n in ("w_gate", "w_up", "w_down")}
    Sf = {n: np.ascontiguousarray(deq(S["w_" + n[2:]], S["s_" + n[2:]]))
          for n in ("w_gate", "w_up", "w_down")}
    wr = np_store(L["w_router"])
    y4, i4, _, _ = orc.layer_forward(x, "bf16", "int4", 2, wr, None, W, S)
    yf, i_f, _, _ = orc.layer_forward(x, "bf16", "f32", 2, wr, None, Wf, Sf)
    assert np.array_equal(i4, i_f)
    assert np.array_equal(y4, yf)


def test_bf16_weights_equal_fp32_of_same_values(orc):
    rng = np.random.default_rng(12)
    Wt = {n: torch.from_numpy(v).to(torch.bfloat16) for n, v in _rand_layer(rng, 3, 16, 8).items()}
    W16 = {n: np_store(v) for n, v in Wt.items()}
    W32 = {n: v.float().numpy() for n, v in Wt.items()}
    x = rng.standard_normal((4, 16)).astype(np.float32)
    wr = rng.standard_normal((3, 16)).astype(np.float32)
    a, _, _, _ = orc.layer_forward(x, "f32", "bf16", 2, wr, None, W16)
    b, _, _, _ = orc.layer_forward(x, "f32", "f32", 2, wr, None, W32)
    assert np.array_equal(a, b)


def test_shared_expert_is_additive_swiglu(orc):
    rng = np.random.default_rng(13)
    d, F = 16, 12
    x = rng.standard_normal((6, d)).astype(np.float32)
    W = _rand_layer(rng, 4, d, F)
    S = _rand_layer(rng, 1, d, F)
    wr = rng.standard_normal((4, d)).astype(np.float32)
    y0, _, _, _ = orc.layer_forward(x, "f32", "f32", 2, wr, None, W)
    y1, _, _, _ = orc.layer_forward(x, "f32", "f32", 2, wr, None, W, S)
    ref = _np_swiglu(x.astype(np.float64), S["w_gate"][0].astype(np.float64),
                     S["w_up"][0].astype(np.float64), S["w_down"][0].astype(np.float64))
    np.testing.assert_allclose(y1 - y0, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(orc.shared_ffn(x, "f32", "f32", S), ref, rtol=1e-12, atol=1e-12)


def test_residual_is_additive(orc):
    rng = np.random.default_rng(14)
    x = rng.standard_normal((6, 16)).astype(np.float32)
    r = rng.standard_normal((6, 16)).astype(np.float32)
    W = _rand_layer(rng, 4, 16, 8)
    wr = rng.standard_normal((4, 16)).astype(np.float32)
    y0, _, _, _ = orc.layer_forward(x, "f32", "f32", 2, wr, None, W)
    y1, _, _, _ = orc.layer_forward(x, "f32", "f32", 2, wr, None, W, residual=r)
    np.testing.assert_allclose(y1 - y0, r, rtol=0, atol=1e-12)


def test_forced_routing_weights(orc):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 16)).astype(np.float32)
    W = _rand_layer(rng, 5, 16, 8)
    wr = rng.standard_normal((5, 16)).astype(np.float32)
    forced = np.array([[4, 0], [1, 2], [3, 4], [0, 1]], np.int32)
    y, idx, w, lg = orc.layer_forward(x, "f32", "f32", 2, wr, None, W, forced_idx=forced)
    assert np.array_equal(idx, forced)
    sel = np.take_along_axis(lg, forced, axis=1)
    np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-12)


def test_steps_compose_to_layer(orc):
    """router -> top-k -> dispatch -> expert FFN -> combine equals the per-token
    definition, on the tiny fp32 workload."""
    cfg = moe_inputs.CONFIGS["tiny_f32"]
    inp = moe_inputs.generate(cfg, seed=0)
    L = inp["layers"][0]
    x = np_store(inp["x"])
    W = layer_np(L)
    wr = np_store(L["w_router"])
    lg = orc.router_logits(x, "f32", wr, None)
    idx, w = orc.topk(lg, cfg.k)
    counts, offsets, perm, inv = orc.dispatch(idx, cfg.E)
    yp = orc.expert_ffn(x, "f32", "f32", W, counts, offsets, perm, cfg.k)
    y = orc.combine(yp, inv, w, cfg.k)
    y_ref, idx_ref, w_ref, lg_ref = orc.layer_forward(x, "f32", "f32", cfg.k, wr, None, W)
    assert np.array_equal(idx, idx_ref)
    np.testing.assert_allclose(lg, lg_ref, rtol=0, atol=0)
    np.testing.assert_allclose(y, y_ref, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_closed_forms(orc):
    d = 16
    h = np.zeros((3, d), np.float32)
    h[0, :] = 3.0                      # constant row -> 3/sqrt(9+eps)
    h[1, 0], h[1, 1] = 3.0, 4.0        # mean square 25/d
    h[2, :] = np.arange(d)
    g = np.linspace(0.5, 2.0, d).astype(np.float32)
    out = orc.rmsnorm(h, "f32", g, 1e-6)
    np.testing.assert_allclose(out[0], 3 / np.sqrt(9 + 1e-6) * g, rtol=1e-14)
    np.testing.assert_allclose(out[1, :2], np.array([3, 4]) / np.sqrt(25 / d + 1e-6) * g[:2],
                               rtol=1e-14)
    assert (out[1, 2:] == 0).all()
    # scale invariance (eps -> 0)
    a = orc.rmsnorm(h[2:3], "f32", g, 0.0)
    b = orc.rmsnorm((h[2:3] * 8).astype(np.float32), "f32", g, 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-14)


# ------------------------------------------------------------- inputs + bias

def test_generator_is_deterministic():
    cfg = moe_inputs.CONFIGS["tiny_f32"]
    a = moe_inputs.generate(cfg, seed=0)
    b = moe_inputs.generate(cfg, seed=0)
    c = moe_inputs.generate(cfg, seed=1)
    assert torch.equal(a["x"], b["x"]) and torch.equal(a["layers"][0]["w_down"],
                                                       b["layers"][0]["w_down"])
    assert not torch.equal(a["x"], c["x"])


def test_stack_routers_are_correlated():
    cfg = moe_inputs.CONFIGS["stack4"].replace(d=256, E=8)
    w0 = moe_inputs.router_weights(cfg, 0, 0).flatten()
    w1 = moe_inputs.router_weights(cfg, 0, 1).flatten()
    c = torch.corrcoef(torch.stack([w0, w1]))[0, 1]
    assert 0.8 < c < 0.98     # 0.7 / sqrt(0.49 + 0.09) ~ 0.92


def test_zipf_bias_reaches_targets(orc):
    """The stored bias makes the oracle's top-2 frequencies follow Zipf(1.1)."""
    cfg = moe_inputs.CONFIGS["mixtral_prefill"]
    b = moe_inputs.router_bias(cfg).numpy()
    x = np_store(moe_inputs.activations(cfg, 0))
    wr = np_store(moe_inputs.router_weights(cfg, 0, 0))
    lg = orc.router_logits(x, "bf16", wr, b)
    idx, _ = orc.topk(lg, cfg.k)
    f = np.bincount(idx.ravel(), minlength=cfg.E) / idx.size
    np.testing.assert_allclose(f, moe_inputs.zipf_targets(cfg.E), atol=0.01)


def test_topk_overlap_brute_force(orc):
    """The one-layer-ahead prediction score against set intersections written
    out in Python: random distinct selections, identical ones (every token
    shares k), disjoint ones (shares 0) and reversed order (order ignored)."""
    rng = np.random.default_rng(11)
    for T, E, k in ((1, 4, 1), (37, 8, 2), (64, 64, 6), (9, 16, 16)):
        pred = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
        act = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
        want = np.zeros(k + 1, np.int64)
        for t in range(T):
            want[len(set(pred[t].tolist()) & set(act[t].tolist()))] += 1
        assert orc.topk_overlap(pred, act).tolist() == want.tolist()
        assert orc.topk_overlap(pred, pred[:, ::-1].copy()).tolist() == [0] * k + [T]
        if 2 * k <= E:
            other = np.array([[e for e in range(E) if e not in row][:k] for row in pred], np.int32)
            assert orc.topk_overlap(pred, other).tolist() == [T] + [0] * k


# ---------------------------------------------------------- small float formats

def test_minifloat_decoder_against_library_formats(orc):
    """The oracle's generic small-float decoder, pinned on formats a library
    implements: every IEEE binary16 code against NumPy, every E4M3 ("fn") code
    against torch.float8_e4m3fn, and the all-finite convention against NumPy
    on every finite binary16 code (the path E2M1 takes)."""
    codes = np.arange(65536, dtype=np.uint32)
    ref = codes.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([orc.dec_minifloat(int(c), 5, 10, 15, orc.MF_IEEE) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    fin = ((codes >> 10) & 31) != 31
    got_f = np.array([orc.dec_minifloat(int(c), 5, 10, 15, orc.MF_FINITE) for c in codes[fin]])
    assert np.array_equal(got_f, ref[fin])
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got8 = np.array([orc.dec_minifloat(c, 4, 3, 7, orc.MF_FN) for c in range(256)])
    assert np.array_equal(np.isnan(got8), np.isnan(e4))
    assert np.array_equal(got8[~np.isnan(e4)], e4[~np.isnan(e4)])


def test_e2m1_and_e8m0_decoders(orc):
    """E2M1 (the OCP MX fp4 element): the sixteen codes are the eight
    magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives (sign in bit 3);
    E8M0 scales against torch.float8_e8m0fnu on every code."""
    mags = [orc.dec_minifloat(c, 2, 1, 1, orc.MF_FINITE) for c in range(8)]
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert orc.dec_minifloat(c | 8, 2, 1, 1, orc.MF_FINITE) == -mags[c]
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([orc.dec_e8m0(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def _dequant_np(cfg_wt, w, s, K):
    """Dequantised fp32-representable weights, computed here with NumPy and
    torch decoders (independently of the oracle's C decoders)."""
    if cfg_wt in ("int4", "int4g64"):
        gs = 128 if cfg_wt == "int4" else 64
        lo = (w & 0xF).astype(np.int32)
        hi = (w >> 4).astype(np.int32)
        q = np.empty(w.shape[:-1] + (K,), np.int32)
        q[..., 0::2], q[..., 1::2] = lo, hi
        q = np.where(q >= 8, q - 16, q)
        sc = s.view(np.float16).astype(np.float64)
        return q * np.repeat(sc, gs, axis=-1)
    x = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    x = np.repeat(x, 32, axis=-1)
    if cfg_wt == "mxfp8":
        e = torch.from_numpy(w.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return e * x
    table = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    nib = np.empty(w.shape[:-1] + (K,), np.uint8)
    nib[..., 0::2], nib[..., 1::2] = w & 0xF, w >> 4
    v = table[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return v * x


@pytest.mark.parametrize("wt", ["int4g64", "mxfp4", "mxfp8"])
def test_quantised_layer_equals_fp32_layer_of_dequantised_weights(orc, wt):
    """A layer with int4-g64, MXFP4 or MXFP8 experts equals the fp32 layer of
    the weights dequantised independently (NumPy / torch decoders): pins code
    order inside bytes, group and block indexing and scale decoding.  The
    dequantised values are exactly representable in fp32."""
    cfg = moe_inputs.MoEConfig(f"q_{wt}", T=9, d=128, E=3, k=2, F=192, act="bf16", wt=wt,
                               model=f"q_{wt}", n_shared=1, w_std=0.05)
    inp = moe_inputs.generate(cfg, seed=0)
    L = inp["layers"][0]
    x = np_store(inp["x"])
    W = layer_np(L)
    S = shared_np(L)
    deq = {}
    for n, K in (("gate", cfg.d), ("up", cfg.d), ("down", cfg.F)):
        deq["w_" + n] = _dequant_np(wt, W["w_" + n], W["s_" + n], K).astype(np.float32)
    deq_s = {("w_" + n): _dequant_np(wt, S["w_" + n], S["s_" + n], K).astype(np.float32)
             for n, K in (("gate", cfg.d), ("up", cfg.d), ("down", cfg.F))}
    for n in deq:
        assert np.array_equal(deq[n].astype(np.float64), _dequant_np(wt, W[n], W["s_" + n[2:]],
                                                                     deq[n].shape[-1]))
    wr = np_store(L["w_router"])
    y_q, idx_q, _, _ = orc.layer_forward(x, "bf16", wt, cfg.k, wr, None, W, S)
    y_f, idx_f, _, _ = orc.layer_forward(x, "bf16", "f32", cfg.k, wr, None, deq, deq_s)
    assert np.array_equal(idx_q, idx_f)
    np.testing.assert_allclose(y_q, y_f, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_mx_quantiser_rounds_to_nearest(elem):
    """The input generator's MX quantiser (not the oracle): every element lies
    within half an element step of the value it encodes; values beyond the
    element format's largest magnitude (possible with the shared exponent
    floor(log2 amax) - emax) saturate to it."""
    w = torch.randn(4, 256, generator=torch.Generator().manual_seed(3)) * 0.02
    codes, sc = moe_inputs.quantise_mx(w, elem)
    deq = _dequant_np("mxfp4" if elem == "e2m1" else "mxfp8", codes.numpy(), sc.numpy(), 256)
    x = np.repeat(torch.from_numpy(sc.numpy().copy()).view(torch.float8_e8m0fnu).double().numpy(), 32, -1)
    v = w.double().numpy() / x
    err = np.abs(deq / x - v)
    # the element grid's spacing at |v|: 2^(floor(log2|v|) - mbits) above the subnormals
    mbits = 1 if elem == "e2m1" else 3
    minexp = 0 if elem == "e2m1" else -6
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(v), 1e-30))), minexp)
    top = 6.0 if elem == "e2m1" else 448.0
    inside = np.abs(v) <= top
    assert (err[inside] <= 0.5 * 2.0 ** (e[inside] - mbits) + 1e-12).all()
    assert np.array_equal(np.abs(deq / x)[~inside], np.full((~inside).sum(), top))
