"""GPU parity: every step of the HIP path, called through the C ABI, against the
fp64 oracle on the same seeded inputs.

Bars: expert indices and the dispatch permutation bit-exact (given the same
router logits); outputs within a per-token relative infinity-norm error of 1e-5
(fp32) or 2e-2 (bf16 / int4); end-to-end index flips only where the oracle's
fp64 k-th / (k+1)-th logit margin is below 1e-5.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import moe_layer_forward_amd as moe
from gpu_common import (DEV, TOL, act_dtype, check_routing_with_flips, device_inputs,
                        oracle_weights, run_layer, say, shape_of, tiled_inputs, tokenwise_rel,
                        weights_struct)
from helpers import np_f64, np_store

pytestmark = pytest.mark.gpu

C = moe_inputs.CONFIGS
SMALL = {
    "tiny_f32": C["tiny_f32"],
    "bf16_decode_small": moe_inputs.MoEConfig(
        "bf16_decode_small", T=8, d=512, E=8, k=2, F=1024, act="bf16", wt="bf16",
        model="s_bf16_dec", w_std=0.05),
    "bf16_prefill_ragged": moe_inputs.MoEConfig(
        "bf16_prefill_ragged", T=600, d=256, E=6, k=2, F=328, act="bf16", wt="bf16",
        model="s_bf16_pre", w_std=0.05),
    # 256-row MFMA tiles with K a multiple of 64 in both projections (copies
    # issued from the compute phase): F = 384 gives gate/up three N-tiles,
    # d = 320 leaves the down pass a 64-row last N-tile, ~320-row groups a
    # ragged second M-tile, and the tail rounds are cut into K parts
    "bf16_prefill_fast": moe_inputs.MoEConfig(
        "bf16_prefill_fast", T=640, d=320, E=4, k=2, F=384, act="bf16", wt="bf16",
        model="s_bf16_fast", w_std=0.05),
    # more gate/up tiles (16 M-tiles x 20 N-tiles) than blocks: blocks run
    # several tiles, the copy stream crosses into the next tile (and into K
    # parts of the split last round)
    "bf16_prefill_stream": moe_inputs.MoEConfig(
        "bf16_prefill_stream", T=4096, d=256, E=2, k=1, F=2560, act="bf16", wt="bf16",
        model="s_bf16_stream", w_std=0.05),
    # 128 experts of ~32 rows on the 64-row MFMA tiles, more tiles than two
    # blocks per CU in both projections (~635 each: blocks take a second tile)
    "bf16_small_split": moe_inputs.MoEConfig(
        "bf16_small_split", T=512, d=1280, E=128, k=8, F=640, act="bf16", wt="bf16",
        model="s_bf16_ssplit", w_std=0.05),
    "int4_shared_small": moe_inputs.MoEConfig(
        "int4_shared_small", T=16, d=512, E=16, k=4, F=256, act="bf16", wt="int4",
        model="s_int4", n_shared=1, w_std=0.05),
    "int4_ktail": moe_inputs.MoEConfig(
        "int4_ktail", T=24, d=384, E=8, k=3, F=640, act="bf16", wt="int4",
        model="s_int4_tail", n_shared=0, w_std=0.05),
    # int4 on the matrix cores (K a multiple of 1024): groups larger than one
    # token pass (P = 16 rows at K = 1024 and 2048, 10 at K = 7168), k = E,
    # and many experts holding 0-2 rows
    "int4_mfma_multipass": moe_inputs.MoEConfig(
        "int4_mfma_multipass", T=40, d=1024, E=4, k=2, F=2048, act="bf16", wt="int4",
        model="s_int4_mp", n_shared=1, w_std=0.05),
    "int4_mfma_wide_k": moe_inputs.MoEConfig(
        "int4_mfma_wide_k", T=20, d=7168, E=4, k=4, F=1024, act="bf16", wt="int4",
        model="s_int4_wk", n_shared=0, w_std=0.05),
    "int4_mfma_many": moe_inputs.MoEConfig(
        "int4_mfma_many", T=8, d=1024, E=256, k=8, F=1024, act="bf16", wt="int4",
        model="s_int4_many", n_shared=1, w_std=0.05),
    # bf16 groups of 5-16 rows (counts 10 10 9 5 13 8 10 15): one group above a
    # GEMV pass sends every group to the one-tile skinny MFMA kernel.  It needs
    # K % 64 == 0 and works in tiles of 32 weight rows: F = 1616 leaves a half
    # last tile in gate/up (and keeps down off the kernel); d = 1040 keeps
    # gate/up off and leaves a half last tile in down
    "bf16_skinny_mix": moe_inputs.MoEConfig(
        "bf16_skinny_mix", T=40, d=1024, E=8, k=2, F=1536, act="bf16", wt="bf16",
        model="s_bf16_sk", w_std=0.05),
    "bf16_skinny_ragged": moe_inputs.MoEConfig(
        "bf16_skinny_ragged", T=24, d=1024, E=4, k=2, F=1616, act="bf16", wt="bf16",
        model="s_bf16_skr", w_std=0.05),
    "bf16_skinny_down_ragged": moe_inputs.MoEConfig(
        "bf16_skinny_down_ragged", T=24, d=1040, E=4, k=2, F=1536, act="bf16", wt="bf16",
        model="s_bf16_skd", w_std=0.05),
    # more token tiles per weight operand: counts 14 12 19 16 17 18 (two
    # tiles take every group), 35 39 39 18 29 (three tiles, 16-row gate/up
    # items), 54 49 64 57 (four tiles, the largest group exactly 64) and
    # 71 50 63 65 71 (groups above 64 on the 64-row MFMA tiles beside four
    # skinny tiles).  F = 1408 is not a multiple of 512: the down pass's last
    # K step has lines past the row end
    "bf16_skinny2": moe_inputs.MoEConfig(
        "bf16_skinny2", T=48, d=1024, E=6, k=2, F=1536, act="bf16", wt="bf16",
        model="s_bf16_sk2", w_std=0.05),
    "bf16_skinny2_mix": moe_inputs.MoEConfig(
        "bf16_skinny2_mix", T=80, d=1024, E=5, k=2, F=1536, act="bf16", wt="bf16",
        model="s_bf16_sk2", w_std=0.05),
    "bf16_skinny4": moe_inputs.MoEConfig(
        "bf16_skinny4", T=112, d=1024, E=4, k=2, F=1408, act="bf16", wt="bf16",
        model="s_bf16_sk4", w_std=0.05),
    "bf16_skinny4_mix": moe_inputs.MoEConfig(
        "bf16_skinny4_mix", T=160, d=1024, E=5, k=2, F=1408, act="bf16", wt="bf16",
        model="s_bf16_sk4", w_std=0.05),
    "f32_ragged": moe_inputs.MoEConfig(
        "f32_ragged", T=37, d=200, E=5, k=3, F=72, act="f32", wt="f32", model="s_f32"),
    # an always-on shared expert with bf16 or fp32 weights runs as a one-expert
    # group of all T tokens through the routed experts' kernel selection:
    # 8 rows (GEMV), 40 rows (64-row MFMA tiles) and 520 rows (256-row MFMA
    # tiles with a ragged third tile; routed groups of ~260 rows beside it)
    "bf16_shared_decode": moe_inputs.MoEConfig(
        "bf16_shared_decode", T=8, d=1024, E=8, k=2, F=1024, act="bf16", wt="bf16",
        model="s_bf16_sh", n_shared=1, w_std=0.05),
    "bf16_shared_mid": moe_inputs.MoEConfig(
        "bf16_shared_mid", T=40, d=1024, E=4, k=2, F=1536, act="bf16", wt="bf16",
        model="s_bf16_sh", n_shared=1, w_std=0.05),
    "bf16_shared_prefill": moe_inputs.MoEConfig(
        "bf16_shared_prefill", T=520, d=512, E=4, k=2, F=768, act="bf16", wt="bf16",
        model="s_bf16_shp", n_shared=1, w_std=0.05),
    "f32_shared": moe_inputs.MoEConfig(
        "f32_shared", T=20, d=128, E=4, k=2, F=96, act="f32", wt="f32", model="s_f32_sh",
        n_shared=1),
    # MX experts on the skinny matrix-core kernel (d and F multiples of 1024):
    # decode batches with the shared expert in the same launch, a down pass
    # with K = 9216 (past int4's 8192), and groups of ~150 rows on the
    # dequantising GEMM
    "mxfp4_skinny": moe_inputs.MoEConfig(
        "mxfp4_skinny", T=16, d=1024, E=16, k=4, F=1024, act="bf16", wt="mxfp4",
        model="s_mx4_sk", n_shared=1, w_std=0.05),
    "mxfp8_skinny": moe_inputs.MoEConfig(
        "mxfp8_skinny", T=8, d=2048, E=8, k=2, F=1024, act="bf16", wt="mxfp8",
        model="s_mx8_sk", n_shared=1, w_std=0.05),
    "mxfp4_wide_k": moe_inputs.MoEConfig(
        "mxfp4_wide_k", T=20, d=7168, E=4, k=4, F=1024, act="bf16", wt="mxfp4",
        model="s_mx4_wk", w_std=0.05),
    "mxfp8_skinny_longk": moe_inputs.MoEConfig(
        "mxfp8_skinny_longk", T=6, d=1024, E=4, k=2, F=9216, act="bf16", wt="mxfp8",
        model="s_mx8_lk", w_std=0.05),
    "mxfp4_rem": moe_inputs.MoEConfig(
        "mxfp4_rem", T=300, d=1024, E=4, k=2, F=1024, act="bf16", wt="mxfp4",
        model="s_mx4_rem", n_shared=1, w_std=0.05),
    "mxfp8_rem": moe_inputs.MoEConfig(
        "mxfp8_rem", T=300, d=1024, E=4, k=2, F=1024, act="bf16", wt="mxfp8",
        model="s_mx8_rem", n_shared=1, w_std=0.05),
    # the shape limits moe.h states: k = 16 of E = 256; d and F at 16384 for
    # bf16 and the quantised formats (bf16 gate/up on the GEMV variant with two
    # tokens per pass, K from 8192 to 16384; int4 on the GEMV, K above the int4
    # matrix-core kernel's 8192, one K of a multiple of 1024 and one not; MXFP8
    # on the dequantising GEMM), at 8192 for fp32, and bf16 groups on the
    # 256-row tiles with K = 16384 in one projection or the other
    "limit_k16_e256": moe_inputs.MoEConfig(
        "limit_k16_e256", T=24, d=128, E=256, k=16, F=64, act="bf16", wt="bf16", model="s_lim_k16"),
    "limit_bf16_d16384": moe_inputs.MoEConfig(
        "limit_bf16_d16384", T=6, d=16384, E=3, k=2, F=64, act="bf16", wt="bf16", model="s_lim_bd"),
    "limit_bf16_f16384": moe_inputs.MoEConfig(
        "limit_bf16_f16384", T=6, d=64, E=3, k=2, F=16384, act="bf16", wt="bf16", model="s_lim_bf"),
    "limit_bf16_d16384_tiles": moe_inputs.MoEConfig(
        "limit_bf16_d16384_tiles", T=320, d=16384, E=2, k=1, F=64, act="bf16", wt="bf16", model="s_lim_bdt"),
    "limit_bf16_f16384_tiles": moe_inputs.MoEConfig(
        "limit_bf16_f16384_tiles", T=320, d=64, E=2, k=1, F=16384, act="bf16", wt="bf16", model="s_lim_bft"),
    "limit_f32_d8192": moe_inputs.MoEConfig(
        "limit_f32_d8192", T=5, d=8192, E=3, k=2, F=32, act="f32", wt="f32", model="s_lim_fd"),
    "limit_f32_f8192": moe_inputs.MoEConfig(
        "limit_f32_f8192", T=5, d=32, E=3, k=2, F=8192, act="f32", wt="f32", model="s_lim_ff"),
    "limit_int4_d16384": moe_inputs.MoEConfig(
        "limit_int4_d16384", T=6, d=16384, E=3, k=2, F=128, act="bf16", wt="int4", model="s_lim_id"),
    "limit_int4_f16384": moe_inputs.MoEConfig(
        "limit_int4_f16384", T=6, d=128, E=3, k=2, F=16384, act="bf16", wt="int4", model="s_lim_if"),
    "limit_int4_d16256": moe_inputs.MoEConfig(
        "limit_int4_d16256", T=6, d=16256, E=3, k=2, F=256, act="bf16", wt="int4", model="s_lim_id2"),
    "limit_mxfp8_d16384": moe_inputs.MoEConfig(
        "limit_mxfp8_d16384", T=6, d=16384, E=3, k=2, F=64, act="bf16", wt="mxfp8", model="s_lim_md"),
    # quantised groups above the skinny kernels' range on the dequantising
    # grouped GEMM: int4-g128 groups of ~150 rows and a shared expert over all
    # 300 tokens on the LDS-staged kernel (K = 1024, 64-row tiles); every group
    # of int4-g64, MXFP4 and MXFP8 on the register-fed kernel (K of 448, 320,
    # 512 or 640 is not a multiple of 512 in both passes; 128-row tiles,
    # ragged last N-tiles: F = 320 gate/up columns in 64-wide tiles, d = 448
    # down rows in 128-wide tiles)
    "int4_dq": moe_inputs.MoEConfig(
        "int4_dq", T=300, d=1024, E=4, k=2, F=1024, act="bf16", wt="int4",
        model="s_int4_dq", n_shared=1, w_std=0.05),
    "int4g64_dq": moe_inputs.MoEConfig(
        "int4g64_dq", T=40, d=448, E=6, k=2, F=320, act="bf16", wt="int4g64",
        model="s_int4g64", n_shared=1, w_std=0.05),
    "mxfp4_dq": moe_inputs.MoEConfig(
        "mxfp4_dq", T=200, d=512, E=4, k=2, F=640, act="bf16", wt="mxfp4",
        model="s_mxfp4", n_shared=1, w_std=0.05),
    "mxfp8_dq": moe_inputs.MoEConfig(
        "mxfp8_dq", T=130, d=448, E=5, k=3, F=320, act="bf16", wt="mxfp8",
        model="s_mxfp8", w_std=0.05),
    # the LDS-staged dequantising kernel (both K multiples of 512; int4-g128
    # of 1024: int4_dq above): 64-row tiles, ragged last M-tiles, K = 512 (the
    # fewest stages it takes) and, for MXFP8, more tasks than blocks so the
    # copy stream runs from one task into the next
    "int4g64_staged": moe_inputs.MoEConfig(
        "int4g64_staged", T=160, d=512, E=4, k=2, F=1024, act="bf16", wt="int4g64",
        model="s_i4g64_st", n_shared=1, w_std=0.05),
    # int4 tiles hold 128 token rows with two stages in LDS: more gate/up tasks
    # (24 M-tiles x 16 N-tiles) than blocks, ragged 128-row tiles
    "int4g64_staged_stream": moe_inputs.MoEConfig(
        "int4g64_staged_stream", T=1536, d=512, E=4, k=2, F=4096, act="bf16", wt="int4g64",
        model="s_i4g64_ss", w_std=0.05),
    "mxfp4_staged": moe_inputs.MoEConfig(
        "mxfp4_staged", T=200, d=1024, E=6, k=2, F=512, act="bf16", wt="mxfp4",
        model="s_mxfp4_st", n_shared=1, w_std=0.05),
    "mxfp8_staged": moe_inputs.MoEConfig(
        "mxfp8_staged", T=1024, d=512, E=4, k=2, F=2048, act="bf16", wt="mxfp8",
        model="s_mxfp8_st", w_std=0.05),
    # MXFP8 tiles hold 128 token rows: groups of ~100 rows (one partial tile)
    # next to groups above 128 (a ragged second tile) ...
    "mxfp8_staged_ragged": moe_inputs.MoEConfig(
        "mxfp8_staged_ragged", T=300, d=512, E=6, k=2, F=1024, act="bf16", wt="mxfp8",
        model="s_mxfp8_sr", w_std=0.05),
    # ... and more gate/up tasks (32 M-tiles x 16 N-tiles) than blocks, so the
    # copy stream runs from one 128-row task into the next
    "mxfp8_staged_stream": moe_inputs.MoEConfig(
        "mxfp8_staged_stream", T=2048, d=256, E=4, k=2, F=4096, act="bf16", wt="mxfp8",
        model="s_mxfp8_ss", w_std=0.05),
    # int4 with K above 8192 on the GEMV (gate/up K = 9216, not a multiple of
    # 1024 times at most 8); down K = 512 also on the GEMV
    "int4_wide_gemv": moe_inputs.MoEConfig(
        "int4_wide_gemv", T=12, d=9216, E=4, k=2, F=512, act="bf16", wt="int4",
        model="s_int4_wg", n_shared=1, w_std=0.05),
}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


# ------------------------------------------------------------------ A1-A3

def _route(cfg, d, T=None):
    T = cfg.T if T is None else T
    shape = shape_of(cfg, T=T)
    logits = torch.empty(T, cfg.E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.k, dtype=torch.float32, device=DEV)
    moe.moe_route(shape, d["x"][:T], d["w_router"], d["b_router"], logits, idx, w)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _check_route(cfg, x, wr, br, L, idx, w, orc):
    ref = orc.router_logits(np_store(x), cfg.act, np_store(wr), np_store(br))
    scale = np.abs(ref).max() + 1e-30
    assert np.abs(L.astype(np.float64) - ref).max() / scale < 1e-5
    # top-k on the GPU's own logits must match bit for bit
    oi, ow = orc.topk(L.astype(np.float64), cfg.k)
    assert np.array_equal(idx, oi)
    np.testing.assert_allclose(w, ow, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-6)


# Router shapes for the 64 x 64-tile kernel (T*E >= 2^20, E >= 64): whole
# tiles and K chunks, and a ragged one (T not a multiple of 64, E = 200 with a
# partial last expert tile, d = 264: a K tail of 8 in the last chunk)
ROUTE_WIDE = {
    "route_wide": moe_inputs.MoEConfig("route_wide", T=4096, d=512, E=256, k=8, F=128, act="bf16",
                                       wt="bf16", model="s_route_wide"),
    "route_wide_ragged": moe_inputs.MoEConfig("route_wide_ragged", T=5300, d=264, E=200, k=6, F=128,
                                              act="bf16", wt="bf16", model="s_route_wr"),
    # logits and top-k in one launch (bf16, T*E >= 4096, E <= 16): a partial
    # last token tile (T = 1000), a partial expert tile (E = 12) and a K tail
    # (d = 264: 9 steps of 32 over 16 K ranges, some of them empty)
    "route_fused_ragged": moe_inputs.MoEConfig("route_fused_ragged", T=1000, d=264, E=12, k=3, F=128,
                                               act="bf16", wt="bf16", model="s_route_fr"),
}


@pytest.mark.parametrize("name", ["tiny_f32", "mixtral_decode", "mixtral_prefill",
                                  "fine_int4_decode", "stack4", "fine_int4_prefill"] + list(ROUTE_WIDE))
def test_route_parity(orc, name):
    cfg = ROUTE_WIDE[name] if name in ROUTE_WIDE else C[name]
    say(f"route parity {name}")
    x = moe_inputs.activations(cfg, 0)
    wr = moe_inputs.router_weights(cfg, 0, 0)
    br = moe_inputs.router_bias(cfg)
    d = {"x": x.to(DEV), "w_router": wr.to(DEV), "b_router": None if br is None else br.to(DEV)}
    L, idx, w = _route(cfg, d)
    _check_route(cfg, x, wr, br, L, idx, w, orc)


def test_route_ties_and_degenerate(orc):
    cfg = moe_inputs.MoEConfig("ties", T=70, d=64, E=256, k=8, F=128, act="f32", wt="f32",
                               model="ties")
    say("route ties E=256 k=8")
    x = torch.zeros(70, 64)
    x[1::2] = torch.randn(35, 64, generator=torch.Generator().manual_seed(1))
    wr = torch.randn(256, 64, generator=torch.Generator().manual_seed(2))
    wr[7] = wr[3]          # duplicate experts -> exact ties
    wr[200] = wr[3]
    d = {"x": x.to(DEV), "w_router": wr.to(DEV), "b_router": None}
    L, idx, w = _route(cfg, d)
    _check_route(cfg, x, wr, None, L, idx, w, orc)
    assert (idx[0::2] == np.arange(8)).all()    # all-equal logits -> experts 0..k-1
    # k = E
    cfg2 = cfg.replace(E=16, k=16)
    d2 = {"x": x.to(DEV), "w_router": wr[:16].contiguous().to(DEV), "b_router": None}
    L2, idx2, w2 = _route(cfg2, d2)
    _check_route(cfg2, x, wr[:16], None, L2, idx2, w2, orc)
    # the one-launch bf16 path (T*E >= 4096, E <= 16): exact ties between
    # duplicated router rows, all-zero tokens, and k = E
    for E3, k3 in ((16, 4), (16, 16)):
        cfg3 = moe_inputs.MoEConfig("ties_bf16", T=512, d=64, E=E3, k=k3, F=128, act="bf16", wt="bf16",
                                    model="ties")
        x3 = torch.zeros(512, 64)
        x3[1::2] = torch.randn(256, 64, generator=torch.Generator().manual_seed(3))
        x3 = x3.to(torch.bfloat16)
        wr3 = wr[:E3].clone()
        wr3[9] = wr3[3]
        d3 = {"x": x3.to(DEV), "w_router": wr3.to(DEV), "b_router": None}
        L3, idx3, w3 = _route(cfg3, d3)
        _check_route(cfg3, x3, wr3, None, L3, idx3, w3, orc)
        assert (idx3[0::2] == np.arange(k3)).all()
        assert (L3[1::2, 9] == L3[1::2, 3]).all()


# --------------------------------------------------------------------- A4

def _dispatch(idx, E, k):
    T = idx.shape[0] // k if idx.ndim == 1 else idx.shape[0]
    shape = moe.make_shape(T, 64, E, k, 64, "f32", "f32")
    ti = torch.from_numpy(np.ascontiguousarray(idx, np.int32).reshape(-1)).to(DEV)
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    perm = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device=DEV)
    inv = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device=DEV)
    moe.moe_dispatch(shape, ti, counts, offsets, perm, inv)
    torch.cuda.synchronize()
    return (counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy()[:T * k],
            inv.cpu().numpy()[:T * k])


@pytest.mark.parametrize("T,k,E,kind", [
    (16, 2, 8, "random"), (8, 2, 8, "random"), (4096, 2, 8, "zipf"), (64, 8, 256, "random"),
    (512, 6, 64, "random"), (1, 1, 1, "random"), (3, 4, 4, "random"), (1000, 3, 7, "one"),
    (2048, 16, 256, "random"), (5, 2, 200, "random"),
    # more than 32 groups of 64 per wave: the keys come in several batches
    (5000, 8, 256, "random"), (9000, 8, 64, "zipf"),
])
def test_dispatch_bit_exact(orc, T, k, E, kind):
    say(f"dispatch T={T} k={k} E={E} {kind}")
    rng = np.random.default_rng(T * 7 + E)
    if kind == "random":
        idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
    elif kind == "zipf":
        p = np.array(moe_inputs.zipf_targets(E))
        idx = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(T)], np.int32)
    else:   # every token on the same k experts
        idx = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    got = _dispatch(idx, E, k)
    ref = orc.dispatch(idx, E)
    for g, r, name in zip(got, ref, ("counts", "offsets", "perm", "inv")):
        assert np.array_equal(g, r), name


def test_dispatch_empty_and_invalid(orc):
    say("dispatch T=0 and out-of-range entries")
    c, o, p, i = _dispatch(np.zeros((0, 2), np.int32), 8, 2)
    assert (c == 0).all() and (o == 0).all()
    idx = np.array([[0, 1], [9, 2], [-1, 1]], np.int32)   # 9 and -1 are ignored
    c, o, p, i = _dispatch(idx, 8, 2)
    assert c.tolist() == [1, 2, 1, 0, 0, 0, 0, 0] and o[-1] == 4
    assert p[:4].tolist() == [0, 1, 5, 3]


# ------------------------------------------------------------ A5-A8 steps

def _steps(cfg, d, tau=0):
    """route -> dispatch -> expert_ffn -> combine through the C ABI."""
    T = cfg.T
    shape = shape_of(cfg, tau)
    logits = torch.empty(T, cfg.E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.k, dtype=torch.float32, device=DEV)
    moe.moe_route(shape, d["x"], d["w_router"], d["b_router"], logits, idx, w)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(T * cfg.k, dtype=torch.int32, device=DEV)
    inv = torch.empty(T * cfg.k, dtype=torch.int32, device=DEV)
    moe.moe_dispatch(shape, idx, counts, offsets, perm, inv)
    yp = torch.empty(T * cfg.k, cfg.d, dtype=torch.float32, device=DEV)
    ys = torch.empty(T, cfg.d, dtype=torch.float32, device=DEV) if cfg.n_shared else None
    ws = torch.empty(moe.moe_workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    moe.moe_expert_ffn(shape, d["x"], weights_struct(d), counts, offsets, perm, yp, ys, ws)
    y = torch.empty(T, cfg.d, dtype=act_dtype(cfg), device=DEV)
    moe.moe_combine(shape, yp, inv, w, ys, None, y)
    torch.cuda.synchronize()
    h = lambda t: None if t is None else t.cpu().numpy()
    return dict(logits=h(logits), idx=h(idx), w=h(w), counts=h(counts), offsets=h(offsets),
                perm=h(perm), inv=h(inv), yp=h(yp), ys=h(ys), y=np_f64(y))


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("tau", [0, -1])
def test_steps_parity(orc, name, tau):
    cfg = SMALL[name]
    if tau == -1 and cfg.wt not in ("bf16", "int4", "mxfp4", "mxfp8"):
        pytest.skip("tau only selects kernels for bf16, int4-g128 and MX weights")
    say(f"steps parity {name} tau={tau}")
    d = device_inputs(cfg)
    g = _steps(cfg, d, tau)
    W, S = oracle_weights(d)
    x = np_store(d["x"])
    # route: bit-exact top-k on the GPU's logits
    oi, ow = orc.topk(g["logits"].astype(np.float64), cfg.k)
    assert np.array_equal(g["idx"], oi)
    np.testing.assert_allclose(g["w"], ow, rtol=1e-6, atol=1e-7)
    # dispatch: bit-exact on the GPU's indices
    rc = orc.dispatch(g["idx"], cfg.E)
    for a, b in zip((g["counts"], g["offsets"], g["perm"], g["inv"]), rc):
        assert np.array_equal(a, b)
    # expert FFN rows
    yp_ref = orc.expert_ffn(x, cfg.act, cfg.wt, W, *rc[:3], cfg.k)
    err = tokenwise_rel(g["yp"], yp_ref)
    say(f"  y_perm max rel {err.max():.3g}")
    assert err.max() < TOL[cfg.wt]
    if cfg.n_shared:
        ys_ref = orc.shared_ffn(x, cfg.act, cfg.wt, S)
        assert tokenwise_rel(g["ys"], ys_ref).max() < TOL[cfg.wt]
    # combine on the GPU's own y_perm: only fp32 summation order differs
    y_ref = orc.combine(g["yp"].astype(np.float64), g["inv"], g["w"].astype(np.float64), cfg.k,
                        ys=None if g["ys"] is None else g["ys"].astype(np.float64))
    cmb_tol = 1e-6 if cfg.act == "f32" else 8e-3   # bf16 output rounding
    assert tokenwise_rel(g["y"], y_ref).max() < cmb_tol


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_end_to_end_small(orc, name):
    cfg = SMALL[name]
    say(f"layer end-to-end {name}")
    d = device_inputs(cfg)
    y, counts, idx = run_layer(cfg, d)
    W, S = oracle_weights(d)
    x = np_store(d["x"])
    wr, br = np_store(d["w_router"]), np_store(d["b_router"])
    y_o, idx_o, _, lg_o = orc.layer_forward(x, cfg.act, cfg.wt, cfg.k, wr, br, W, S)
    gi = idx.cpu().numpy()
    flips = check_routing_with_flips(gi, idx_o, lg_o, cfg.k)
    y_f, _, _, _ = orc.layer_forward(x, cfg.act, cfg.wt, cfg.k, wr, br, W, S, forced_idx=gi)
    err = tokenwise_rel(np_f64(y), y_f)
    say(f"  max rel {err.max():.3g} flips {flips}")
    assert err.max() < TOL[cfg.wt]
    assert np.array_equal(counts.cpu().numpy(), np.bincount(gi.ravel(), minlength=cfg.E))


def test_pack_int4_tiled_layout():
    """moe_pack_int4_tiled against the tiled layout as moe.h defines it, written
    out piece by piece on the host; ragged matrix count, K of 2 and 3 groups."""
    for n_mats, N, K in ((3, 48, 256), (1, 16, 384), (2, 128, 1024)):
        say(f"pack int4 tiled n_mats={n_mats} N={N} K={K}")
        g = torch.Generator().manual_seed(N + K)
        src = torch.randint(0, 256, (n_mats, N, K // 2), dtype=torch.uint8, generator=g)
        dst = torch.full_like(src, 0xA5).to(DEV)
        moe.moe_pack_int4_tiled(src.to(DEV), dst, n_mats, N, K)
        torch.cuda.synchronize()
        got = dst.cpu().numpy().reshape(n_mats, -1)
        a = src.numpy()
        want = np.empty_like(got)
        NG = K // 128
        for m in range(n_mats):
            for s_ in range(N // 16):
                for gi in range(NG):
                    for q in range(4):
                        for r in range(16):
                            o = ((s_ * NG + gi) * 64 + 16 * q + r) * 16
                            want[m, o:o + 16] = a[m, 16 * s_ + r, 64 * gi + 16 * q:64 * gi + 16 * q + 16]
        assert np.array_equal(got, want)
    # nothing to do for zero matrices
    moe.moe_pack_int4_tiled(None, None, 0, 16, 128)


def test_pack_mxfp8_tiled_layout():
    """moe_pack_mxfp8_tiled against the tiled layout as moe.h defines it,
    written out piece by piece on the host."""
    for n_mats, N, K in ((3, 48, 256), (1, 16, 384), (2, 128, 1024)):
        say(f"pack mxfp8 tiled n_mats={n_mats} N={N} K={K}")
        g = torch.Generator().manual_seed(N + K + 1)
        src = torch.randint(0, 256, (n_mats, N, K), dtype=torch.uint8, generator=g)
        dst = torch.full_like(src, 0xA5).to(DEV)
        moe.moe_pack_mxfp8_tiled(src.to(DEV), dst, n_mats, N, K)
        torch.cuda.synchronize()
        got = dst.cpu().numpy().reshape(n_mats, -1)
        a = src.numpy()
        want = np.empty_like(got)
        NG = K // 128
        for m in range(n_mats):
            for s_ in range(N // 16):
                for gi in range(NG):
                    for w in range(2):
                        for q in range(4):
                            for r in range(16):
                                o = ((s_ * NG + gi) * 128 + 64 * w + 16 * q + r) * 16
                                c = 128 * gi + 32 * q + 16 * w
                                want[m, o:o + 16] = a[m, 16 * s_ + r, c:c + 16]
        assert np.array_equal(got, want)
    moe.moe_pack_mxfp8_tiled(None, None, 0, 16, 128)


TILED = ["int4_mfma_multipass", "int4_mfma_wide_k", "int4_mfma_many", "mxfp4_skinny", "mxfp4_wide_k",
         "mxfp8_skinny", "mxfp8_skinny_longk"]


@pytest.mark.parametrize("name", TILED)
def test_layer_int4_tiled(orc, name):
    """Tiled codes (int4, MXFP4 or MXFP8): the layer against the oracle (which
    reads the row-major codes), and bit-identical to the row-major run (same
    arithmetic)."""
    cfg = SMALL[name]
    say(f"layer {cfg.wt} tiled {name}")
    d = device_inputs(cfg)
    y, counts, idx = run_layer(cfg, tiled_inputs(d, cfg.wt), wt=f"{cfg.wt}_tiled")
    W, S = oracle_weights(d)
    x = np_store(d["x"])
    wr, br = np_store(d["w_router"]), np_store(d["b_router"])
    gi = idx.cpu().numpy()
    y_f, idx_o, _, lg_o = orc.layer_forward(x, cfg.act, cfg.wt, cfg.k, wr, br, W, S)
    flips = check_routing_with_flips(gi, idx_o, lg_o, cfg.k)
    y_f, _, _, _ = orc.layer_forward(x, cfg.act, cfg.wt, cfg.k, wr, br, W, S, forced_idx=gi)
    err = tokenwise_rel(np_f64(y), y_f)
    say(f"  max rel {err.max():.3g} flips {flips}")
    assert err.max() < TOL[cfg.wt]
    # row-major codes on the same skinny kernels (tau < 0: no group on the
    # dequantising GEMM): the same arithmetic, bit for bit
    y_rm, _, idx_rm = run_layer(cfg, d, tau=-1)
    assert torch.equal(idx, idx_rm) and torch.equal(y, y_rm)


@pytest.mark.parametrize("name", ["mxfp4_skinny", "mxfp8_skinny"])
def test_tiled_edge_cases(orc, name):
    """Tiled MX codes with a shared expert: T = 0 (counts cleared, nothing
    else launched with work), T = 1, and every token on the same k experts
    (groups of all T rows next to empty ones)."""
    cfg = SMALL[name]
    wt = f"{cfg.wt}_tiled"
    say(f"tiled edge cases {name}")
    d = device_inputs(cfg)
    t = tiled_inputs(d, cfg.wt)
    W, S = oracle_weights(d)
    wr = np_store(d["w_router"])
    shape = shape_of(cfg, T=0, wt=wt)
    ws = torch.empty(max(256, moe.moe_workspace_bytes(shape)), dtype=torch.uint8, device=DEV)
    counts = torch.full((cfg.E,), 5, dtype=torch.int32, device=DEV)
    moe.moe_layer_forward(shape, d["x"], d["w_router"], d["b_router"], weights_struct(t), None, d["x"],
                          counts, None, ws)
    torch.cuda.synchronize()
    assert (counts.cpu() == 0).all()
    b = torch.zeros(cfg.E)
    for j in range(cfg.k):
        b[j] = 1e3 - 100 * j
    br = None if d["b_router"] is None else np_store(d["b_router"])
    for T, bias in ((1, None), (cfg.T, b)):
        dd = t if bias is None else dict(t, b_router=bias.to(DEV))
        y, c, i = run_layer(cfg, dd, x=d["x"][:T].contiguous(), wt=wt)
        if bias is not None:
            assert c.cpu().tolist()[:cfg.k] == [T] * cfg.k and int(c.sum()) == T * cfg.k
        y_f, _, _, _ = orc.layer_forward(np_store(d["x"][:T]), cfg.act, cfg.wt, cfg.k, wr,
                                         br if bias is None else bias.numpy(), W, S,
                                         forced_idx=i.cpu().numpy())
        err = tokenwise_rel(np_f64(y), y_f)
        say(f"  T={T} counts {c.cpu().tolist()} max rel {err.max():.3g}")
        assert err.max() < TOL[cfg.wt]


@pytest.mark.parametrize("name,tau", [("bf16_small_split", 0), ("bf16_prefill_ragged", 0),
                                      ("bf16_prefill_stream", 0), ("bf16_prefill_ragged", 16)])
def test_layer_matches_steps_bitwise(name, tau):
    """Inside moe_layer_forward the dispatch kernel also writes the grouped
    GEMM's tile lists; moe_expert_ffn builds them with its own launch.  The
    lists are the same, so the layer equals the four steps bit for bit, with
    only 64-row tiles (bf16_small_split), both lists (bf16_prefill_ragged, and
    with an explicit tau) and only 256-row tiles (bf16_prefill_stream)."""
    cfg = SMALL[name]
    say(f"layer vs steps bitwise {name} tau={tau}")
    d = device_inputs(cfg)
    y, counts, idx = run_layer(cfg, d, tau=tau)
    g = _steps(cfg, d, tau=tau)
    assert np.array_equal(idx.cpu().numpy(), g["idx"])
    assert np.array_equal(counts.cpu().numpy(), g["counts"])
    assert np.array_equal(np_f64(y), g["y"])


def test_residual_and_determinism(orc):
    cfg = SMALL["bf16_prefill_ragged"]
    say("residual + determinism")
    d = device_inputs(cfg)
    res = torch.randn(cfg.T, cfg.d, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    y1, c1, i1 = run_layer(cfg, d, residual=res)
    y2, c2, i2 = run_layer(cfg, d, residual=res)
    assert torch.equal(y1, y2) and torch.equal(i1, i2) and torch.equal(c1, c2)
    W, S = oracle_weights(d)
    y_f, _, _, _ = orc.layer_forward(np_store(d["x"]), cfg.act, cfg.wt, cfg.k, np_store(d["w_router"]),
                                     None, W, S, residual=np_store(res), forced_idx=i1.cpu().numpy())
    assert tokenwise_rel(np_f64(y1), y_f).max() < TOL["bf16"]


def test_tau_does_not_change_routing():
    cfg = SMALL["bf16_prefill_ragged"]
    say("tau invariance")
    d = device_inputs(cfg)
    ref = None
    for tau in (-1, 0, 1, 50, 10000):
        g = _steps(cfg, d, tau)
        if ref is None:
            ref = g
            continue
        for n in ("idx", "counts", "offsets", "perm", "inv"):
            assert np.array_equal(g[n], ref[n]), (tau, n)
        assert tokenwise_rel(g["y"], ref["y"]).max() < 1e-2


def test_edge_cases(orc):
    """T = 0, T = 1, k = E, and all tokens on one expert (maximal imbalance)."""
    say("edge cases")
    base = SMALL["bf16_prefill_ragged"]
    d = device_inputs(base)
    # T = 0: nothing launched except the zero histogram
    shape = shape_of(base, T=0)
    ws = torch.empty(moe.moe_workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    counts = torch.full((base.E,), 5, dtype=torch.int32, device=DEV)
    moe.moe_layer_forward(shape, d["x"], d["w_router"], None, weights_struct(d), None, d["x"],
                          counts, None, ws)
    torch.cuda.synchronize()
    assert (counts.cpu() == 0).all()
    W, S = oracle_weights(d)
    wr = np_store(d["w_router"])
    for T in (1, 17):
        y, c, i = run_layer(base, d, x=d["x"][:T].contiguous())
        y_f, _, _, _ = orc.layer_forward(np_store(d["x"][:T]), "bf16", "bf16", base.k, wr, None, W,
                                         forced_idx=i.cpu().numpy())
        assert tokenwise_rel(np_f64(y), y_f).max() < TOL["bf16"]
    # k = E
    cfgE = base.replace(k=base.E, T=40)
    y, c, i = run_layer(cfgE, d, x=d["x"][:40].contiguous())
    assert (c.cpu() == 40).all()
    y_f, _, _, _ = orc.layer_forward(np_store(d["x"][:40]), "bf16", "bf16", cfgE.k, wr, None, W,
                                     forced_idx=i.cpu().numpy())
    assert tokenwise_rel(np_f64(y), y_f).max() < TOL["bf16"]
    # one expert takes every token: a large bias on experts 0 and 1
    b = torch.zeros(base.E)
    b[0], b[1] = 1e3, 5e2
    d1 = dict(d, b_router=b.to(DEV))
    for tau in (0, -1):
        y, c, i = run_layer(base, d1, tau=tau)
        assert c.cpu().tolist()[:2] == [base.T, base.T]
        y_f, _, _, _ = orc.layer_forward(np_store(d["x"]), "bf16", "bf16", base.k, wr, b.numpy(), W,
                                         forced_idx=i.cpu().numpy())
        assert tokenwise_rel(np_f64(y), y_f).max() < TOL["bf16"]


def test_groups_straddling_tau(orc):
    """Expert groups of tau-1, tau and tau+1 rows take different kernels."""
    say("groups straddling tau")
    cfg = SMALL["bf16_prefill_ragged"]
    d = device_inputs(cfg)
    T, tau = 17, 16
    x = d["x"][:T].contiguous()
    # bias chosen so expert 0 gets all 17 tokens and k=2 picks the runner-up per token
    b = torch.zeros(cfg.E)
    b[0] = 1e3
    d1 = dict(d, b_router=b.to(DEV))
    W, S = oracle_weights(d)
    for TT in (tau - 1, tau, tau + 1):
        y, c, i = run_layer(cfg, d1, tau=tau, x=x[:TT].contiguous())
        assert int(c[0]) == TT
        y_f, _, _, _ = orc.layer_forward(np_store(x[:TT]), "bf16", "bf16", cfg.k, np_store(d["w_router"]),
                                         b.numpy(), W, forced_idx=i.cpu().numpy())
        assert tokenwise_rel(np_f64(y), y_f).max() < TOL["bf16"]


@pytest.mark.parametrize("name", ["bf16_prefill_ragged", "bf16_prefill_fast"])
def test_mfma_tile_boundaries(orc, name):
    """Expert groups around the M-tile sizes: 64-row tiles for groups of at
    most 128 rows (one or two tiles), 256-row tiles (ragged tail) above.  With
    K a multiple of 64 (gate/up of both configs, down of the second) a ragged
    256-row tile splits its 32-row fragments between the two wave groups:
    129 rows (3 + 2 fragments), 200 (4 + 3), 257 (a last tile of one row:
    1 + 0), 300 (1 + 1), 330 (2 + 1), 353 (2 + 2), 384 (2 + 2)."""
    say(f"mfma tile boundaries {name}")
    cfg = SMALL[name]
    d = device_inputs(cfg)
    b = torch.zeros(cfg.E)
    b[0] = 1e3          # expert 0 takes every token; the runner-ups spread the rest
    d1 = dict(d, b_router=b.to(DEV))
    W, S = oracle_weights(d)
    for TT in (64, 65, 128, 129, 200, 257, 300, 330, 353, 384):
        x = d["x"][:TT].contiguous()
        y, c, i = run_layer(cfg, d1, tau=16, x=x)
        assert int(c[0]) == TT
        y_f, _, _, _ = orc.layer_forward(np_store(x), "bf16", "bf16", cfg.k, np_store(d["w_router"]),
                                         b.numpy(), W, forced_idx=i.cpu().numpy())
        err = tokenwise_rel(np_f64(y), y_f).max()
        say(f"  T={TT} counts {c.cpu().tolist()} max rel {err:.3g}")
        assert err < TOL["bf16"]


# Default tile lists by the mean group T*k/E (bf16 weights, tau = 0):
# at most 64 rows (and small experts) -> every group on 64-row tiles, a group
# above 128 rows as several of them; at least 512 rows -> every group on
# 256-row tiles, small groups as ragged ones; a mean group of twice the
# streaming range or more also sends groups of a few rows to the tiles.
SINGLE_LIST = {
    "small_only": moe_inputs.MoEConfig(
        "small_only", T=256, d=256, E=16, k=4, F=384, act="bf16", wt="bf16",
        model="s_small_only", w_std=0.05),
    "big_only": moe_inputs.MoEConfig(
        "big_only", T=1024, d=320, E=4, k=2, F=384, act="bf16", wt="bf16",
        model="s_big_only", w_std=0.05),
    # 64-row tiles with a K tail in both passes (d = 264 and F = 200: the last
    # K pair holds one 8-element chunk) and N not a multiple of the tile width
    "small_only_ktail": moe_inputs.MoEConfig(
        "small_only_ktail", T=256, d=264, E=16, k=4, F=200, act="bf16", wt="bf16",
        model="s_small_kt", w_std=0.05),
}


@pytest.mark.parametrize("name", list(SINGLE_LIST))
def test_single_tile_list(orc, name):
    """Layer parity where the default picks one tile list.  64-row list:
    natural routing (groups of ~64 rows), then one expert taking every token
    of batches of 129, 200 and 256 tokens (three or four 64-row tiles of one
    expert).  256-row list: natural routing (~512 rows per expert), then a
    negative bias that leaves one expert fewer and fewer rows (a group below
    128 rows in one ragged 256-row tile)."""
    cfg = SINGLE_LIST[name]
    say(f"single tile list {name}")
    d = device_inputs(cfg)
    W, S = oracle_weights(d)
    wr = np_store(d["w_router"])
    cases = [(cfg.T, np.zeros(cfg.E, np.float32))]
    if name.startswith("small_only"):
        for TT in (129, 200, 256):
            b = np.zeros(cfg.E, np.float32)
            b[0] = 1e3
            cases.append((TT, b))
    else:
        for lo in (1.5, 3.0, 5.0):
            b = np.zeros(cfg.E, np.float32)
            b[3] = -lo
            cases.append((cfg.T, b))
    seen = []
    for TT, b in cases:
        xs = d["x"][:TT].contiguous()
        y, c, i = run_layer(cfg, dict(d, b_router=torch.from_numpy(b).to(DEV)), x=xs)
        gi = i.cpu().numpy()
        y_f, _, _, _ = orc.layer_forward(np_store(xs), "bf16", "bf16", cfg.k, wr, b, W, forced_idx=gi)
        err = tokenwise_rel(np_f64(y), y_f).max()
        cl = c.cpu().tolist()
        seen.append(cl)
        say(f"  T={TT} counts {cl} max rel {err:.3g}")
        assert err < TOL["bf16"]
        assert np.array_equal(np.asarray(cl), np.bincount(gi.ravel(), minlength=cfg.E))
    if name.startswith("small_only"):
        assert max(seen[0]) <= 128 and [c[0] for c in seen[1:]] == [129, 200, 256]
    else:
        assert min(seen[0]) > 128 and min(c[3] for c in seen[1:]) < 128


@pytest.mark.parametrize("name", ["int4_dq", "mxfp4_rem", "mxfp8_rem"])
def test_int4_groups_on_both_sides_of_tau(orc, name):
    """int4-g128 and MX weights with the default tau (32 rows) and a mean
    group below twice that: groups of at most 32 rows on the skinny
    matrix-core kernel, larger ones on the dequantising GEMM, in one call --
    expert 0 takes every token (a bias), the runner-ups spread over the rest."""
    cfg = SMALL[name]
    say(f"{name}: groups on both sides of tau")
    d = device_inputs(cfg)
    W, S = oracle_weights(d)
    wr = np_store(d["w_router"])
    b = np.zeros(cfg.E, np.float32)
    b[0] = 1e3
    for TT in (40, 90):
        xs = d["x"][:TT].contiguous()
        y, c, i = run_layer(cfg, dict(d, b_router=torch.from_numpy(b).to(DEV)), x=xs)
        cl = c.cpu().tolist()
        y_f, _, _, _ = orc.layer_forward(np_store(xs), "bf16", cfg.wt, cfg.k, wr, b, W, S,
                                         forced_idx=i.cpu().numpy())
        err = tokenwise_rel(np_f64(y), y_f).max()
        say(f"  T={TT} counts {cl} max rel {err:.3g}")
        assert cl[0] == TT and min(cl[1:]) <= 32 and TT * cfg.k < 2 * 32 * cfg.E
        assert err < TOL[cfg.wt]


@pytest.mark.parametrize("name", ["int4_dq", "mxfp4_rem", "mxfp8_rem"])
def test_int4_dq_remainders(orc, name):
    """Weights with every group on the dequantising GEMM (T*k >= 64 E).
    int4-g128: a group's last partial 128-row tile of at most 16 rows runs on
    the skinny matrix-core kernel instead, a longer one on the GEMM; MX
    weights keep every row on the GEMM.  Hand-made groups through
    moe_expert_ffn: remainders 0, 1, 8, 12, 16 and 17, whole groups of 1 to 17
    rows, an empty expert, and the shared expert over T = 136 (a remainder of
    8 rows) and T = 150 (22 rows)."""
    cfg = SMALL[name]
    say(f"{name}: dq remainders on the skinny kernel")
    d = device_inputs(cfg)
    W, S = oracle_weights(d)
    cases = {150: ([140, 16, 0, 144], [145, 17, 9, 129], [256, 1, 2, 41]), 136: ([136, 8, 0, 128],)}
    for T, mixes in cases.items():
        x = d["x"][:T].contiguous()
        xs = np_store(x)
        shape = shape_of(cfg, 0, T=T)
        ys_ref = orc.shared_ffn(xs, "bf16", cfg.wt, S)
        ws = torch.empty(moe.moe_workspace_bytes(shape), dtype=torch.uint8, device=DEV)
        for cs in mixes:
            assert sum(cs) == T * cfg.k
            off = np.concatenate([[0], np.cumsum(cs)]).astype(np.int32)
            perm = np.random.default_rng(sum(cs) + cs[0]).permutation(T * cfg.k).astype(np.int32)
            yp = torch.empty(T * cfg.k, cfg.d, dtype=torch.float32, device=DEV)
            ys = torch.empty(T, cfg.d, dtype=torch.float32, device=DEV)
            moe.moe_expert_ffn(shape, x, weights_struct(d), torch.tensor(cs, dtype=torch.int32, device=DEV),
                               torch.from_numpy(off).to(DEV), torch.from_numpy(perm).to(DEV), yp, ys, ws)
            torch.cuda.synchronize()
            ref = orc.expert_ffn(xs, "bf16", cfg.wt, W, np.array(cs, np.int32), off, perm, cfg.k)
            e1 = tokenwise_rel(yp.cpu().numpy(), ref).max()
            e2 = tokenwise_rel(ys.cpu().numpy(), ys_ref).max()
            say(f"  T={T} counts {cs}: y_perm max rel {e1:.3g}, shared {e2:.3g}")
            assert e1 < TOL[cfg.wt] and e2 < TOL[cfg.wt]


def test_rmsnorm_parity(orc):
    say("rmsnorm")
    for act in ("f32", "bf16"):
        h = torch.randn(33, 2048, generator=torch.Generator().manual_seed(3)) * 3
        h = h.to(torch.float32 if act == "f32" else torch.bfloat16)
        g = torch.linspace(0.5, 1.5, 2048)
        out = torch.empty_like(h).to(DEV)
        shape = moe.make_shape(33, 2048, 8, 2, 64, act, act)
        moe.moe_rmsnorm(shape, h.to(DEV), g.to(DEV), 1e-6, out)
        torch.cuda.synchronize()
        ref = orc.rmsnorm(np_store(h), act, g.numpy(), 1e-6)
        tol = 1e-6 if act == "f32" else 8e-3
        assert tokenwise_rel(np_f64(out), ref).max() < tol


def test_read_ceiling_reads_every_word():
    # the measurement helper folds every 32-bit word into the sink: XOR check
    say("read ceiling helper")
    g = torch.Generator().manual_seed(5)
    for n_words in (4, 4 * 1000 + 4, 1 << 22):
        h = torch.randint(-2**31, 2**31 - 1, (n_words,), generator=g, dtype=torch.int64).to(torch.int32)
        buf = h.to(DEV)
        sink = torch.zeros(1, dtype=torch.int32, device=DEV)
        moe.measure.moe_read_ceiling(buf, n_words * 4, sink)
        torch.cuda.synchronize()
        ref = np.bitwise_xor.reduce(h.numpy().view(np.uint32))
        assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(ref)


def test_mfma_ceiling_runs():
    """The matrix-core ceiling helper: every wave writes its sum (the products
    of its constant fragments), the clock counters advance, the flop count is
    the launch's."""
    sink = torch.full((4096,), float("nan"), dtype=torch.float32, device=DEV)
    clk = torch.zeros(2, dtype=torch.int64, device=DEV)
    flops = moe.measure.moe_mfma_ceiling(16, sink, 4096 * 4, clk)
    torch.cuda.synchronize()
    n = flops // (8 * 16 * 8 * 32768)
    s = sink[: n * 8].cpu()
    assert torch.isfinite(s).all()
    cyc, ticks = clk.cpu().tolist()
    assert cyc > 0 and ticks >= 0


def test_skinny_groups_exercised(orc):
    """The skinny configs really have the group sizes their comments claim."""
    for name, check in [("bf16_skinny_mix", lambda c: ((c > 8) & (c <= 16)).any() and (c <= 8).any()
                         and (c <= 16).all()),
                        ("bf16_skinny2", lambda c: ((c > 16) & (c <= 32)).any() and (c <= 16).any()
                         and (c <= 32).all()),
                        ("bf16_skinny2_mix", lambda c: ((c > 32) & (c <= 48)).any() and (c <= 48).all()),
                        ("bf16_skinny4", lambda c: (c == 64).any() and (c > 48).all() and (c <= 64).all()),
                        ("bf16_skinny4_mix", lambda c: (c > 64).any() and ((c > 48) & (c <= 64)).any())]:
        cfg = SMALL[name]
        d = device_inputs(cfg)
        _, counts, _ = run_layer(cfg, d)
        c = counts.cpu().numpy()
        say(f"  {name} counts {c.tolist()}")
        assert check(c), name


SKINNY_TAU = [
    # two token tiles with a half last weight tile: F = 1616 (N % 32 == 16 in
    # gate/up); the default tau drops to 16 because the down pass (K = 1616)
    # cannot use the kernel, which then runs on the GEMV
    (moe_inputs.MoEConfig("bf16_skinny2_ragged", T=56, d=1024, E=6, k=2, F=1616, act="bf16",
                          wt="bf16", model="s_bf16_sk2r", w_std=0.05), 32, 17, 32),
    # three and four token tiles (16-row gate/up items) with short rows, where
    # the default tau stops the kernel at 32 rows
    (SMALL["bf16_skinny2_mix"], 64, 33, 48),
    (SMALL["bf16_skinny4"], 64, 49, 64),
    (SMALL["bf16_skinny4_mix"], 64, 49, 64),
]


@pytest.mark.parametrize("cfg,tau,lo,hi", SKINNY_TAU, ids=[c[0].name for c in SKINNY_TAU])
def test_skinny_explicit_tau(orc, cfg, tau, lo, hi):
    """Layer parity with an explicit tau that sends the largest group below the
    MFMA tiles (lo..hi rows) to the skinny kernel's widest variant."""
    d = device_inputs(cfg)
    y, counts, idx = run_layer(cfg, d, tau=tau)
    c = counts.cpu().numpy()
    say(f"  {cfg.name} tau {tau} counts {c.tolist()}")
    small = c[c <= tau]
    assert small.size and lo <= small.max() <= hi
    W, S = oracle_weights(d)
    x = np_store(d["x"])
    wr, br = np_store(d["w_router"]), np_store(d["b_router"])
    gi = idx.cpu().numpy()
    y_f, _, _, _ = orc.layer_forward(x, cfg.act, cfg.wt, cfg.k, wr, br, W, S, forced_idx=gi)
    err = tokenwise_rel(np_f64(y), y_f)
    say(f"  max rel {err.max():.3g}")
    assert err.max() < TOL[cfg.wt]


FUSED_ROUTE = [  # (T, E, k, act, d): decode batches routed, ranked and dispatched by one kernel
    (1, 8, 2, "bf16", 4096), (5, 8, 2, "bf16", 1024), (8, 8, 8, "bf16", 512), (4, 16, 3, "bf16", 2056),
    (3, 13, 13, "f32", 136), (2, 5, 1, "f32", 64), (8, 7, 4, "bf16", 6144),
]


@pytest.mark.parametrize("T,E,k,act,d", FUSED_ROUTE, ids=[f"T{c[0]}E{c[1]}k{c[2]}{c[3]}d{c[4]}" for c in FUSED_ROUTE])
def test_decode_fused_routing(orc, T, E, k, act, d):
    """moe_layer_forward on decode batches, where one kernel computes the
    router logits, the top-k and the dispatch: expert choices against the
    oracle's (flip rule), usage counts, outputs on the GPU's choice; router
    rows 0 and 2 are equal, so every token has an exact tie between them."""
    cfg = moe_inputs.MoEConfig(f"fused_T{T}E{E}k{k}", T=T, d=d, E=E, k=k, F=256, act=act, wt=act,
                               model=f"s_fused_{E}_{d}", w_std=0.05)
    d_ = device_inputs(cfg)
    wr = d_["w_router"].clone()
    if E > 2:
        wr[2] = wr[0]
    d_["w_router"] = wr.contiguous()
    y, counts, idx = run_layer(cfg, d_)
    gi = idx.cpu().numpy()
    W, S = oracle_weights(d_)
    x = np_store(d_["x"])
    y_o, idx_o, _, lg_o = orc.layer_forward(x, cfg.act, cfg.wt, k, np_store(wr), None, W, S)
    flips = check_routing_with_flips(gi, idx_o, lg_o, k)
    assert np.array_equal(counts.cpu().numpy(), np.bincount(gi.ravel(), minlength=E))
    if E > 2:
        # the tie between experts 0 and 2 resolves to the lower index
        for t in range(T):
            row = gi[t].tolist()
            if 2 in row:
                assert 0 in row and row.index(0) < row.index(2)
    y_f, _, _, _ = orc.layer_forward(x, cfg.act, cfg.wt, k, np_store(wr), None, W, S, forced_idx=gi)
    err = tokenwise_rel(np_f64(y), y_f)
    say(f"  fused routing T={T} E={E} k={k}: max rel {err.max():.3g} flips {flips}")
    assert err.max() < TOL[cfg.wt]
