// extern "C" entry points of libmoe.so: argument validation, workspace carving
// and the launch sequence of the layer.  Declared and documented in moe.h.
//
// Conventions follow [P4] "Colibri：轻量级MoE推理引擎的C语言实践" §3.3 (int status,
// negative on error, caller-provided message buffer) and §3.2 (no allocation
// during inference); the fixed scratch budget computed up front follows [P3]
// (wzjinhao.cn) §2.3.  Validation runs before any HIP call, so a rejected call
// has enqueued nothing.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"
#include "plan.h"

#include <algorithm>
#include <atomic>
#include "moe.h"

using namespace moe;

namespace {

constexpr int kDefaultTau = 16;
constexpr size_t kAlign = 256;

int fail(char* err, size_t len, int code, const char* fmt, ...) {
    if (err && len > 0) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(err, len, fmt, ap);
        va_end(ap);
    }
    return code;
}

// MOE_DEBUG_SYNC is read once per process (a benign race: every reader
// computes the same value)
bool debug_sync() {
    static std::atomic<int> v{-1};
    int r = v.load(std::memory_order_relaxed);
    if (r < 0) {
        const char* e = getenv("MOE_DEBUG_SYNC");
        r = (e && e[0] && e[0] != '0') ? 1 : 0;
        v.store(r, std::memory_order_relaxed);
    }
    return r == 1;
}

int hip_check(hipError_t e, hipStream_t s, const char* what, char* err, size_t len) {
    if (e != hipSuccess)
        return fail(err, len, MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
    if (debug_sync()) {
        e = hipStreamSynchronize(s);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess)
            return fail(err, len, MOE_EHIP, "%s (MOE_DEBUG_SYNC): %s", what, hipGetErrorString(e));
    }
    return MOE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define NEED_PTR(p, name)                                                                 \
    do {                                                                                  \
        if (!(p)) return fail(err, err_len, MOE_EINVAL, "%s is NULL", name);              \
        if (!aligned16(p)) return fail(err, err_len, MOE_EINVAL, "%s is not 16-byte aligned", name); \
    } while (0)
#define OPT_PTR(p, name)                                                                  \
    do {                                                                                  \
        if ((p) && !aligned16(p))                                                         \
            return fail(err, err_len, MOE_EINVAL, "%s is not 16-byte aligned", name);      \
    } while (0)

int check_shape(const moe_shape* s, char* err, size_t err_len) {
    if (!s) return fail(err, err_len, MOE_EINVAL, "shape is NULL");
    if (s->T < 0 || s->T > (1 << 24)) return fail(err, err_len, MOE_EINVAL, "T=%d out of range [0, 2^24]", s->T);
    if (s->E < 1 || s->E > 256) return fail(err, err_len, MOE_EINVAL, "E=%d out of range [1, 256]", s->E);
    if (s->k < 1 || s->k > s->E || s->k > 16)
        return fail(err, err_len, MOE_EINVAL, "k=%d must satisfy 1 <= k <= min(E, 16) (E=%d)", s->k, s->E);
    if (s->d < 8 || s->d % 8) return fail(err, err_len, MOE_EINVAL, "d=%d must be a positive multiple of 8", s->d);
    if (s->F < 8 || s->F % 8) return fail(err, err_len, MOE_EINVAL, "F=%d must be a positive multiple of 8", s->F);
    if (s->n_shared != 0 && s->n_shared != 1)
        return fail(err, err_len, MOE_EINVAL, "n_shared=%d must be 0 or 1", s->n_shared);
    if (s->act != MOE_F32 && s->act != MOE_BF16)
        return fail(err, err_len, MOE_EINVAL, "act=%d is not MOE_F32 or MOE_BF16", s->act);
    if (s->wt < MOE_F32 || s->wt > MOE_MXFP8_TILED)
        return fail(err, err_len, MOE_EINVAL, "wt=%d is not a moe_dtype", s->wt);
    const bool int4 = s->wt == MOE_INT4_G128 || s->wt == MOE_INT4_G128_TILED;
    const bool quant = s->wt >= MOE_INT4_G128;
    if (int4 && (s->d % 128 || s->F % 128))
        return fail(err, err_len, MOE_EINVAL, "int4-g128 weights need d and F multiples of 128 (d=%d F=%d)",
                    s->d, s->F);
    if (quant && !int4 && (s->d % 64 || s->F % 64))
        return fail(err, err_len, MOE_EINVAL, "int4-g64 and MX weights need d and F multiples of 64 (d=%d F=%d)",
                    s->d, s->F);
    const bool ok_combo = (s->act == MOE_F32 && s->wt == MOE_F32) ||
                          (s->act == MOE_BF16 && (s->wt == MOE_BF16 || quant));
    if (!ok_combo)
        return fail(err, err_len, MOE_EUNSUPPORTED, "activation dtype %d with weight dtype %d is not built",
                    s->act, s->wt);
    // the MFMA paths address x and h with 32-bit buffer offsets
    if ((s->wt == MOE_BF16 || quant) && ((size_t)s->T * s->k * s->F * 2 >= ((size_t)1 << 31) ||
                                         (size_t)s->T * s->d * 2 >= ((size_t)1 << 31)))
        return fail(err, err_len, MOE_EUNSUPPORTED, "T*k*F and T*d bf16 buffers must stay below 2 GiB");
    // the tiled layouts are read by the skinny matrix-core kernel only
    if (s->wt == MOE_INT4_G128_TILED && (!i4mfma_supported(s->d, s->F) || !i4mfma_supported(s->F, s->d)))
        return fail(err, err_len, MOE_EUNSUPPORTED,
                    "tiled int4 weights need d and F multiples of 1024 and at most 8192 (d=%d F=%d)", s->d, s->F);
    if (s->wt == MOE_MXFP4_TILED &&
        (!i4mfma_supported(s->d, s->F, kFmtFp4) || !i4mfma_supported(s->F, s->d, kFmtFp4)))
        return fail(err, err_len, MOE_EUNSUPPORTED, "tiled MXFP4 weights need d and F multiples of 1024 (d=%d F=%d)",
                    s->d, s->F);
    if (s->wt == MOE_MXFP8_TILED &&
        (!i4mfma_supported(s->d, s->F, kFmtFp8) || !i4mfma_supported(s->F, s->d, kFmtFp8)))
        return fail(err, err_len, MOE_EUNSUPPORTED, "tiled MXFP8 weights need d and F multiples of 1024 (d=%d F=%d)",
                    s->d, s->F);
    // the GEMV's register-resident token fragments bound K; the quantised
    // formats are held to the 16384 the header states (the int4 GEMV could
    // take 32768; the dequantising GEMM has no such bound)
    const int kmax = quant ? 16384 : gemv_max_k(s->wt);
    if (s->d > kmax || s->F > kmax)
        return fail(err, err_len, MOE_EUNSUPPORTED, "d=%d / F=%d exceed this build's limit %d for this dtype",
                    s->d, s->F, kmax);
    return MOE_OK;
}

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t logits, idx, w, counts, offsets, perm, inv, tiles, h, yp, hs, ys, sid, part, total;
    int part_cap;
};

bool is_int4(const moe_shape* s) { return s->wt == MOE_INT4_G128 || s->wt == MOE_INT4_G128_TILED; }

// MX weights whose d and F the skinny matrix-core kernel takes (ffn_i4mfma.hip)
int mx_fmt(const moe_shape* s) {
    return (s->wt == MOE_MXFP4 || s->wt == MOE_MXFP4_TILED)   ? kFmtFp4
           : (s->wt == MOE_MXFP8 || s->wt == MOE_MXFP8_TILED) ? kFmtFp8
                                                               : -1;
}
// code bytes in the tiled layout: only the skinny matrix-core kernel reads them
bool tiled_codes(const moe_shape* s) {
    return s->wt == MOE_INT4_G128_TILED || s->wt == MOE_MXFP4_TILED || s->wt == MOE_MXFP8_TILED;
}
bool mx_skinny(const moe_shape* s) {
    const int f = mx_fmt(s);
    return f >= 0 && i4mfma_supported(s->d, s->F, f) && i4mfma_supported(s->F, s->d, f);
}

constexpr int kDefaultInt4Tau = 32;
// int4-g128 groups on the dequantising GEMM: a last partial tile of at most
// this many rows goes to the skinny matrix-core kernel instead.  Such
// a tile would stream and widen its expert's whole weight matrix for a few
// rows (~11 us of the whole GPU per 128-row int4 tile at the fine-grained
// shape, d = 7168, F = 2048); the skinny kernel streams it at the HBM rate
// once per token pass (9 rows at d = 7168, 16 at d <= 2048: one or two
// passes, ~4-7 us).
constexpr int kDqRemainderRows = 16;

// Format code of the dequantising grouped GEMM for this weight dtype, or -1
// when it does not serve it (fp32, bf16, tiled int4 codes)
int dq_format(const moe_shape* s) {
    if (s->wt == MOE_INT4_G128 || s->wt == MOE_INT4_G64) return 0;
    if (s->wt == MOE_MXFP4) return 1;
    if (s->wt == MOE_MXFP8) return 2;
    return -1;
}

// Groups above this many rows run the dequantising GEMM (-1: none does):
// int4-g128, and MX weights whose d and F the skinny kernel takes, keep
// groups of at most tau rows (0: 32) on the skinny kernels -- with the
// default, once the mean group is twice that, every group goes to the GEMM
// and the skinny launches (which would find no work) are left out; int4-g64
// and other MX shapes run every group on it.
int dq_tau(const moe_shape* s) {
    if (tiled_codes(s)) return -1;
    if (s->wt == MOE_INT4_G128 || mx_skinny(s)) {
        if (s->tau < 0) return -1;
        if (s->tau > 0) return s->tau;
        return (long)s->T * s->k >= 2L * kDefaultInt4Tau * s->E ? 0 : kDefaultInt4Tau;
    }
    return dq_format(s) >= 0 ? 0 : -1;
}

// The shared expert runs as a group of its own (one expert that every token
// picks once: counts, offsets and an identity perm) for bf16 and fp32 layers
// and wherever the dequantising GEMM may take it; otherwise (tiled int4,
// row-major int4 with T within the skinny kernels' range) it rides in the
// skinny int4 launches.
bool shared_as_group(const moe_shape* s) {
    if (!s->n_shared) return false;
    if (tiled_codes(s)) return false;
    if (!is_int4(s) && !mx_skinny(s)) return true;
    const int t = dq_tau(s);
    return t >= 0 && s->T > t;
}

int effective_tau(const moe_shape* s);
int tile_mode(const moe_shape* s);

// Partial tiles the split tail round of the 256-row MFMA kernel may use: at
// most one per block of its grid, which never exceeds max_mt x N-tiles.
int part_cap(const moe_shape* s) {
    const int tau = effective_tau(s);
    if (tau < 0 || s->T <= tau || tile_mode(s) == MFMA_TILES_SMALL) return 0;
    const long nn = std::max(mfma_ntiles_n(0, s->F), mfma_ntiles_n(1, s->d));
    const long c = (long)mfma_max_tiles(s->T, s->k, s->E) * nn;
    return (int)std::min<long>(c, mfma_part_cap());
}

Layout layout(const moe_shape* s) {
    const size_t T = s->T, k = s->k, E = s->E, d = s->d, F = s->F;
    const size_t hb = (s->act == MOE_F32) ? 4 : 2;
    const size_t tk = T * k;
    Layout L;
    size_t o = 0;
    L.logits = o; o += up(T * E * 4);
    L.idx = o; o += up(tk * 4);
    L.w = o; o += up(tk * 4);
    L.counts = o; o += up(E * 4);
    L.offsets = o; o += up((E + 1) * 4);
    L.perm = o; o += up(tk * 4);
    L.inv = o; o += up(tk * 4);
    L.tiles = o; o += up((size_t)std::max(mfma_plan_ints(s->T, s->k, s->E), dq_plan_ints(s->T, s->k, s->E)) * 4);
    L.h = o; o += up(tk * F * hb);
    L.yp = o; o += up(tk * d * 4);
    L.hs = o; o += s->n_shared ? up(T * F * hb) : 0;
    L.ys = o; o += s->n_shared ? up(T * d * 4) : 0;
    L.sid = o; o += shared_as_group(s) ? up((3 + T) * 4) : 0;
    L.part_cap = part_cap(s);
    L.part = o; o += up((size_t)L.part_cap * 256 * 256 * 4);
    L.total = o;
    return L;
}

// the skinny MFMA kernel can serve both projections of this shape
bool skinny_applies(const moe_shape* s) {
    return s->wt == MOE_BF16 && s->act == MOE_BF16 && skinny_supported(s->d, s->F, s->T) &&
           skinny_supported(s->F, s->d, s->T * s->k);
}

int effective_tau(const moe_shape* s) {
    if (s->wt != MOE_BF16) return -1;      // fp32 and int4: GEMV for every group
    if (s->tau < 0) return -1;
    if (s->tau > 0) return s->tau;
    // default: the skinny kernel up to 64 rows where K gives its items eight
    // or more steps (d, F >= 4096); with shorter rows its per-item reduction
    // and extra token reads cost more than the 64-row MFMA tiles above one
    // token tile
    const int td = (skinny_applies(s) && s->d >= 4096 && s->F >= 4096) ? kSkinnyMaxRows : kDefaultTau;
    // when the mean group is at least twice that, groups at or below it are
    // rare: every group goes to the MFMA tiles (a 64-row tile streams its
    // expert's weights once, as one GEMV or skinny pass does), and the GEMV
    // and skinny launches, which would find no work, are left out
    return (long)s->T * s->k >= 2L * td * s->E ? 0 : td;
}

// Tile lists of the bf16 grouped GEMM.  Explicit tau: groups up to 128 rows
// on 64-row tiles, larger ones on 256-row tiles.  Default tau: with T <= 128
// no group exceeds 128 rows, so only the 64-row list can be filled; with a
// mean group of at most 64 rows and experts of at most 32 MiB, every group
// goes to 64-row tiles (a rare group above 128 rows streams its weights once
// per 64 rows, a few microseconds at that size, against ~20 us for the
// 256-row launches that would otherwise run empty); with a mean group of at
// least 512 rows every group goes to 256-row tiles (a rare small group pays
// padded MFMA work, not extra weight reads).
int tile_mode(const moe_shape* s) {
    if (s->tau != 0) return MFMA_TILES_BOTH;
    const long tk = (long)s->T * s->k;
    const double expert_bytes = 3.0 * s->F * s->d * 2.0;
    if (s->T <= 2 * kMfmaSmallRows) return MFMA_TILES_SMALL;
    if (tk <= (long)kMfmaSmallRows * s->E && expert_bytes <= 32.0 * (1 << 20)) return MFMA_TILES_SMALL;
    if (tk >= 512L * s->E) return MFMA_TILES_BIG;
    return MFMA_TILES_BOTH;
}

// Workspace regions one expert-FFN pass writes: h, the MFMA tile plan and
// the partial tiles of the split tail round.
struct FfnBufs {
    void* h;
    int32_t* tiles;
    float* part;
    int part_cap;
    bool plan_ready;     // the dispatch kernel already wrote the MFMA tile lists
};

// The FFN launch sequence of the routed experts, shared by moe_expert_ffn and
// moe_layer_forward; an int4 shared expert rides along in the same launches,
// a bf16 or fp32 one runs afterwards as a one-expert group (run_ffn).
int run_groups(const moe_shape* s, const void* x, const moe_weights* w, const int32_t* counts,
               const int32_t* offsets, const int32_t* perm, float* y_perm, float* y_shared,
               const FfnBufs& b, void* hs, hipStream_t st, char* err, size_t err_len) {
    const int tau = effective_tau(s);
    const bool use_mfma = tau >= 0 && s->T > tau;
    void* h = b.h;
    int32_t* tiles = b.tiles;
    float* part = b.part_cap ? b.part : nullptr;
    const int part_cap = b.part_cap;
    const int max_mt = mfma_max_tiles(s->T, s->k, s->E);
    const int tmode = tile_mode(s);
    // quantised groups above dqt rows: the dequantising grouped GEMM
    const int dqf = dq_format(s), dqt = dq_tau(s);
    const bool use_dq = dqf >= 0 && dqt >= 0 && s->T > dqt;
    // some groups stay on the streaming kernels (GEMV, skinny bf16 or int4):
    // not when the dequantising GEMM or the MFMA tiles take every group
    const bool skinny_q = dqt != 0 && !(use_mfma && tau == 0);
    const int dq_mt = dq_max_tiles(s->T, s->k, s->E);
    const int gs = s->wt == MOE_INT4_G64 ? 64 : 128;
    const bool dq_staged = use_dq && dq_staged_ok(dqf, gs, s->d) && dq_staged_ok(dqf, gs, s->F);
    // int4-g128 with every group on the dequantising GEMM: short last tiles
    // to the skinny int4 kernel (a one-expert group of T rows has one only
    // when T leaves a short one)
    const int dq_bm = use_dq ? dq_tile_rows(dqf, dq_staged) : 0;
    const int sfmt = mx_fmt(s) >= 0 ? mx_fmt(s) : kFmtInt4;       // the skinny kernel's code format
    // (int4 only: MXFP4's 64-row GEMM tiles cost less than a second weight
    // stream on the skinny kernel -- fine-grained prefill 3.92-3.96 -> 4.02 ms
    // with it -- and no MXFP8 layer here has fine-grained groups)
    const bool dq_rem = kDqRemainderRows > 0 && use_dq && dqt == 0 && dq_staged && s->wt == MOE_INT4_G128 &&
                        i4mfma_supported(s->d, s->F) && i4mfma_supported(s->F, s->d) &&
                        (s->E > 1 || (s->T % dq_bm != 0 && s->T % dq_bm <= kDqRemainderRows));
    const int max_rows_gemv = use_mfma ? tau : s->T;   // a group holds at most T rows
    int rc;

    if (s->T == 0) return MOE_OK;
    if (use_mfma && !b.plan_ready) {
        rc = hip_check(launch_mfma_plan(counts, offsets, s->T, s->k, s->E, tau, tmode, tiles, max_mt, st), st,
                       "mfma plan", err, err_len);
        if (rc) return rc;
    }
    if (use_dq) {
        rc = hip_check(launch_dq_plan(counts, offsets, s->E, dqt, dqf, dq_staged, tiles, dq_mt,
                                      dq_rem ? kDqRemainderRows : 0, st),
                       st, "dq plan", err, err_len);
        if (rc) return rc;
    }
    // routed experts (g) and the shared expert (q: one expert over all T rows)
    GemvArgs g{};
    g.counts = counts;
    g.offsets = offsets;
    g.perm = perm;
    g.topk = s->k;
    g.T = s->T;
    g.E = s->E;
    g.tau = use_mfma ? tau : (use_dq ? dqt : -1);
    GemvArgs q{};
    q.topk = 1; q.T = s->T; q.E = 1; q.tau = -1;
    const GemvArgs* qp = (s->n_shared && (is_int4(s) || mx_skinny(s)) && !shared_as_group(s)) ? &q : nullptr;
    const int active = (s->T * s->k < s->E) ? s->T * s->k : s->E;   // experts that can be hit
    const bool tiled = tiled_codes(s);
    // bf16 groups below the MFMA tiles: when one of them is larger than a
    // GEMV pass (lo rows), the skinny MFMA kernel (one pass of up to 64
    // tokens) takes every group below the tiles in one balanced launch and
    // the GEMV stands aside; otherwise the GEMV serves them.  Both kernels
    // decide from the counts on the device.  The skinny kernel is only
    // launched when such a group can occur: a group holds at most T rows, and
    // everything below the tiles must fit one skinny pass (tau <= 64); a
    // negative tau keeps the GEMV for all
    const int tau_m = use_mfma ? tau : s->T;                   // largest group below the tiles
    auto skinny_lo = [&](int mode, int K, int N, int in_rows) -> int {
        if (s->wt != MOE_BF16 || s->act != MOE_BF16 || s->tau < 0 || tau_m > kSkinnyMaxRows ||
            !skinny_supported(K, N, in_rows))
            return -1;
        const int lo = gemv_pass_tokens(s->wt, mode, K);
        return tau_m > lo ? lo : -1;
    };
    // one pass (gate/up or down) of the routed and the shared expert: int4 on
    // the matrix cores in one launch, else one GEMV launch each
    auto pass = [&](int mode, const char* what) -> int {
        if (tiled || mx_skinny(s) || (s->wt == MOE_INT4_G128 && i4mfma_supported(g.K, g.N)))
            return hip_check(launch_i4mfma(mode, tiled, &g, qp, st, sfmt), st, what, err, err_len);
        g.rows_per_item = gemv_rows_per_item(s->wt, mode, g.K, g.N, active);
        const int in_rows = mode == 0 ? s->T : s->T * s->k;
        const int lo = skinny_lo(mode, g.K, g.N, in_rows);
        const int gemv_tau = g.tau;
        if (lo >= 0) {
            g.tau = lo;                                            // the GEMV keeps groups of <= lo rows
            g.yield_hi = tau_m;                                    // unless a larger one sends all to skinny
        }
        int r = hip_check(launch_gemv(s->wt, s->act, mode, g, s->E, max_rows_gemv, st), st, what, err, err_len);
        g.tau = gemv_tau;
        g.yield_hi = 0;
        if (r) return r;
        if (lo >= 0) {
            r = hip_check(launch_skinny(mode, g.w0, g.w1, g.in, in_rows, g.out, g.counts, g.offsets, g.perm, g.N,
                                        g.K, g.topk, s->E, lo, tau_m, st),
                          st, what, err, err_len);
            if (r) return r;
        }
        if (!qp) return r;
        q.rows_per_item = gemv_rows_per_item(s->wt, mode, q.K, q.N, 1);
        return hip_check(launch_gemv(s->wt, s->act, mode, q, 1, s->T, st), st, what, err, err_len);
    };

    // gate/up + SwiGLU
    g.w0 = w->w_gate; g.w1 = w->w_up;
    g.s0 = (const uint16_t*)w->s_gate; g.s1 = (const uint16_t*)w->s_up;
    g.in = x; g.out = h; g.N = s->F; g.K = s->d;
    q.w0 = w->sh_gate; q.w1 = w->sh_up;
    q.s0 = (const uint16_t*)w->sh_s_gate; q.s1 = (const uint16_t*)w->sh_s_up;
    q.in = x; q.out = hs; q.N = s->F; q.K = s->d;
    if (skinny_q) {
        rc = pass(0, "gate/up");
        if (rc) return rc;
    }
    // the remainder rows the dq plan listed, on the skinny int4 kernel
    auto remainders = [&](int mode, const char* what) -> int {
        GemvArgs r = g;
        r.counts = dq_remainders(tiles, dq_mt);
        r.offsets = r.counts + s->E;
        r.tau = -1;
        return hip_check(launch_i4mfma(mode, false, &r, nullptr, st, sfmt), st, what, err, err_len);
    };
    if (use_dq) {
        rc = hip_check(launch_dq_ffn(0, dqf, gs, dq_staged, w->w_gate, w->w_up, w->s_gate, w->s_up, x, h, perm, tiles,
                                     s->F, s->d, s->k, dq_mt, s->T, st),
                       st, "dq gate/up", err, err_len);
        if (rc) return rc;
        if (dq_rem && (rc = remainders(0, "dq gate/up remainders"))) return rc;
    }
    if (use_mfma) {
        rc = hip_check(launch_mfma_ffn(0, tmode, w->w_gate, w->w_up, x, h, perm, tiles, s->F, s->d, s->k, s->T, max_mt,
                                       s->E, s->T, part, part_cap, st),
                       st, "mfma gate/up", err, err_len);
        if (rc) return rc;
    }
    // down
    g.w0 = w->w_down; g.w1 = nullptr;
    g.s0 = (const uint16_t*)w->s_down; g.s1 = nullptr;
    g.in = h; g.out = y_perm; g.N = s->d; g.K = s->F;
    q.w0 = w->sh_down; q.w1 = nullptr;
    q.s0 = (const uint16_t*)w->sh_s_down; q.s1 = nullptr;
    q.in = hs; q.out = y_shared; q.N = s->d; q.K = s->F;
    if (skinny_q) {
        rc = pass(1, "down");
        if (rc) return rc;
    }
    if (use_dq) {
        rc = hip_check(launch_dq_ffn(1, dqf, gs, dq_staged, w->w_down, nullptr, w->s_down, nullptr, h, y_perm, perm,
                                     tiles, s->d, s->F, s->k, dq_mt, s->T * s->k, st),
                       st, "dq down", err, err_len);
        if (rc) return rc;
        if (dq_rem && (rc = remainders(1, "dq down remainders"))) return rc;
    }
    if (use_mfma) {
        rc = hip_check(launch_mfma_ffn(1, tmode, w->w_down, nullptr, h, y_perm, perm, tiles, s->d, s->F, s->k, s->T,
                                       max_mt, s->E, s->T * s->k, part, part_cap, st),
                       st, "mfma down", err, err_len);
        if (rc) return rc;
    }
    return MOE_OK;
}

// Routed experts, then (bf16 and fp32 layers) the shared expert through the
// same kernel selection as a group of all T tokens: groups above tau on the
// MFMA tiles, smaller ones on the skinny kernel or the GEMV.  Its y_perm is
// y_shared (identity order) and its h the shared region of the workspace.
int run_ffn(const moe_shape* s, const void* x, const moe_weights* w, const int32_t* counts,
            const int32_t* offsets, const int32_t* perm, float* y_perm, float* y_shared,
            char* ws, hipStream_t st, char* err, size_t err_len, bool plan_ready = false) {
    const Layout L = layout(s);
    const FfnBufs b{ws + L.h, reinterpret_cast<int32_t*>(ws + L.tiles), reinterpret_cast<float*>(ws + L.part),
                    L.part_cap, plan_ready};
    void* hs = s->n_shared ? ws + L.hs : nullptr;
    int rc = run_groups(s, x, w, counts, offsets, perm, y_perm, y_shared, b, hs, st, err, err_len);
    if (rc || !shared_as_group(s) || s->T == 0) return rc;
    moe_shape sh = *s;
    sh.E = 1;
    sh.k = 1;
    sh.n_shared = 0;
    moe_weights sw{};
    sw.w_gate = w->sh_gate;
    sw.w_up = w->sh_up;
    sw.w_down = w->sh_down;
    sw.s_gate = w->sh_s_gate;
    sw.s_up = w->sh_s_up;
    sw.s_down = w->sh_s_down;
    int32_t* sid = reinterpret_cast<int32_t*>(ws + L.sid);
    rc = hip_check(launch_identity_group(sid, sid + 1, sid + 3, s->T, st), st, "shared group", err, err_len);
    if (rc) return rc;
    // the routed plan and partial tiles are consumed by now (stream order); a
    // one-expert group needs no more of either than the routed experts do
    const FfnBufs bs{hs, b.tiles, b.part, std::min(part_cap(&sh), L.part_cap), false};
    return run_groups(&sh, x, &sw, sid, sid + 1, sid + 3, y_shared, nullptr, bs, nullptr, st, err, err_len);
}

int check_weights(const moe_shape* s, const moe_weights* w, char* err, size_t err_len) {
    if (!w) return fail(err, err_len, MOE_EINVAL, "weights is NULL");
    NEED_PTR(w->w_gate, "w_gate");
    NEED_PTR(w->w_up, "w_up");
    NEED_PTR(w->w_down, "w_down");
    const bool int4 = s->wt >= MOE_INT4_G128;    // every quantised format carries scales
    if (int4) {
        NEED_PTR(w->s_gate, "s_gate");
        NEED_PTR(w->s_up, "s_up");
        NEED_PTR(w->s_down, "s_down");
    }
    if (s->n_shared) {
        NEED_PTR(w->sh_gate, "sh_gate");
        NEED_PTR(w->sh_up, "sh_up");
        NEED_PTR(w->sh_down, "sh_down");
        if (int4) {
            NEED_PTR(w->sh_s_gate, "sh_s_gate");
            NEED_PTR(w->sh_s_up, "sh_s_up");
            NEED_PTR(w->sh_s_down, "sh_s_down");
        }
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_strerror(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_ENOMEM: return "workspace too small";
        case MOE_EHIP: return "HIP error";
        case MOE_EUNSUPPORTED: return "unsupported by this build";
        default: return "unknown status";
    }
}

size_t moe_workspace_bytes(const moe_shape* shape) {
    if (check_shape(shape, nullptr, 0) != MOE_OK) return 0;
    return layout(shape).total;
}

int moe_route(const moe_shape* shape, const void* x, const float* w_router, const float* b_router,
              float* logits, int32_t* topk_idx, float* topk_w, void* stream, char* err, size_t err_len) {
    int rc = check_shape(shape, err, err_len);
    if (rc) return rc;
    if (shape->T > 0) {
        NEED_PTR(x, "x");
        NEED_PTR(w_router, "w_router");
        NEED_PTR(logits, "logits");
        NEED_PTR(topk_idx, "topk_idx");
        NEED_PTR(topk_w, "topk_w");
    }
    OPT_PTR(b_router, "b_router");
    hipStream_t st = (hipStream_t)stream;
    return hip_check(launch_route(shape->act, x, w_router, b_router, logits, topk_idx, topk_w, shape->T,
                                  shape->d, shape->E, shape->k, st),
                     st, "route", err, err_len);
}

int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* inv, void* stream, char* err, size_t err_len) {
    int rc = check_shape(shape, err, err_len);
    if (rc) return rc;
    NEED_PTR(counts, "counts");
    NEED_PTR(offsets, "offsets");
    if (shape->T > 0) {
        NEED_PTR(topk_idx, "topk_idx");
        NEED_PTR(perm, "perm");
        NEED_PTR(inv, "inv");
    }
    hipStream_t st = (hipStream_t)stream;
    return hip_check(launch_dispatch(topk_idx, counts, offsets, perm, inv, shape->T, shape->k, shape->E, st),
                     st, "dispatch", err, err_len);
}

int moe_expert_ffn(const moe_shape* shape, const void* x, const moe_weights* w, const int32_t* counts,
                   const int32_t* offsets, const int32_t* perm, float* y_perm, float* y_shared, void* ws,
                   size_t ws_bytes, void* stream, char* err, size_t err_len) {
    int rc = check_shape(shape, err, err_len);
    if (rc) return rc;
    rc = check_weights(shape, w, err, err_len);
    if (rc) return rc;
    if (shape->T > 0) {
        NEED_PTR(x, "x");
        NEED_PTR(counts, "counts");
        NEED_PTR(offsets, "offsets");
        NEED_PTR(perm, "perm");
        NEED_PTR(y_perm, "y_perm");
        if (shape->n_shared) NEED_PTR(y_shared, "y_shared");
    }
    const size_t need = layout(shape).total;
    if (!ws || ws_bytes < need)
        return fail(err, err_len, MOE_ENOMEM, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
    if (((uintptr_t)ws & (kAlign - 1)) != 0)
        return fail(err, err_len, MOE_EINVAL, "workspace is not 256-byte aligned");
    return run_ffn(shape, x, w, counts, offsets, perm, y_perm, y_shared, (char*)ws, (hipStream_t)stream, err,
                   err_len);
}

int moe_combine(const moe_shape* shape, const float* y_perm, const int32_t* inv, const float* topk_w,
                const float* y_shared, const void* residual, void* y, void* stream, char* err,
                size_t err_len) {
    int rc = check_shape(shape, err, err_len);
    if (rc) return rc;
    if (shape->T > 0) {
        NEED_PTR(y_perm, "y_perm");
        NEED_PTR(inv, "inv");
        NEED_PTR(topk_w, "topk_w");
        NEED_PTR(y, "y");
    }
    OPT_PTR(y_shared, "y_shared");
    OPT_PTR(residual, "residual");
    hipStream_t st = (hipStream_t)stream;
    return hip_check(launch_combine(shape->act, y_perm, inv, topk_w, y_shared, residual, y, shape->T, shape->d,
                                    shape->k, st),
                     st, "combine", err, err_len);
}

int moe_layer_forward(const moe_shape* shape, const void* x, const float* w_router, const float* b_router,
                      const moe_weights* w, const void* residual, void* y, int32_t* counts_out,
                      int32_t* topk_idx_out, void* ws, size_t ws_bytes, void* stream, char* err,
                      size_t err_len) {
    int rc = check_shape(shape, err, err_len);
    if (rc) return rc;
    rc = check_weights(shape, w, err, err_len);
    if (rc) return rc;
    if (shape->T > 0) {
        NEED_PTR(x, "x");
        NEED_PTR(w_router, "w_router");
        NEED_PTR(y, "y");
    }
    OPT_PTR(b_router, "b_router");
    OPT_PTR(residual, "residual");
    OPT_PTR(counts_out, "counts_out");
    OPT_PTR(topk_idx_out, "topk_idx_out");
    const Layout L = layout(shape);
    if (!ws || ws_bytes < L.total)
        return fail(err, err_len, MOE_ENOMEM, "workspace of %zu bytes needed, %zu given", L.total,
                    ws ? ws_bytes : 0);
    if (((uintptr_t)ws & (kAlign - 1)) != 0)
        return fail(err, err_len, MOE_EINVAL, "workspace is not 256-byte aligned");

    char* W = (char*)ws;
    hipStream_t st = (hipStream_t)stream;
    float* logits = (float*)(W + L.logits);
    int32_t* idx = topk_idx_out ? topk_idx_out : (int32_t*)(W + L.idx);
    float* gw = (float*)(W + L.w);
    int32_t* counts = counts_out ? counts_out : (int32_t*)(W + L.counts);
    int32_t* offsets = (int32_t*)(W + L.offsets);
    int32_t* perm = (int32_t*)(W + L.perm);
    int32_t* inv = (int32_t*)(W + L.inv);
    float* yp = (float*)(W + L.yp);
    float* ys = shape->n_shared ? (float*)(W + L.ys) : nullptr;

    if (shape->T == 0) {
        // no tokens: the usage histogram is all zero
        return hip_check(launch_dispatch(idx, counts, offsets, perm, inv, 0, shape->k, shape->E, st), st,
                         "dispatch", err, err_len);
    }
    bool plan_ready = false;
    if (route_dispatch_small_supported(shape->T, shape->E, shape->k)) {
        // a decode batch: router, top-k and dispatch in one launch
        rc = hip_check(launch_route_dispatch_small(shape->act, x, w_router, b_router, logits, idx, gw, counts,
                                                   offsets, perm, inv, shape->T, shape->d, shape->E, shape->k, st),
                       st, "route+dispatch", err, err_len);
        if (rc) return rc;
    } else {
        rc = hip_check(launch_route(shape->act, x, w_router, b_router, logits, idx, gw, shape->T, shape->d,
                                    shape->E, shape->k, st),
                       st, "route", err, err_len);
        if (rc) return rc;
        // the routed experts' MFMA tile lists come out of the dispatch kernel
        const int tau = effective_tau(shape);
        if (tau >= 0 && shape->T > tau) {
            const MfmaPlanArgs plan = mfma_plan_args(shape->T, shape->k, shape->E, tau, tile_mode(shape),
                                                     (int32_t*)(W + L.tiles),
                                                     mfma_max_tiles(shape->T, shape->k, shape->E));
            plan_ready = true;
            rc = hip_check(launch_dispatch(idx, counts, offsets, perm, inv, shape->T, shape->k, shape->E, st, &plan),
                           st, "dispatch", err, err_len);
        } else {
            rc = hip_check(launch_dispatch(idx, counts, offsets, perm, inv, shape->T, shape->k, shape->E, st), st,
                           "dispatch", err, err_len);
        }
        if (rc) return rc;
    }
    rc = run_ffn(shape, x, w, counts, offsets, perm, yp, ys, W, st, err, err_len, plan_ready);
    if (rc) return rc;
    return hip_check(launch_combine(shape->act, yp, inv, gw, ys, residual, y, shape->T, shape->d, shape->k, st),
                     st, "combine", err, err_len);
}

int moe_rmsnorm(const moe_shape* shape, const void* h, const float* gamma, float eps, void* out, void* stream,
                char* err, size_t err_len) {
    if (!shape) return fail(err, err_len, MOE_EINVAL, "shape is NULL");
    if (shape->T < 0 || shape->d < 8 || shape->d % 8)
        return fail(err, err_len, MOE_EINVAL, "T=%d d=%d: need T >= 0 and d a positive multiple of 8", shape->T,
                    shape->d);
    if (shape->act != MOE_F32 && shape->act != MOE_BF16)
        return fail(err, err_len, MOE_EINVAL, "act=%d is not MOE_F32 or MOE_BF16", shape->act);
    if (!(eps >= 0.0f)) return fail(err, err_len, MOE_EINVAL, "eps must be >= 0");
    if (shape->T > 0) {
        NEED_PTR(h, "h");
        NEED_PTR(out, "out");
    }
    OPT_PTR(gamma, "gamma");
    hipStream_t st = (hipStream_t)stream;
    return hip_check(launch_rmsnorm(shape->act, h, gamma, eps, out, shape->T, shape->d, st), st, "rmsnorm", err,
                     err_len);
}

int moe_topk_overlap(const moe_shape* shape, const int32_t* pred_idx, const int32_t* actual_idx, int32_t* hist,
                     void* stream, char* err, size_t err_len) {
    int rc = check_shape(shape, err, err_len);
    if (rc) return rc;
    NEED_PTR(hist, "hist");
    if (shape->T > 0) {
        NEED_PTR(pred_idx, "pred_idx");
        NEED_PTR(actual_idx, "actual_idx");
    }
    hipStream_t st = (hipStream_t)stream;
    return hip_check(launch_topk_overlap(pred_idx, actual_idx, hist, shape->T, shape->k, st), st, "topk overlap",
                     err, err_len);
}

int moe_pack_int4_tiled(const void* src, void* dst, int64_t n_mats, int32_t N, int32_t K, void* stream, char* err,
                        size_t err_len) {
    if (n_mats < 0) return fail(err, err_len, MOE_EINVAL, "n_mats=%lld is negative", (long long)n_mats);
    if (N < 16 || N % 16) return fail(err, err_len, MOE_EINVAL, "N=%d must be a positive multiple of 16", N);
    if (K < 128 || K % 128) return fail(err, err_len, MOE_EINVAL, "K=%d must be a positive multiple of 128", K);
    const size_t bytes = (size_t)n_mats * (size_t)N * (size_t)(K / 2);
    if (n_mats > 0 && bytes / (size_t)n_mats / (size_t)N != (size_t)(K / 2))
        return fail(err, err_len, MOE_EINVAL, "n_mats * N * K/2 overflows");
    if (!bytes) return MOE_OK;
    NEED_PTR(src, "src");
    NEED_PTR(dst, "dst");
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (a < b + bytes && b < a + bytes) return fail(err, err_len, MOE_EINVAL, "src and dst overlap");
    hipStream_t st = (hipStream_t)stream;
    return hip_check(launch_pack_int4_tiled(src, dst, (size_t)n_mats, N, K, st), st, "pack int4", err, err_len);
}

int moe_pack_mxfp8_tiled(const void* src, void* dst, int64_t n_mats, int32_t N, int32_t K, void* stream,
                         char* err, size_t err_len) {
    if (n_mats < 0) return fail(err, err_len, MOE_EINVAL, "n_mats=%lld is negative", (long long)n_mats);
    if (N < 16 || N % 16) return fail(err, err_len, MOE_EINVAL, "N=%d must be a positive multiple of 16", N);
    if (K < 128 || K % 128) return fail(err, err_len, MOE_EINVAL, "K=%d must be a positive multiple of 128", K);
    const size_t bytes = (size_t)n_mats * (size_t)N * (size_t)K;
    if (n_mats > 0 && bytes / (size_t)n_mats / (size_t)N != (size_t)K)
        return fail(err, err_len, MOE_EINVAL, "n_mats * N * K overflows");
    if (!bytes) return MOE_OK;
    NEED_PTR(src, "src");
    NEED_PTR(dst, "dst");
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (a < b + bytes && b < a + bytes) return fail(err, err_len, MOE_EINVAL, "src and dst overlap");
    hipStream_t st = (hipStream_t)stream;
    return hip_check(launch_pack_mxfp8_tiled(src, dst, (size_t)n_mats, N, K, st), st, "pack mxfp8", err, err_len);
}

}  // extern "C"
