// Expert FFN for int4-g128 weights at decode-sized groups: a skinny MFMA GEMM.
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §3.1 (w1/w3 gate and up,
// w2 down, no bias) and §3.3 (each expert streams its own weights for the
// tokens the dispatcher gave it); [P5] "一只蜂鸟如何喂饱九头大象" §7.3
// (int4 experts with per-group scales).  Weight format: int4 two's complement,
// two per byte (even K index in the low nibble), one fp16 scale per 128 K.
//
// Why MFMA at 1-16 tokens per expert: a dot-product GEMV spends ~7 VALU ops per
// packed dword on dequantisation plus 4 per token, and a cross-lane fold per
// row; at ~2-3 tokens per expert that is as slow as the HBM stream itself.
// Here the contraction runs on the matrix cores (v_mfma_f32_16x16x32_bf16 with
// the tokens as the 16-wide M side, padded) and the VALU only dequantises:
//
//  * every lane loads 16 bytes (32 nibbles) of one weight row per scale group:
//    lane l covers row l%16, K = 128 g + 32 (l/16) + [0, 32).  Dword i of that
//    load is the B operand of MFMA i of the group, so the 4 MFMAs of a group
//    cover exactly its 128 K and one fp16 scale applies to their sum;
//  * a dword becomes 8 bf16 with one shift and one mask-and-XOR per pair:
//    ((w >> 4s) & 0x000F000F) ^ 0x43084308 is the bf16 pair (136 + q_s,
//    136 + q_{s+4}), exact.  The token rows are kept in LDS in the matching
//    order (elements 0,4,1,5,2,6,3,7 of every 8), so an A fragment is one
//    16-byte LDS read, and the per-group sums of x held beside them remove the
//    136 offset: acc += s_g (C_g - 136 sum_g x);
//  * rows of up to P tokens (P set by K so that P rows fit the 160 KB of LDS,
//    at most 16) are staged once per (expert, token pass) and shared by the 8
//    waves of the block; token slots past the group read an all-zero row;
//  * a persistent grid (one 512-thread block per CU) walks equal-sized work
//    items (active expert, token pass, 128 rows); each wave owns 16 rows and
//    runs a flat stream of (item, group) steps with the weight loads of 8
//    groups in flight in a register ring (16 KB per wave for gate+up), so the
//    stream continues across item boundaries; the buffer range
//    check returns zeros past the last row and past the block's range, so
//    loads never branch;
//  * row-major weights give each load instruction 16 rows x 64 bytes, half
//    of a 128-byte line per row; the loads of two consecutive groups (the two
//    halves of every line) are issued back to back so they meet in the cache.
//    The tiled layout (MOE_INT4_G128_TILED, written once by moe_pack_int4_tiled)
//    stores exactly what one load instruction reads as 1 KB of consecutive
//    bytes, and the groups of a 16-row set one after another; those loads go
//    out non-temporal (whole lines, read once), which reads ~11% faster;
//  * a shared expert, when present, is one more slot of the same launch (all
//    T tokens, its own weights and buffers), so its passes overlap the routed
//    experts' instead of running as a separate small launch;
//  * gate and up share each A fragment; the SwiGLU epilogue writes h (bf16),
//    the down pass writes fp32 rows of y_perm (y_shared for the shared slot).
//
// MXFP4 and MXFP8 weights ([P5] §6: models shipped as native MX checkpoints)
// run the same kernel: the same 128-K groups, lane l holding 32 codes of row
// l%16 at K = 128 g + 32 (l/16) (16 bytes of E2M1 codes, or 32 of E4M3), but
// every 32 codes carry their own E8M0 scale, which is exactly the 32 codes a
// lane holds.  A lane widens its codes with v_cvt_scalef32_pk_bf16_fp4/_fp8,
// two per instruction and already times the scale (exact in bf16), so the
// MFMAs accumulate straight into the sums: no offset, no per-group sums, and
// the token rows are staged in plain element order.  The scale bytes of four
// groups of a row (16 bytes) go out with the weights of the first of them,
// into a ring of four such chunks.  fp8 codes take two 16-byte loads per
// group and matrix, so their ring holds 4 steps instead of 8 (the same bytes
// in flight).  Row-major fp8 codes give each of those loads 16 rows x four
// 16-byte pieces 32 bytes apart; their tiled layout (MOE_MXFP8_TILED, written
// once by moe_pack_mxfp8_tiled) stores each load's 1 KB consecutively, two
// per group of a 16-row set, which streams ~25% faster at the Mixtral shape.
#include <type_traits>

#include "common.h"
#include "devinfo.h"
#include "kernels.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kItemRows = 16 * kWaves;      // rows of one work item
constexpr int kLdsBytes = 160 * 1024;
constexpr int kMaxE = 256;
constexpr int kStaticLds = 4608;            // the __shared__ arrays below, rounded up

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                             0x00020000);
}
// buffer-load cache policy bit: nt (streamed, not kept in the caches)
constexpr int kNonTemporal = 2;
template <int AUX = 0>
__device__ __forceinline__ u32x4_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
}

template <int I>
using ic = std::integral_constant<int, I>;

// E8M0 scale code -> 2^(code - 127) in fp32 (code 0: 2^-127, a subnormal)
__device__ __forceinline__ float mx_scale(uint32_t code) {
    return __uint_as_float(code ? (code << 23) : 0x00400000u);
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(ic<B>{});
        static_for<B + 1, E>(f);
    }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Position in the flat stream of (work item, scale group) steps of a block.
// Every field is wave-uniform.
struct Cursor {
    int idx;      // step index in the block's range
    int u;        // expert slot
    int pass;     // token pass within the expert
    int chunk;    // 128-row chunk
    int g;        // scale group
    int c, o;     // rows of the expert's group, its first dispatch row
    int e;        // expert id; -1: the shared expert
};

}  // namespace

struct I4Args {
    const uint8_t* w0;         // routed gate (mode 0) or down (mode 1): [E][N][K/2]
    const uint8_t* w1;         // routed up (mode 0)
    const uint16_t* s0;        // fp16 scales [E][N][K/128]
    const uint16_t* s1;
    const uint16_t* in;        // bf16 x [T][K] (mode 0) or h [T*k][K] (mode 1)
    void* out;                 // bf16 h [T*k][N] (mode 0) or fp32 y_perm [T*k][N] (mode 1)
    const int32_t* counts;     // null: no routed experts
    const int32_t* offsets;
    const int32_t* perm;       // mode 0: token of dispatch row p = perm[p] / topk
    const uint8_t* sw0;        // shared expert ([1][N][K/2] ...), null: none
    const uint8_t* sw1;
    const uint16_t* ss0;
    const uint16_t* ss1;
    const uint16_t* sin;       // bf16 x [T][K] (mode 0) or h_shared [T][K] (mode 1)
    void* sout;                // bf16 h_shared [T][N] (mode 0) or fp32 y_shared [T][N] (mode 1)
    int N, K, topk, T, E, tau, P;
};

template <int MODE, int RING, bool TILED, int FMT>
__global__ __launch_bounds__(kThreads, 1) void i4_mfma_kernel(I4Args a) {
    constexpr int G = MODE == 0 ? 2 : 1;
    constexpr bool MX = FMT != kFmtInt4;
    constexpr bool FP8 = FMT == kFmtFp8;
    constexpr int NW = FP8 ? 2 : 1;             // 16-byte code loads per lane, group and matrix
    static_assert(MX || RING == 8, "the int4 scale prefetch runs 8 steps ahead, as far as the ring");
    static_assert(RING % 2 == 0 && RING <= 16, "steps are loaded in pairs within the 16-step unroll");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __shared__ int s_act[kMaxE + 1], s_cnt[kMaxE + 1], s_off[kMaxE + 1], s_ipref[kMaxE + 2];
    __shared__ int s_tot[2], s_src[16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K, N = a.N, P = a.P;
    const int NG = K / 128;                                  // scale groups per row (multiple of 8)
    const int nrc = (N + kItemRows - 1) / kItemRows;         // 128-row chunks per matrix
    const uint32_t rb = FP8 ? (uint32_t)K : (uint32_t)K / 2;          // code bytes per row
    const uint32_t srow = MX ? (uint32_t)K / 32 : (uint32_t)NG * 2;   // scale bytes per row
    const uint32_t RS = (uint32_t)K * 2 + 16;                // LDS bytes per staged token row
    char* xrows = smem;                                      // P token rows, then the zero row
    float* xsum = reinterpret_cast<float*>(smem + (size_t)(P + 1) * RS);   // [NG][16]

    // ---- the expert slots of this launch (routed experts with work, then the
    // shared one), their item counts and the prefix over them
    if (wave == 0) {
        int cnt[4], its[4], act[4];
        int na = 0, ni = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            const int c = (a.counts && e < a.E) ? a.counts[e] : 0;
            act[j] = c > 0 && (a.tau < 0 || c <= a.tau);
            cnt[j] = c;
            its[j] = act[j] ? ((c + P - 1) / P) * nrc : 0;
            na += act[j];
            ni += its[j];
        }
        const int ia = wave_incl_scan(na, lane), ii = wave_incl_scan(ni, lane);
        int k = ia - na, p = ii - ni;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (act[j]) {
                const int e = 4 * lane + j;
                s_act[k] = e;
                s_cnt[k] = cnt[j];
                s_off[k] = a.offsets[e];
                s_ipref[k] = p;
                ++k;
                p += its[j];
            }
        }
        if (lane == 63) {
            int u = ia, tot = ii;
            if (a.sw0 && a.T > 0) {
                s_act[u] = -1;
                s_cnt[u] = a.T;
                s_off[u] = 0;
                s_ipref[u] = tot;
                tot += ((a.T + P - 1) / P) * nrc;
                ++u;
            }
            s_tot[0] = u;
            s_tot[1] = tot;
            s_ipref[u] = tot;
        }
    }
    // the all-zero token row read by padded token slots
    for (int i = tid; i < (int)(RS / 16); i += kThreads)
        *reinterpret_cast<u32x4_t*>(xrows + (size_t)P * RS + (size_t)i * 16) = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();

    const int U = s_tot[0];
    const long n_items = s_tot[1];
    const long ib = n_items * blockIdx.x / gridDim.x;
    const long ie = n_items * (blockIdx.x + 1) / gridDim.x;
    if (ib >= ie) return;
    const int nsteps = (int)(ie - ib) * NG;

    // ---- start of the block's range
    Cursor cur;
    {
        int lo = 0, hi = U - 1;   // last slot whose first item is <= ib
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_ipref[mid] <= ib) lo = mid; else hi = mid - 1;
        }
        cur.u = lo;
        const int rel = (int)(ib - s_ipref[lo]);
        cur.pass = rel / nrc;
        cur.chunk = rel - cur.pass * nrc;
        cur.g = 0;
        cur.idx = 0;
        cur.e = __builtin_amdgcn_readfirstlane(s_act[lo]);
        cur.c = __builtin_amdgcn_readfirstlane(s_cnt[lo]);
        cur.o = __builtin_amdgcn_readfirstlane(s_off[lo]);
    }
    // advance by n steps, n = 1 or 8 (NG is a multiple of 8, so 8 steps never
    // cross a row-chunk boundary without landing on it)
    auto advance = [&](Cursor& q, int n) {
        q.idx += n;
        q.g += n;
        if (q.g < NG) return;
        q.g = 0;
        if (++q.chunk < nrc) return;
        q.chunk = 0;
        if ((++q.pass) * P < q.c) return;
        q.pass = 0;
        if (++q.u < U) {
            q.e = __builtin_amdgcn_readfirstlane(s_act[q.u]);
            q.c = __builtin_amdgcn_readfirstlane(s_cnt[q.u]);
            q.o = __builtin_amdgcn_readfirstlane(s_off[q.u]);
        }
    };

    const uint32_t mat_bytes = rb * (uint32_t)N;
    const uint32_t lrow = (uint32_t)(wave * 16 + (lane & 15));
    const uint32_t lq = (uint32_t)(lane >> 4);
    // lane part of a weight offset, the offset step from one group to the
    // next and from a lane's first 16-byte piece of a group to its second
    // (fp8): row-major (row lrow, bytes 64 g + 16 lq; fp8 codes 128 g + 32 lq)
    // or tiled (16-row set `wave` of the item, 1 KB per group and piece,
    // lane-ordered 16-byte pieces)
    const uint32_t woff_l =
        TILED ? (uint32_t)wave * 16u * rb + (uint32_t)lane * 16u : lrow * rb + lq * (FP8 ? 32u : 16u);
    constexpr uint32_t kGroupStep = TILED ? 1024u * NW : (FP8 ? 128u : 64u);
    constexpr uint32_t kPieceStep = TILED ? 1024u : 16u;
    const uint32_t soff_l = lrow * srow;                      // lane part of a scale offset
    const uint32_t lrow16 = (uint32_t)(lane & 15);

    // ---- weight loads of steps q and q+1 into ring slots S, S+1: the two
    // halves of the same 128-byte lines, back to back (zeros past the range);
    // MX: at the first step of a four-group chunk (position P16 of the 16-step
    // unroll a multiple of 4) the chunk's scale bytes go out first
    u32x4_t wq[RING][G][NW];
    u32x4_t sq[4][G];                             // MX: scale bytes of four groups, per row
    auto weight_ptr = [&](const Cursor& q, int m) -> const uint8_t* {
        if (q.e >= 0) return (m == 0 ? a.w0 : a.w1) + (size_t)q.e * mat_bytes;
        return m == 0 ? a.sw0 : a.sw1;
    };
    auto scale_ptr = [&](const Cursor& q, int m) -> const uint8_t* {
        const uint16_t* sp = q.e >= 0 ? (m == 0 ? a.s0 : a.s1) : (m == 0 ? a.ss0 : a.ss1);
        return reinterpret_cast<const uint8_t*>(sp) + (q.e >= 0 ? (size_t)q.e * N * srow : 0);
    };
    auto issue_pair = [&](Cursor& q, auto slot, auto pos) {
        constexpr int S = decltype(slot)::value, P16 = decltype(pos)::value;
        Cursor q1 = q;
        advance(q1, 1);
        const uint32_t n0 = q.idx < nsteps ? mat_bytes : 0u, n1 = q1.idx < nsteps ? mat_bytes : 0u;
        if constexpr (MX && P16 % 4 == 0) {
            // row lrow's scale bytes of groups q.g .. q.g + 3 (q.g is a multiple of 4)
            const uint32_t so = soff_l + (uint32_t)q.chunk * kItemRows * srow + (uint32_t)q.g * 4u;
            const uint32_t sn = q.idx < nsteps ? (uint32_t)N * srow : 0u;
#pragma unroll
            for (int m = 0; m < G; ++m) sq[(P16 / 4) % 4][m] = ld16(rsrc(scale_ptr(q, m), sn), so);
        }
        const uint32_t o0 = woff_l + (uint32_t)q.chunk * kItemRows * rb + (uint32_t)q.g * kGroupStep;
        const uint32_t o1 = woff_l + (uint32_t)q1.chunk * kItemRows * rb + (uint32_t)q1.g * kGroupStep;
#pragma unroll
        for (int m = 0; m < G; ++m)
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                wq[S][m][w] = ld16<TILED ? kNonTemporal : 0>(rsrc(weight_ptr(q, m), n0), o0 + kPieceStep * w);
                wq[S + 1][m][w] = ld16<TILED ? kNonTemporal : 0>(rsrc(weight_ptr(q1, m), n1), o1 + kPieceStep * w);
            }
        q = q1;
        advance(q, 1);
    };
    // fp16 scales of a 16-row set (16 rows x NG x 2 bytes, contiguous): lane
    // (row n, q) loads chunks q and q + 4 (8 groups each) of row n with two
    // back-to-back loads that together cover every line of the set once
    u32x4_t snext[G][2], scur[G][2];
    auto issue_scales = [&](const Cursor& q) {
        const uint32_t so = soff_l + (uint32_t)q.chunk * kItemRows * srow + lq * 16u;
        const uint32_t sn = q.idx < nsteps ? (uint32_t)N * srow : 0u;
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const uint16_t* sp = q.e >= 0 ? (m == 0 ? a.s0 : a.s1) + (size_t)q.e * N * NG
                                          : (m == 0 ? a.ss0 : a.ss1);
            snext[m][0] = ld16(rsrc(sp, sn), so);
            // chunks 4..7 exist only past 32 groups; else an offset the range
            // check rejects (no memory access; a conditional load would make
            // the compiler wait for it at once)
            snext[m][1] = ld16(rsrc(sp, sn), NG > 32 ? so + 64u : 0xffffffffu);
        }
    };

    // ---- staging of a token pass into LDS (block-wide)
    int tag_u = -1, tag_pass = -1;
    auto stage = [&](const Cursor& q) {
        __syncthreads();   // every wave is done with the previous rows
        const int j0 = q.pass * P;
        const int nt = min(P, q.c - j0);
        const bool routed = q.e >= 0;
        const uint16_t* in = routed ? a.in : a.sin;
        if (tid < 16 && tid < nt) {
            const int p = q.o + j0 + tid;
            s_src[tid] = (MODE == 0 && routed && a.perm) ? a.perm[p] / a.topk : p;
        }
        if constexpr (!MX)
            for (int i = tid; i < NG * 16; i += kThreads)   // group sums of the padded slots
                if ((i & 15) >= nt) xsum[i] = 0.f;
        __syncthreads();
        // nt rows of K/8 16-byte chunks; nch is a multiple of 128, so every
        // wave is either wholly inside or wholly past the range, and 16
        // consecutive lanes hold the 16 chunks of one scale group
        const int nch = K / 8;
        const int total = nt * nch;
        constexpr int B = 4;
        for (int i0 = wave * 64; i0 < total; i0 += kThreads * B) {
            uint4 v[B];
            int t[B], ch[B];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const int i = i0 + j * kThreads + lane;
                t[j] = i / nch;
                ch[j] = i - t[j] * nch;
                if (i0 + j * kThreads < total)
                    v[j] = *reinterpret_cast<const uint4*>(in + (size_t)s_src[t[j]] * K + (size_t)ch[j] * 8);
            }
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (i0 + j * kThreads >= total) break;
                u32x4_t o;
                if constexpr (MX) {
                    // plain element order: the widened codes come out in it
                    o = u32x4_t{v[j].x, v[j].y, v[j].z, v[j].w};
                } else {
                    // elements (0,1)(2,3)(4,5)(6,7) -> pairs (0,4)(1,5)(2,6)(3,7)
                    o.x = (v[j].x & 0xffffu) | (v[j].z << 16);
                    o.y = (v[j].x >> 16) | (v[j].z & 0xffff0000u);
                    o.z = (v[j].y & 0xffffu) | (v[j].w << 16);
                    o.w = (v[j].y >> 16) | (v[j].w & 0xffff0000u);
                }
                *reinterpret_cast<u32x4_t*>(xrows + (size_t)t[j] * RS + (size_t)ch[j] * 16) = o;
                if constexpr (!MX) {
                    float sum = bf16_lo(v[j].x) + bf16_hi(v[j].x) + bf16_lo(v[j].y) + bf16_hi(v[j].y) +
                                bf16_lo(v[j].z) + bf16_hi(v[j].z) + bf16_lo(v[j].w) + bf16_hi(v[j].w);
                    sum = group_sum<16>(sum);
                    if ((ch[j] & 15) == 0) xsum[(ch[j] >> 4) * 16 + t[j]] = sum;
                }
            }
        }
        __syncthreads();
        tag_u = q.u;
        tag_pass = q.pass;
    };

    // per-lane LDS addresses of the A fragments and of the group sums
    const uint32_t tok = (uint32_t)(lane & 15);
    uint32_t xa = 0;                            // set at each stage
    const uint32_t xs_l = lq * 16u;             // bytes: tokens 4q..4q+3 of a group's 16
    floatx4 acc[G];
#pragma unroll
    for (int m = 0; m < G; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Cursor& q, auto slot, auto half, auto pos) {
        constexpr int S = decltype(slot)::value,
                      H = decltype(half)::value,   // group index within its 8-group chunk
                      P16 = decltype(pos)::value;  // position in the 16-step unroll
        const char* xg = xrows + xa + (uint32_t)q.g * 256u;
        u32x4_t af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const u32x4_t*>(xg + i * 16);
        if constexpr (MX) {
            // this lane's 32 codes share the scale of byte 4 (g % 4) + l/16 of the chunk
#pragma unroll
            for (int m = 0; m < G; ++m) {
                const uint32_t code = (sq[(P16 / 4) % 4][m][P16 % 4] >> (8u * lq)) & 0xffu;
                const float sc = mx_scale(code);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    u32x4_t b;
                    if constexpr (FP8) {
                        const uint32_t w0 = wq[S][m][i >> 1][2 * (i & 1)], w1 = wq[S][m][i >> 1][2 * (i & 1) + 1];
                        b.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false));
                        b.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true));
                        b.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false));
                        b.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true));
                    } else {
                        const uint32_t w = wq[S][m][0][i];
                        b.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
                        b.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
                        b.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
                        b.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
                    }
                    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[i]),
                                                                      __builtin_bit_cast(bf16x8_t, b), acc[m], 0, 0, 0);
                }
            }
            return;
        }
        // the scale of (row n, group g) sits in lane n + 16 (c % 4), register
        // c / 4 of the row set's scales, c = g / 8
        const int c8 = q.g >> 3;
        const int src = (int)((lrow16 + 16u * (uint32_t)(c8 & 3)) << 2);
        const floatx4 xs = *reinterpret_cast<const floatx4*>(
            reinterpret_cast<const char*>(xsum) + (uint32_t)q.g * 64u + xs_l);
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const uint32_t wd[4] = {wq[S][m][0].x, wq[S][m][0].y, wq[S][m][0].z, wq[S][m][0].w};
            floatx4 c = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4_t b;
                b.x = (wd[i] & 0x000f000fu) ^ 0x43084308u;
                b.y = ((wd[i] >> 4) & 0x000f000fu) ^ 0x43084308u;
                b.z = ((wd[i] >> 8) & 0x000f000fu) ^ 0x43084308u;
                b.w = ((wd[i] >> 12) & 0x000f000fu) ^ 0x43084308u;
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[i]),
                                                             __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
            }
            const uint32_t own = (c8 >> 2) ? scur[m][1][H >> 1] : scur[m][0][H >> 1];
            const uint32_t sw = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)own);
            const float sc = f16_to_f32((uint16_t)((H & 1) ? (sw >> 16) : (sw & 0xffffu)));
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[m][v] = fmaf(sc, fmaf(-136.0f, xs[v], c[v]), acc[m][v]);
        }
    };

    auto epilogue = [&](const Cursor& q) {
        const int j0 = q.pass * P;
        const int nt = min(P, q.c - j0);
        const int row = q.chunk * kItemRows + wave * 16 + (lane & 15);
        void* out = q.e >= 0 ? a.out : a.sout;
        if (row < N) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = (int)lq * 4 + v;
                if (t < nt) {
                    const size_t oi = (size_t)(q.o + j0 + t) * N + row;
                    if constexpr (MODE == 0)
                        reinterpret_cast<uint16_t*>(out)[oi] = f32_to_bf16(silu(acc[0][v]) * acc[1][v]);
                    else
                        reinterpret_cast<float*>(out)[oi] = acc[0][v];
                }
            }
        }
#pragma unroll
        for (int m = 0; m < G; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    };

    // ---- prologue: RING steps of weights and the first scale chunk in flight
    // Loads complete in order, so a row set's scales go out as far ahead as
    // the weight ring reaches (8 steps)
    Cursor L = cur;       // next step whose weights are loaded
    Cursor Sc = cur;      // int4: loads a row set's scales when it reaches its start
    if constexpr (!MX) {
        issue_scales(Sc);
        advance(Sc, 8);
    }
    static_for<0, RING / 2>([&](auto k) {
        issue_pair(L, ic<2 * decltype(k)::value>{}, ic<2 * decltype(k)::value>{});
    });

    // One step at unrolled position k (0..15): ring slot k % RING.  Every
    // other step refills the two slots just consumed with the steps RING
    // ahead.  Steps carry no exit test, so the compiler's wait counts see the
    // whole ring.
    Cursor C = cur;
    auto step = [&](auto kk) {
        constexpr int k = decltype(kk)::value;
        if constexpr (k % 8 == 0) {
            if (C.g == 0 && (C.u != tag_u || C.pass != tag_pass)) {
                stage(C);
                const int nt = min(P, C.c - C.pass * P);
                xa = (tok < (uint32_t)nt ? tok : (uint32_t)P) * RS + lq * 64u;
            }
        }
        if constexpr (!MX && k % 8 == 0) {
            if (C.g == 0) {
#pragma unroll
                for (int m = 0; m < G; ++m) { scur[m][0] = snext[m][0]; scur[m][1] = snext[m][1]; }
            }
        }
        compute(C, ic<k % RING>{}, ic<k % 8>{}, ic<k>{});
        if constexpr (!MX && k % 8 == 0) {
            if (Sc.g == 0) issue_scales(Sc);
            advance(Sc, 8);
        }
        if constexpr (k % 8 == 7) {
            if (C.g == NG - 1) epilogue(C);
        }
        if constexpr (k % 2 == 1) issue_pair(L, ic<(k - 1) % RING>{}, ic<(k - 1 + RING) % 16>{});
        advance(C, 1);
    };
    // nsteps is a multiple of 8 (NG is)
    for (int n = nsteps >> 4; n > 0; --n) static_for<0, 16>(step);
    if (nsteps & 8) static_for<0, 8>(step);
}

// ------------------------------------------------------------------ host side

// Token rows per pass for a given K: P rows plus the zero row plus the group
// sums must fit the LDS of one block.
static int i4_pass_tokens(int K) {
    const long rs = (long)K * 2 + 16;
    const long xs = (long)(K / 128) * 16 * 4;
    long p = (kLdsBytes - xs - kStaticLds) / rs - 1;
    if (p > 16) p = 16;
    return (int)p;
}

bool i4mfma_supported(int K, int N, int fmt) {
    // K a multiple of 8 groups of 128; int4: at most 64 groups (two scale
    // registers per row set); MX scales come in four-group chunks, no bound
    if (K % 1024 != 0 || K <= 0 || N <= 0 || (fmt == kFmtInt4 && K > 8192)) return false;
    if (i4_pass_tokens(K) < 1) return false;
    // 32-bit buffer offsets of a matrix, including the padded last chunk
    const size_t rb = fmt == kFmtFp8 ? (size_t)K : (size_t)K / 2;
    return (size_t)(N + kItemRows) * rb < ((size_t)1 << 31);
}

hipError_t launch_i4mfma(int mode, bool tiled, const GemvArgs* routed, const GemvArgs* shared, hipStream_t s,
                         int fmt) {
    if (fmt != kFmtInt4 && fmt != kFmtFp4 && fmt != kFmtFp8) return hipErrorInvalidValue;
    const GemvArgs& g = routed ? *routed : *shared;
    I4Args a{};
    if (routed) {
        a.w0 = reinterpret_cast<const uint8_t*>(routed->w0);
        a.w1 = reinterpret_cast<const uint8_t*>(routed->w1);
        a.s0 = routed->s0;
        a.s1 = routed->s1;
        a.in = reinterpret_cast<const uint16_t*>(routed->in);
        a.out = routed->out;
        a.counts = routed->counts;
        a.offsets = routed->offsets;
        a.perm = routed->perm;
        a.topk = routed->topk;
        a.E = routed->E;
        a.tau = routed->tau;
        if (!a.counts || !a.offsets) return hipErrorInvalidValue;
    }
    if (shared) {
        a.sw0 = reinterpret_cast<const uint8_t*>(shared->w0);
        a.sw1 = reinterpret_cast<const uint8_t*>(shared->w1);
        a.ss0 = shared->s0;
        a.ss1 = shared->s1;
        a.sin = reinterpret_cast<const uint16_t*>(shared->in);
        a.sout = shared->out;
        if (!a.sw0) return hipErrorInvalidValue;
    }
    a.N = g.N;
    a.K = g.K;
    a.T = g.T;
    a.P = i4_pass_tokens(g.K);
    if (a.E > kMaxE || a.P < 1) return hipErrorInvalidValue;
    const size_t lds = (size_t)(a.P + 1) * ((size_t)g.K * 2 + 16) + (size_t)(g.K / 128) * 16 * 4;

    const int n_cu = cu_count();
    // 8 scale groups per wave in flight: 16 KB (gate/up) or 8 KB (down); fp8
    // codes take twice the bytes per group, so 4 groups
    auto k = mode == 0 ? (fmt == kFmtFp8   ? (tiled ? i4_mfma_kernel<0, 4, true, kFmtFp8> : i4_mfma_kernel<0, 4, false, kFmtFp8>)
                          : fmt == kFmtFp4 ? (tiled ? i4_mfma_kernel<0, 8, true, kFmtFp4> : i4_mfma_kernel<0, 8, false, kFmtFp4>)
                          : tiled          ? i4_mfma_kernel<0, 8, true, kFmtInt4>
                                           : i4_mfma_kernel<0, 8, false, kFmtInt4>)
                       : (fmt == kFmtFp8   ? (tiled ? i4_mfma_kernel<1, 4, true, kFmtFp8> : i4_mfma_kernel<1, 4, false, kFmtFp8>)
                          : fmt == kFmtFp4 ? (tiled ? i4_mfma_kernel<1, 8, true, kFmtFp4> : i4_mfma_kernel<1, 8, false, kFmtFp4>)
                          : tiled          ? i4_mfma_kernel<1, 8, true, kFmtInt4>
                                           : i4_mfma_kernel<1, 8, false, kFmtInt4>);
    // dynamic LDS beyond 64 KB: the budget left next to the static arrays,
    // set once per device and kernel variant
    static std::atomic<int> attr_set[12][kMaxDevices];
    const int ki = mode * 6 + 2 * fmt + (tiled ? 1 : 0);
    per_device_int(attr_set[ki], [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)(kLdsBytes - kStaticLds));
        return 1;
    });
    hipLaunchKernelGGL(k, dim3(n_cu), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

// Row-major code bytes -> the tiled layout the kernel above streams, PW
// 16-byte pieces per lane and group (4-bit codes 1, fp8 codes 2): within each
// matrix, 16-byte piece (set, g, w, q*16 + r) of the output (set-major, then
// group g, then piece w, then lane) is bytes [64 PW g + 16 PW q + 16 w, +16)
// of row 16 set + r.  A permutation of 16-byte pieces: one thread per output
// piece, coalesced stores.
template <int PW>
__global__ __launch_bounds__(256) void pack_tiled_kernel(const u32x4_t* __restrict__ src,
                                                         u32x4_t* __restrict__ dst, size_t n_pieces, int N, int K) {
    const size_t per_row = (size_t)K * PW / 32;        // 16-byte pieces per row
    const size_t per_mat = (size_t)N * per_row;
    const int NG = K / 128;
    for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_pieces;
         j += (size_t)gridDim.x * blockDim.x) {
        const size_t mat = j / per_mat, rem = j - mat * per_mat;
        const int lane = (int)(rem & 63);
        const size_t t = (rem >> 6) / PW;
        const int w = (int)((rem >> 6) - t * PW);
        const size_t set = t / NG;
        const int g = (int)(t - set * NG);
        const size_t row = set * 16 + (lane & 15);
        dst[j] = src[mat * per_mat + row * per_row + (size_t)g * 4 * PW + (size_t)(lane >> 4) * PW + w];
    }
}

template <int PW>
static hipError_t launch_pack(const void* src, void* dst, size_t n_mats, int N, int K, hipStream_t s) {
    const size_t n = n_mats * (size_t)N * (size_t)(K / 32) * PW;
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(pack_tiled_kernel<PW>, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s,
                       reinterpret_cast<const u32x4_t*>(src), reinterpret_cast<u32x4_t*>(dst), n, N, K);
    return hipGetLastError();
}

hipError_t launch_pack_int4_tiled(const void* src, void* dst, size_t n_mats, int N, int K, hipStream_t s) {
    return launch_pack<1>(src, dst, n_mats, N, K, s);
}

hipError_t launch_pack_mxfp8_tiled(const void* src, void* dst, size_t n_mats, int N, int K, hipStream_t s) {
    return launch_pack<2>(src, dst, n_mats, N, K, s);
}

}  // namespace moe
