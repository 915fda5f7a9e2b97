// Expert FFN for quantised expert weights on the matrix cores: int4 with
// fp16 group scales (groups of 128 or 64 K elements) and the OCP microscaling
// formats MXFP4 (E2M1 elements) and MXFP8 (E4M3 elements), both with one E8M0
// power-of-two scale per 32 K elements.
//
// [P5] "一只蜂鸟如何喂饱九头大象" §7.3: int4 experts with group scales
// (group size 64 against 128 and per-row); §6: models whose checkpoints ship
// native MXFP4 or FP8 weights.  [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎"
// §3.3: a tiled expert GEMM over the tokens of each expert.
//
// gfx950 design: a grouped GEMM for expert groups of any size (int4-g128
// groups above a threshold; every group of the other formats).  The weights
// stay quantised in HBM and are widened to bf16 in registers right before
// v_mfma_f32_32x32x16_bf16, so the matrix cores see the same operands a bf16
// layer would:
//  * MXFP4 / MXFP8: v_cvt_scalef32_pk_bf16_fp4 / _fp8 turn two codes into two
//    bf16 already multiplied by the block's power-of-two scale -- exact, since
//    an E2M1 or E4M3 value times 2^e is a bf16 number;
//  * int4: q (a signed bit-field extract) times the fp16 group scale in fp32,
//    rounded to the nearest bf16 (the one rounding of this path: at most 2^-9
//    of the weight).
// Tiles: 128 token rows x 128 weight rows (gate/up: 64 gate rows and the 64
// matching up rows, so each lane holds g and u of the same (token, column) and
// the SwiGLU epilogue needs no exchange), one 256-thread block of four waves,
// wave (wm, wn) owning 64 tokens x 64 weight rows as 2 x 2 fragments of 32x32.
// The product is token-major (tokens as the MFMA A operand): a lane's
// accumulators hold one weight row for 16 tokens.  K runs in pairs of 64:
//  * token rows (gathered through perm for gate/up) go global -> registers ->
//    LDS (two pair slots, 128-byte rows with the 16-byte chunks XOR-swizzled
//    by (row/2)&7, conflict-free fragment reads), one pair ahead;
//  * weight codes and scales go global -> registers straight in operand
//    layout, two pairs ahead (a ring of three pairs): lane l takes row
//    l%32 of its fragment and the 32 K elements [32h, 32h+32) of the pair,
//    h = l/32, so one 16-byte load holds a lane's int4 or fp4 codes of a pair
//    (two for fp8), and MFMA step s of the pair multiplies K elements
//    32h + 8s .. +7 of both operands (the same K permutation on both sides);
//  * buffer loads with the range check return zeros for rows past N and token
//    rows past the group, so no load is branched.
// A persistent grid (two blocks per CU) walks the (M-tile, N-tile) list with N
// fastest, so the blocks of one XCD share an M-tile's token rows in L2.
#include <type_traits>

#include "common.h"
#include "devinfo.h"
#include "kernels.h"

namespace moe {

namespace {

typedef __bf16 dq_bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 dq_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float dq_floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int dq_u32x4_t __attribute__((ext_vector_type(4)));

constexpr int DQ_BM = 128;          // token rows of a tile
constexpr int DQ_PK = 64;           // K per pair
constexpr int DQ_THREADS = 256;
constexpr uint32_t DQ_OOB = 0x80000000u;   // beyond any buffer: the range check yields 0

enum { DQ_INT4 = 0, DQ_MXFP4 = 1, DQ_MXFP8 = 2 };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dq_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

// element offset of logical 16-byte chunk ch (0..7) of row r in a pair slot
__device__ __forceinline__ int dq_swz(int r, int ch) { return r * DQ_PK + ((ch ^ ((r >> 1) & 7)) << 3); }

struct DqArgs {
    const uint8_t* w0;       // gate (mode 0) or down (mode 1) codes, [E][N][K*bits/8]
    const uint8_t* w1;       // up codes (mode 0)
    const uint8_t* s0;       // scales of w0: fp16 [E][N][K/gs] (int4) or E8M0 [E][N][K/32]
    const uint8_t* s1;
    const uint16_t* in;      // x [T][K] (mode 0) or h [T*k][K] (mode 1), bf16
    void* out;               // h bf16 [T*k][N] (mode 0) or y_perm fp32 [T*k][N] (mode 1)
    const int32_t* perm;
    const int32_t* tiles;    // plan: expert[max_mt], row0[max_mt], rows[max_mt], count
    int N, K, topk, max_mt, in_rows, gs;
};

// One K step (8 K elements per lane) of a weight fragment, widened to bf16.
// c: the lane's codes of the pair (16 bytes; fp8: 32 in c and c2), s: the
// step (0..3), scale: fp32 group scale (int4) or the power of two (MX).
template <int FMT>
__device__ __forceinline__ dq_bf16x8_t dq_widen(const dq_u32x4_t& c, const dq_u32x4_t& c2, int s, float scale) {
    uint32_t p[4];
    if constexpr (FMT == DQ_INT4) {
        // signed 4-bit fields: v_bfe_i32 sign-extends, but the builtin is
        // typed unsigned, so its result is read back as int
        const uint32_t w = c[s];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = (float)(int)__builtin_amdgcn_sbfe(w, 8 * i, 4) * scale;
            const float hi = (float)(int)__builtin_amdgcn_sbfe(w, 8 * i + 4, 4) * scale;
            p[i] = pack_bf16x2(lo, hi);
        }
    } else if constexpr (FMT == DQ_MXFP4) {
        const uint32_t w = c[s];
        p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
        p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
        p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
        p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    } else {
        // 8 bytes of step s: words 2s and 2s+1 of the lane's 32 bytes
        const uint32_t w0 = s < 2 ? c[2 * s] : c2[2 * s - 4];
        const uint32_t w1 = s < 2 ? c[2 * s + 1] : c2[2 * s - 3];
        p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false));
        p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true));
        p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false));
        p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true));
    }
    dq_u32x4_t r = {p[0], p[1], p[2], p[3]};
    return __builtin_bit_cast(dq_bf16x8_t, r);
}

// E8M0 code -> the fp32 power of two 2^(code - 127) (code 0: 2^-127, subnormal)
__device__ __forceinline__ float dq_e8m0(uint32_t code) {
    return __uint_as_float(code ? (code << 23) : 0x00400000u);
}

template <int MODE, int FMT>
__global__ __launch_bounds__(DQ_THREADS, 2) void dq_ffn_kernel(DqArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][DQ_BM * DQ_PK];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int h = lane >> 5, r32 = lane & 31;
    const int K = a.K, N = a.N;
    const int n_mt = a.tiles[3 * a.max_mt];
    const int nN = MODE == 0 ? (N + 63) / 64 : (N + 127) / 128;
    const int total = n_mt * nN;
    const int P = K / DQ_PK;
    // code bytes per weight row and per pair half; scales per row and their size
    const uint32_t crow = FMT == DQ_MXFP8 ? (uint32_t)K : (uint32_t)K / 2;
    const uint32_t chalf = FMT == DQ_MXFP8 ? 32u : 16u;
    const int sper = FMT == DQ_INT4 ? K / a.gs : K / 32;
    const uint32_t ssz = FMT == DQ_INT4 ? 2u : 1u;
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t RA = dq_rsrc(a.in, (uint32_t)a.in_rows * row_bytes);
    // blocks are dealt round-robin to the 8 XCDs: consecutive slots share one
    const int nblk = gridDim.x;
    const int per = nblk / 8;
    const int slot = (nblk % 8 == 0) ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;

    for (int task = slot; task < total; task += nblk) {
        const int mt = task / nN, nt = task - mt * nN;
        const int e = a.tiles[mt], p0 = a.tiles[a.max_mt + mt], rows = a.tiles[2 * a.max_mt + mt];
        // token-row loads: rows 32*wave + 8i + lane/8, 16-byte chunk lane%8
        uint32_t aoff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 32 * wave + 8 * i + (lane >> 3);
            int src = -1;
            if (r < rows) src = MODE == 0 ? a.perm[p0 + r] / a.topk : p0 + r;
            aoff[i] = src >= 0 ? (uint32_t)src * row_bytes + (uint32_t)(lane & 7) * 16u : DQ_OOB;
        }
        // this lane's weight row of fragment ni, its code and scale buffers
        __amdgpu_buffer_rsrc_t RW[2], RS[2];
        uint32_t woff[2], soff[2];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            const uint8_t* wb = (MODE == 0 && ni == 1) ? a.w1 : a.w0;
            const uint8_t* sb = (MODE == 0 && ni == 1) ? a.s1 : a.s0;
            const int row = MODE == 0 ? nt * 64 + 32 * wn + r32 : nt * 128 + 64 * wn + 32 * ni + r32;
            RW[ni] = dq_rsrc(wb + (size_t)e * N * crow, (uint32_t)N * crow);
            RS[ni] = dq_rsrc(sb + (size_t)e * N * sper * ssz, (uint32_t)N * (uint32_t)sper * ssz);
            woff[ni] = row < N ? (uint32_t)row * crow + (uint32_t)h * chalf : DQ_OOB;
            soff[ni] = row < N ? (uint32_t)row * (uint32_t)sper * ssz : DQ_OOB;
        }
        dq_floatx16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        // register rings: token chunks of the next pair; codes and scales of
        // three pairs (the one in use and the next two)
        dq_u32x4_t ta[4];
        dq_u32x4_t wc[3][2], wc2[3][2];
        float ws[3][2];
        auto load_tokens = [&](int j) __attribute__((always_inline)) {
            const uint32_t kb = (uint32_t)j * DQ_PK * 2u;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ta[i] = __builtin_amdgcn_raw_buffer_load_b128(RA, aoff[i] == DQ_OOB ? DQ_OOB : aoff[i] + kb, 0, 0);
        };
        auto store_tokens = [&](int j) __attribute__((always_inline)) {
            uint16_t* dst = sA[j & 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * wave + 8 * i + (lane >> 3);
                *reinterpret_cast<dq_u32x4_t*>(&dst[dq_swz(r, lane & 7)]) = ta[i];
            }
        };
        auto load_weights = [&](int j, auto ring) __attribute__((always_inline)) {
            constexpr int R = decltype(ring)::value;
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const bool in = woff[ni] != DQ_OOB && j < P;
                const uint32_t o = in ? woff[ni] + (uint32_t)j * 2u * chalf : DQ_OOB;
                wc[R][ni] = __builtin_amdgcn_raw_buffer_load_b128(RW[ni], o, 0, 0);
                if constexpr (FMT == DQ_MXFP8)
                    wc2[R][ni] = __builtin_amdgcn_raw_buffer_load_b128(RW[ni], in ? o + 16u : DQ_OOB, 0, 0);
                if constexpr (FMT == DQ_INT4) {
                    const uint32_t g = (uint32_t)(j * DQ_PK / a.gs);
                    const uint16_t sv = __builtin_amdgcn_raw_buffer_load_b16(
                        RS[ni], in ? soff[ni] + g * 2u : DQ_OOB, 0, 0);
                    ws[R][ni] = f16_to_f32(sv);
                } else {
                    const uint32_t g = (uint32_t)(2 * j + h);
                    const uint8_t sv = __builtin_amdgcn_raw_buffer_load_b8(RS[ni], in ? soff[ni] + g : DQ_OOB, 0, 0);
                    ws[R][ni] = dq_e8m0(sv);
                }
            }
        };
        // pair j from ring slot R: four K steps of 2 x 2 MFMAs
        auto compute = [&](int j, auto ring) __attribute__((always_inline)) {
            constexpr int R = decltype(ring)::value;
            const uint16_t* src = sA[j & 1];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                dq_bf16x8_t fa[2], fb[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    fa[mi] = *reinterpret_cast<const dq_bf16x8_t*>(&src[dq_swz(64 * wm + 32 * mi + r32, 4 * h + s)]);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) fb[ni] = dq_widen<FMT>(wc[R][ni], wc2[R][ni], s, ws[R][ni]);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
            }
        };
        // one pair: the barrier ends every read of the other token slot and
        // publishes pair j's tokens; then pair j+1's tokens go to that slot,
        // pair j+2's tokens are requested, pair j is multiplied and its ring
        // slot is refilled with pair j+3's weights
        auto step = [&](int j, auto ring) __attribute__((always_inline)) {
            __syncthreads();
            if (j + 1 < P) store_tokens(j + 1);
            if (j + 2 < P) load_tokens(j + 2);
            compute(j, ring);
            load_weights(j + 3, ring);
        };

        // prologue: pair 0's tokens in LDS, pair 1's in registers, weights of
        // pairs 0..2 requested
        __syncthreads();                      // the previous task's reads of sA are done
        load_tokens(0);
        load_weights(0, std::integral_constant<int, 0>{});
        load_weights(1, std::integral_constant<int, 1>{});
        load_weights(2, std::integral_constant<int, 2>{});
        store_tokens(0);
        if (P > 1) load_tokens(1);
        for (int j = 0; j < P; j += 3) {
            step(j, std::integral_constant<int, 0>{});
            if (j + 1 < P) step(j + 1, std::integral_constant<int, 1>{});
            if (j + 2 < P) step(j + 2, std::integral_constant<int, 2>{});
        }

        // epilogue: lane l holds weight row (fragment ni) l%32 for tokens
        // 8*(v/4) + 4*(l/32) + v%4 of fragment mi
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 64 * wm + 32 * mi + 8 * (v >> 2) + 4 * h + (v & 3);
                if (r >= rows) continue;
                const size_t orow = (size_t)(p0 + r) * N;
                if constexpr (MODE == 0) {
                    const int f = nt * 64 + 32 * wn + r32;
                    if (f < N) {
                        const float hv = silu(acc[mi][0][v]) * acc[mi][1][v];
                        reinterpret_cast<uint16_t*>(a.out)[orow + f] = (uint16_t)pack_bf16x2(hv, 0.f);
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        const int n = nt * 128 + 64 * wn + 32 * ni + r32;
                        if (n < N) reinterpret_cast<float*>(a.out)[orow + n] = acc[mi][ni][v];
                    }
                }
            }
        }
    }
}

// One 256-thread block: per expert with more than tau rows, ceil(rows/128)
// tiles; an exclusive scan over the experts places them.
__global__ __launch_bounds__(256) void dq_plan_kernel(const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ offsets, int E, int tau,
                                                     int32_t* __restrict__ tiles, int max_mt) {
    __shared__ int s[2][256];
    const int tid = threadIdx.x;
    int c = 0, nb = 0;
    if (tid < E) {
        c = counts[tid];
        if (c > tau && c > 0) nb = (c + DQ_BM - 1) / DQ_BM;
    }
    int cur = 0;
    s[0][tid] = nb;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        int v = s[cur][tid];
        if (tid >= o) v += s[cur][tid - o];
        s[cur ^ 1][tid] = v;
        cur ^= 1;
        __syncthreads();
    }
    if (tid < E) {
        const int o0 = offsets[tid];
        const int b = s[cur][tid] - nb;
        for (int i = 0; i < nb; ++i) {
            tiles[b + i] = tid;
            tiles[max_mt + b + i] = o0 + i * DQ_BM;
            tiles[2 * max_mt + b + i] = min(DQ_BM, c - i * DQ_BM);
        }
    }
    if (tid == 255) tiles[3 * max_mt] = s[cur][255];
}

}  // namespace

int dq_max_tiles(int T, int k, int E) { return (T * k + DQ_BM - 1) / DQ_BM + E; }
int dq_plan_ints(int T, int k, int E) { return 3 * dq_max_tiles(T, k, E) + 1; }

bool dq_supported(int K, int N) {
    // whole K pairs; 32-bit buffer offsets of a matrix (fp8: one byte per element)
    return K > 0 && K % DQ_PK == 0 && N > 0 && (size_t)N * (size_t)K < ((size_t)1 << 31);
}

hipError_t launch_dq_plan(const int32_t* counts, const int32_t* offsets, int E, int tau, int32_t* tiles,
                          int max_mt, hipStream_t s) {
    if (E > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dq_plan_kernel, dim3(1), dim3(256), 0, s, counts, offsets, E, tau, tiles, max_mt);
    return hipGetLastError();
}

hipError_t launch_dq_ffn(int mode, int fmt, int gs, const void* w0, const void* w1, const void* s0, const void* s1,
                         const void* in, void* out, const int32_t* perm, const int32_t* tiles, int N, int K, int topk,
                         int max_mt, int in_rows, hipStream_t s) {
    if (!dq_supported(K, N) || (fmt == DQ_INT4 && (gs != 64 && gs != 128)) || fmt < 0 || fmt > 2)
        return hipErrorInvalidValue;
    DqArgs a;
    a.w0 = reinterpret_cast<const uint8_t*>(w0);
    a.w1 = reinterpret_cast<const uint8_t*>(w1);
    a.s0 = reinterpret_cast<const uint8_t*>(s0);
    a.s1 = reinterpret_cast<const uint8_t*>(s1);
    a.in = reinterpret_cast<const uint16_t*>(in);
    a.out = out;
    a.perm = perm;
    a.tiles = tiles;
    a.N = N;
    a.K = K;
    a.topk = topk;
    a.max_mt = max_mt;
    a.in_rows = in_rows;
    a.gs = fmt == DQ_INT4 ? gs : 32;
    const int nN = mode == 0 ? (N + 63) / 64 : (N + 127) / 128;
    const long slots = (long)max_mt * nN;
    const long cap = 2L * cu_count();
    const int grid = (int)(slots < cap ? slots : cap);
#define DQ_LAUNCH(M, F) hipLaunchKernelGGL((dq_ffn_kernel<M, F>), dim3(grid), dim3(DQ_THREADS), 0, s, a)
    if (mode == 0) {
        if (fmt == DQ_INT4) DQ_LAUNCH(0, DQ_INT4);
        else if (fmt == DQ_MXFP4) DQ_LAUNCH(0, DQ_MXFP4);
        else DQ_LAUNCH(0, DQ_MXFP8);
    } else {
        if (fmt == DQ_INT4) DQ_LAUNCH(1, DQ_INT4);
        else if (fmt == DQ_MXFP4) DQ_LAUNCH(1, DQ_MXFP4);
        else DQ_LAUNCH(1, DQ_MXFP8);
    }
#undef DQ_LAUNCH
    return hipGetLastError();
}

}  // namespace moe
