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
#include "lds_dma.h"

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

// ---------------------------------------------------------------------------
// The staged kernel, for shapes where the matrix cores, not the weight
// stream, bound the pass.
//
// Tile: 64 token rows x 512 weight rows (gate/up: 256 gate rows and the 256
// matching up rows), one 512-thread block per CU.  Wave w owns 64 weight
// rows -- gate/up: gate and up rows 32 w .. +31, so g and u of one (token, f)
// meet in one lane; down: rows 64 w .. +63 -- against all 64 tokens: 2 x 2
// fragments of v_mfma_f32_32x32x16_bf16, so each weight element is widened
// by one wave and feeds two MFMAs.  The product is weight-major (weights as
// the MFMA A operand): a lane's accumulators hold four consecutive output
// columns of one token, so h and y_perm go out as 8- and 16-byte stores.
//
// K runs in stages (128 K for 4-bit codes, 64 K for fp8: 64 code bytes per
// weight row either way), three stages in LDS, one block barrier each.
// Token rows (gathered through perm for gate/up), weight codes and, every few
// stages, an 8-byte window of scales per weight row arrive by global -> LDS
// copies issued two stages ahead and counted by hand (vmcnt).  The token and
// code copies of a stage go out one by one between the MFMAs of the stage
// before; their offsets are worked out once per task.  The copy stream runs
// on across the block's tasks: the next task's 64 dispatch entries come in
// by one more copy at the start of a task, so the switch to the next task
// needs no load the compiler would wait for.  LDS rows are XOR-swizzled on
// their 16-byte chunks so that the fragment reads of 16 consecutive rows hit
// distinct bank groups.  Within a 64-K sub-stage, lane half h of every MFMA
// covers K 32h .. +31 (step s: 32h + 8s .. +7) of both operands, so a lane's
// codes of a sub-stage are one 16-byte (4-bit) or 32-byte (fp8) read and one
// scale group covers all of them.
constexpr int DT_BM = 64;
constexpr int DT_BN = 512;
constexpr int DT_NS = 3;            // K stages in LDS
constexpr int DT_SW = 3;            // scale windows in LDS
constexpr int DT_GM = 8;            // M-tiles per scheduling group
constexpr int DT_THREADS = 512;
constexpr int DT_WST = DT_BN * 64;  // code bytes of a stage (32 KB)

enum { DT_I4G128 = 0, DT_I4G64 = 1, DT_FP4 = 2, DT_FP8 = 3 };

template <int F, bool WIDE>
struct DtFmt {
    static constexpr int KS = F == DT_FP8 ? 64 : 128;          // K per stage
    static constexpr int SUB = KS / 64;                        // 64-K sub-stages
    // token rows of a tile: 128 (WIDE) or 64.  Stages in LDS: three (copies
    // two stages ahead), or two (one ahead) for 128 rows of 4-bit stages,
    // whose tokens take twice the fp8 stage's bytes
    static constexpr int BM = WIDE ? 2 * DT_BM : DT_BM;
    static constexpr int NS = (WIDE && F != DT_FP8) ? 2 : DT_NS;
    static constexpr int AHEAD = NS - 1;
    static constexpr int TT = BM / 32;                         // 32-token MFMA fragments
    static constexpr int TROW = KS * 2;                        // token bytes per row and stage
    static constexpr int TOK = BM * TROW;                      // token bytes of a stage
    static constexpr int STAGE = TOK + DT_WST;
    static constexpr int TCOPY = TOK / 1024 / 8;               // token copies per wave and stage
    static constexpr int BASE = TCOPY + DT_WST / 1024 / 8;     // token + code copies per wave and stage
    // scale bytes per weight row and stage; stages per 8-byte window
    static constexpr int SPB = F == DT_I4G128 ? 2 : F == DT_I4G64 ? 4 : F == DT_FP4 ? 4 : 2;
    static constexpr int WIN = 8 / SPB;
};

// One dword copy per lane (lane l lands at lds_addr + 4 l).
__device__ __forceinline__ void dma4(const int32x4_t& desc, uint32_t off, uint32_t lds_addr) {
    int32x4_t d;
    d.x = __builtin_amdgcn_readfirstlane(desc.x);
    d.y = __builtin_amdgcn_readfirstlane(desc.y);
    d.z = __builtin_amdgcn_readfirstlane(desc.z);
    d.w = __builtin_amdgcn_readfirstlane(desc.w);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("buffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(d), "{m0}"(m0)
                 : "memory");
}

// Byte B of x as fp32 in one instruction (v_cvt_f32_ubyteN: there is no
// builtin, and from shifts and masks the compiler emits an extract first).
template <int B>
__device__ __forceinline__ float dt_ubyte(uint32_t x) {
    float r;
    if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// 8 bf16 of MFMA step s (K elements 8s .. 8s+7 of the lane's 32) from the
// lane's codes c (4-bit: 16 bytes; fp8: 32 bytes in c, c2), times the scale
template <int F>
__device__ __forceinline__ dq_bf16x8_t dt_widen(const dq_u32x4_t& c, const dq_u32x4_t& c2, int s, float scale) {
    uint32_t p[4];
    if constexpr (F == DT_I4G128 || F == DT_I4G64) {
        // offset-binary nibbles u = q + 8 in bytes (each byte to fp32 is one
        // v_cvt_f32_ubyteN), then (u - 8) * scale in fp32 (exact: 4 x 11
        // significant bits) rounded once to bf16
        const uint32_t t = c[s] ^ 0x88888888u;
        const uint32_t lo = t & 0x0F0F0F0Fu, hi = (t >> 4) & 0x0F0F0F0Fu;
        const float off = -8.0f * scale;
        p[0] = pack_bf16x2(fmaf(dt_ubyte<0>(lo), scale, off), fmaf(dt_ubyte<0>(hi), scale, off));
        p[1] = pack_bf16x2(fmaf(dt_ubyte<1>(lo), scale, off), fmaf(dt_ubyte<1>(hi), scale, off));
        p[2] = pack_bf16x2(fmaf(dt_ubyte<2>(lo), scale, off), fmaf(dt_ubyte<2>(hi), scale, off));
        p[3] = pack_bf16x2(fmaf(dt_ubyte<3>(lo), scale, off), fmaf(dt_ubyte<3>(hi), scale, off));
    } else if constexpr (F == DT_FP4) {
        const uint32_t w = c[s];
        p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
        p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
        p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
        p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    } else {
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

typedef const __attribute__((address_space(4))) int32_t* dt_cptr;

// wait until at most n (0 or one of the group sizes a wave issues: B, B + 1
// with the perm copy, B + 2 with a scale window, B + 3 with both) of this
// wave's copies are outstanding
template <int B>
__device__ __forceinline__ void dt_wait(int n) {
    if (n == 0) wait_vmcnt<0>();
    else if (n <= B) wait_vmcnt<B>();
    else if (n == B + 1) wait_vmcnt<B + 1>();
    else if (n == B + 2) wait_vmcnt<B + 2>();
    else wait_vmcnt<B + 3>();
}

template <int MODE, int F, bool WIDE>
__global__ __launch_bounds__(DT_THREADS, 1) void dq_tile_kernel(DqArgs a) {
    using Fm = DtFmt<F, WIDE>;
    constexpr int BASE = Fm::BASE;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Fm::NS * Fm::STAGE + DT_SW * DT_BN * 8 + Fm::BM * 4];
    uint8_t* const sc_base = smem + Fm::NS * Fm::STAGE;
    const int32_t* const s_perm = reinterpret_cast<const int32_t*>(sc_base + DT_SW * DT_BN * 8);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, r32 = lane & 31;
    const int K = a.K, N = a.N;
    const dt_cptr tl = (dt_cptr)a.tiles;
    const int max_mt = a.max_mt;
    const int n_mt = tl[3 * max_mt];
    const int nN = MODE == 0 ? (N + DT_BN / 2 - 1) / (DT_BN / 2) : (N + DT_BN - 1) / DT_BN;
    const int total = n_mt * nN;
    const int nblk = gridDim.x;
    // blocks are dealt round-robin to the 8 XCDs: consecutive slots share one
    const int per = nblk / 8;
    const int slot = (nblk % 8 == 0) ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
    if (slot >= total) return;
    const int NKB = K / Fm::KS;
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const uint32_t crow = F == DT_FP8 ? (uint32_t)K : (uint32_t)K / 2u;          // code bytes per row
    const uint32_t srow = F == DT_I4G128 ? (uint32_t)K / 64u : (uint32_t)K / 32u;  // scale bytes per row
    const int32x4_t RA = make_desc(a.in, (uint32_t)a.in_rows * row_bytes);
    const int32x4_t RP = make_desc(a.perm, MODE == 0 ? (uint32_t)a.in_rows * (uint32_t)a.topk * 4u : 0u);

    // task t -> (M-tile, N-tile): groups of DT_GM M-tiles x all N-tiles, M fastest
    auto task_tile = [&](int t, int& mt, int& nt) {
        const int grp = t / (DT_GM * nN);
        const int gm0 = grp * DT_GM;
        const int gsz = min(DT_GM, n_mt - gm0);
        const int rem = t - grp * DT_GM * nN;
        mt = gm0 + rem % gsz;
        nt = rem / gsz;
    };

    // ---- copy side.  Wave w copies token rows BM/8 w .. +BM/8-1, weight rows
    // 64 w .. +63 (LDS order: gate/up 256 gate rows, then 256 up rows) and
    // their scale windows.  Per task: the lane parts of every copy offset.
    // Token copy i: 4-bit stages, rows BM/8 w + 4i + l/16 with 16 chunks per
    // row; fp8 stages, rows BM/8 w + 8i + l/8 with 8 chunks.  Code copy i: rows
    // 64w + 16i + l/4, 4 chunks.  Scale copy i: rows 64w + 32i + l/2, dword l%2.
    int i_e = 0, i_nt = 0, i_rows = 0, i_p0 = 0;
    uint32_t t_off[Fm::TCOPY], w_off[4], s_off[2];
    int32x4_t RW[2], RS[2];                    // gate (or down) and up codes and scales of the task's expert
    // token rows BM/8 w .. +BM/8-1 of wave w: copy i holds 8 rows of 128
    // bytes (fp8 stages) or 4 rows of 256 bytes (4-bit stages)
    constexpr int RPW = Fm::BM / 8;
    auto token_row = [&](int i) {
        return F == DT_FP8 ? RPW * wave + 8 * i + (lane >> 3) : RPW * wave + 4 * i + (lane >> 4);
    };
    auto set_task = [&](int t) {
        int mt;
        task_tile(t, mt, i_nt);
        i_e = tl[mt];
        i_p0 = tl[max_mt + mt];
        i_rows = tl[2 * max_mt + mt];
        const size_t eo = (size_t)i_e * N;
        RW[0] = make_desc(a.w0 + eo * crow, (uint32_t)N * crow);
        RW[1] = make_desc((MODE == 0 ? a.w1 : a.w0) + eo * crow, (uint32_t)N * crow);
        RS[0] = make_desc(a.s0 + eo * srow, (uint32_t)N * srow);
        RS[1] = make_desc((MODE == 0 ? a.s1 : a.s0) + eo * srow, (uint32_t)N * srow);
        const int half = MODE == 0 ? DT_BN / 2 : DT_BN;     // weight rows of one matrix in a tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lr = 64 * wave + 16 * i + (lane >> 2);
            const int lc = (lane & 3) ^ ((lr >> 2) & 3);
            const int gr = i_nt * half + (MODE == 0 ? (lr & (DT_BN / 2 - 1)) : lr);
            w_off[i] = gr < N ? (uint32_t)gr * crow + (uint32_t)lc * 16u : DQ_OOB;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int lr = 64 * wave + 32 * i + (lane >> 1);
            const int gr = i_nt * half + (MODE == 0 ? (lr & (DT_BN / 2 - 1)) : lr);
            s_off[i] = gr < N ? (uint32_t)gr * srow + (uint32_t)(lane & 1) * 4u : DQ_OOB;
        }
    };
    auto set_rows = [&](const int (&src)[Fm::TCOPY]) {
#pragma unroll
        for (int i = 0; i < Fm::TCOPY; ++i) {
            const int r = token_row(i);
            const int lc = F == DT_FP8 ? ((lane & 7) ^ ((r >> 1) & 7)) : ((lane & 15) ^ (r & 15));
            t_off[i] = r < i_rows ? (uint32_t)src[i] * row_bytes + (uint32_t)lc * 16u : DQ_OOB;
        }
    };

    // The copies of stage kb of the copy-side task into stage slot st.  A
    // scale window (when kb opens one, into window slot ws) and the next
    // task's dispatch entries (when asked: wave 0, gate/up) go out at once;
    // the token and code copies are only prepared and go out one by one
    // between the MFMAs of the current stage (fire).  Returns this wave's
    // number of copies.
    int32x4_t c_desc[BASE];
    uint32_t c_off[BASE], c_lds[BASE];
    bool c_live = false;                           // a prepared group is waiting to go out
    auto issue = [&](int kb, int st, int ws, int perm_p0) -> int {
        int n = 0;
        if (kb % Fm::WIN == 0) {
            const uint32_t wb = (uint32_t)kb * Fm::SPB;
            const int m = MODE == 0 && wave >= 4 ? 1 : 0;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                dma4(RS[m], s_off[i] == DQ_OOB ? DQ_OOB : s_off[i] + wb,
                     lds_addr(sc_base + ws * DT_BN * 8 + (64 * wave + 32 * i) * 8));
            n += 2;
        }
        if (MODE == 0 && perm_p0 >= 0 && wave < Fm::BM / 64) {
            // the next task's BM dispatch entries, 64 per wave of the first BM/64
            dma4(RP, (uint32_t)(perm_p0 + 64 * wave + lane) * 4u, lds_addr(s_perm + 64 * wave));
            ++n;
        }
        uint8_t* stage = smem + st * Fm::STAGE;
#pragma unroll
        for (int i = 0; i < Fm::TCOPY; ++i) {
            c_desc[i] = RA;
            c_off[i] = t_off[i] == DQ_OOB ? DQ_OOB : t_off[i] + (uint32_t)kb * Fm::TROW;
            c_lds[i] = lds_addr(stage + (RPW * wave + (F == DT_FP8 ? 8 * i : 4 * i)) * Fm::TROW);
        }
        const int m = MODE == 0 && wave >= 4 ? 1 : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c_desc[Fm::TCOPY + i] = RW[m];
            c_off[Fm::TCOPY + i] = w_off[i] == DQ_OOB ? DQ_OOB : w_off[i] + (uint32_t)kb * 64u;
            c_lds[Fm::TCOPY + i] = lds_addr(stage + Fm::TOK + (64 * wave + 16 * i) * 64);
        }
        return n + BASE;
    };
    auto fire = [&](int i) __attribute__((always_inline)) {
        if (c_live) dma16(c_desc[i], c_off[i], c_lds[i]);
    };

    // ---- the first task: its dispatch entries by ordinary loads (no copy in flight yet)
    set_task(slot);
    {
        int src[Fm::TCOPY];
#pragma unroll
        for (int i = 0; i < Fm::TCOPY; ++i) {
            const int r = token_row(i);
            src[i] = MODE == 0 ? (r < i_rows ? a.perm[i_p0 + r] / a.topk : 0) : i_p0 + r;
        }
        set_rows(src);
    }
    // copy-side cursor (task, stage index, LDS slots); windows counted in stream order
    int i_task = slot, i_kb = 0, i_st = 0, i_win = 0;
    bool i_live = true, i_fresh = false;
    // prepare the stage at the cursor and advance it.  The first stage of a
    // later task reads that task's dispatch entries from s_perm: they were
    // copied with the group of the previous task's first stage, at least two
    // steps (one wait and one barrier) earlier.
    auto issue_next = [&](int perm_p0) -> int {
        c_live = i_live;
        if (!i_live) return 0;
        if (i_fresh) {
            set_task(i_task);
            int src[Fm::TCOPY];
#pragma unroll
            for (int i = 0; i < Fm::TCOPY; ++i) {
                const int r = token_row(i);
                src[i] = MODE == 0 ? s_perm[r] / a.topk : i_p0 + r;
            }
            set_rows(src);
            i_fresh = false;
        }
        const int ws = i_win % DT_SW;
        if (i_kb % Fm::WIN == 0) ++i_win;
        const int n = issue(i_kb, i_st, ws, perm_p0);
        i_st = i_st + 1 == Fm::NS ? 0 : i_st + 1;
        if (++i_kb == NKB) {
            i_kb = 0;
            i_task += nblk;
            i_live = i_task < total;
            i_fresh = i_live;
        }
        return n;
    };

    // ---- compute side: the lane's weight rows (LDS) of its two fragments
    int lr[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
        lr[ni] = MODE == 0 ? ni * (DT_BN / 2) + 32 * wave + r32 : 64 * wave + 32 * ni + r32;
    dq_floatx16 acc[Fm::TT][2];                     // [token fragment][weight fragment]
#pragma unroll
    for (int t = 0; t < Fm::TT; ++t)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[t][ni][v] = 0.f;

    // One stage: 4 SUB steps (sub-stage b = j/4, MFMA step j%4) of four
    // MFMAs; step j's token fragments are read at step j-2, a sub-stage's
    // codes and scales three steps before it starts, and the next group's
    // copies go out between the steps (scheduling fences keep them there).
    constexpr int STEPS = 4 * Fm::SUB;
    auto compute = [&](int st, int ws, int kb) __attribute__((always_inline)) {
        const uint8_t* tok = smem + st * Fm::STAGE;
        const uint8_t* wts = tok + Fm::TOK;
        const uint8_t* sc = sc_base + ws * DT_BN * 8 + (kb % Fm::WIN) * Fm::SPB;
        dq_u32x4_t c[Fm::SUB][2], c2[Fm::SUB][2];
        float scale[Fm::SUB][2];
        auto read_codes = [&](int b) __attribute__((always_inline)) {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int R = lr[ni];
                const uint8_t* wr = wts + R * 64;
                const int sw = (R >> 2) & 3;
                if constexpr (F == DT_FP8) {
                    c[b][ni] = *reinterpret_cast<const dq_u32x4_t*>(wr + (((2 * h) ^ sw) << 4));
                    c2[b][ni] = *reinterpret_cast<const dq_u32x4_t*>(wr + (((2 * h + 1) ^ sw) << 4));
                } else {
                    c[b][ni] = *reinterpret_cast<const dq_u32x4_t*>(wr + (((2 * b + h) ^ sw) << 4));
                    c2[b][ni] = c[b][ni];
                }
                const uint8_t* sr = sc + R * 8;
                if constexpr (F == DT_I4G128)
                    scale[b][ni] = f16_to_f32(*reinterpret_cast<const uint16_t*>(sr));
                else if constexpr (F == DT_I4G64)
                    scale[b][ni] = f16_to_f32(*reinterpret_cast<const uint16_t*>(sr + 2 * b));
                else if constexpr (F == DT_FP4)
                    scale[b][ni] = dq_e8m0(sr[2 * b + h]);
                else
                    scale[b][ni] = dq_e8m0(sr[h]);
            }
        };
        auto read_tok = [&](int j, int t) __attribute__((always_inline)) {
            const int b = j >> 2, s4 = j & 3;
            const int T = 32 * t + r32;
            const int ch = F == DT_FP8 ? 4 * h + s4 : 8 * b + 4 * h + s4;
            const int sw = F == DT_FP8 ? ((T >> 1) & 7) : (T & 15);
            return *reinterpret_cast<const dq_bf16x8_t*>(tok + T * Fm::TROW + ((ch ^ sw) << 4));
        };
        read_codes(0);
        dq_bf16x8_t tf[3][Fm::TT];                  // token fragments, read two steps ahead
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int t = 0; t < Fm::TT; ++t) tf[j][t] = read_tok(j, t);
#pragma unroll
        for (int j = 0; j < STEPS; ++j) {
            const int b = j >> 2, s4 = j & 3;
            if (j + 2 < STEPS) {
#pragma unroll
                for (int t = 0; t < Fm::TT; ++t) tf[(j + 2) % 3][t] = read_tok(j + 2, t);
            }
            if (Fm::SUB > 1 && j == 1) read_codes(1);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const dq_bf16x8_t wf = dt_widen<F>(c[b][ni], c2[b][ni], s4, scale[b][ni]);
#pragma unroll
                for (int t = 0; t < Fm::TT; ++t)
                    acc[t][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, tf[j % 3][t], acc[t][ni], 0, 0, 0);
            }
            // copies [j BASE / STEPS, (j + 1) BASE / STEPS) go out after step j
#pragma unroll
            for (int i = j * BASE / STEPS; i < (j + 1) * BASE / STEPS; ++i) {
                __builtin_amdgcn_sched_barrier(0);
                fire(i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // lane l, accumulator element v of fragment (t, ni): token 32 t + l%32,
    // weight row 8 (v/4) + 4 h + v%4 of the fragment (four consecutive
    // outputs per v/4)
    auto epilogue = [&](int task) {
        int mt, nt;
        task_tile(task, mt, nt);
        const int p0 = tl[max_mt + mt], rows = tl[2 * max_mt + mt];
#pragma unroll
        for (int t = 0; t < Fm::TT; ++t) {
            const int tr = 32 * t + r32;
            if (tr < rows) {
                const size_t orow = (size_t)(p0 + tr) * N;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (MODE == 0) {
                        const int f = nt * (DT_BN / 2) + 32 * wave + 8 * q + 4 * h;
                        if (f < N) {
                            const dq_floatx16& g = acc[t][0];
                            const dq_floatx16& u = acc[t][1];
                            uint2 o;
                            o.x = pack_bf16x2(silu(g[4 * q]) * u[4 * q], silu(g[4 * q + 1]) * u[4 * q + 1]);
                            o.y = pack_bf16x2(silu(g[4 * q + 2]) * u[4 * q + 2], silu(g[4 * q + 3]) * u[4 * q + 3]);
                            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow + f) = o;
                        }
                    } else {
#pragma unroll
                        for (int ni = 0; ni < 2; ++ni) {
                            const int n = nt * DT_BN + 64 * wave + 32 * ni + 8 * q + 4 * h;
                            if (n < N)
                                *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow + n) =
                                    make_float4(acc[t][ni][4 * q], acc[t][ni][4 * q + 1], acc[t][ni][4 * q + 2],
                                                acc[t][ni][4 * q + 3]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < Fm::TT; ++t)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[t][ni][v] = 0.f;
    };

    // ---- the stream: stage g is prepared at step g - AHEAD and its token and
    // code copies go out during that step's MFMAs (the prologue issues the
    // first AHEAD stages at once).  Step g: this wave's copies of stage g have
    // landed once at most the newer groups (stage g + 1 with AHEAD = 2, none
    // with AHEAD = 1) are outstanding; the barrier then publishes stage g to
    // every wave and tells that everyone is done with stage g - 1, whose slot
    // receives stage g + AHEAD.
    int n_prev = 0;
#pragma unroll
    for (int p = 0; p < Fm::AHEAD; ++p) {
        n_prev = issue_next(-1);
#pragma unroll
        for (int i = 0; i < BASE; ++i) fire(i);
    }
    int c_task = slot, c_kb = 0, c_st = 0, c_win = 0;
    for (;;) {
        dt_wait<BASE>(Fm::AHEAD == 2 ? n_prev : 0);
        block_barrier();
        // at a task's first stage the next task's dispatch entries go out
        // with this group; they are read when the copy side reaches that task
        int pp = -1;
        if (MODE == 0 && c_kb == 0 && c_task + nblk < total) {
            int mt, nt;
            task_tile(c_task + nblk, mt, nt);
            pp = tl[max_mt + mt];
        }
        n_prev = issue_next(pp);
        if (c_kb % Fm::WIN == 0) ++c_win;
        compute(c_st, (c_win - 1) % DT_SW, c_kb);
        c_st = c_st + 1 == Fm::NS ? 0 : c_st + 1;
        if (++c_kb == NKB) {
            epilogue(c_task);
            c_kb = 0;
            c_task += nblk;
            if (c_task >= total) break;
        }
    }
    // every copy has been waited for: the last wait saw no group outstanding
}

// One 256-thread block: per expert with more than tau rows, ceil(rows/bm)
// tiles of bm rows; an exclusive scan over the experts places them.  With a
// remainder table (rem: counts [E] then offsets [E]), a group's last partial
// tile of at most rem_max rows is left out and its rows listed there instead
// (every other expert's entry is zero).
__global__ __launch_bounds__(256) void dq_plan_kernel(const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ offsets, int E, int tau, int bm,
                                                     int32_t* __restrict__ tiles, int max_mt, int rem_max,
                                                     int32_t* __restrict__ rem) {
    __shared__ int s[2][256];
    const int tid = threadIdx.x;
    int c = 0, nb = 0;
    if (tid < E) {
        c = counts[tid];
        int rc = 0;
        if (c > tau && c > 0) {
            nb = (c + bm - 1) / bm;
            const int r = c - (c / bm) * bm;
            if (rem && r > 0 && r <= rem_max) {
                nb = c / bm;
                rc = r;
            }
        }
        if (rem) {
            rem[tid] = rc;
            rem[E + tid] = rc ? offsets[tid] + nb * bm : 0;
        }
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
            tiles[max_mt + b + i] = o0 + i * bm;
            tiles[2 * max_mt + b + i] = min(bm, c - i * bm);
        }
    }
    if (tid == 255) tiles[3 * max_mt] = s[cur][255];
}

}  // namespace

// bounds for the smaller tile height, so one plan region serves both kernels
int dq_max_tiles(int T, int k, int E) { return (T * k + DT_BM - 1) / DT_BM + E; }
int dq_plan_ints(int T, int k, int E) { return 3 * dq_max_tiles(T, k, E) + 1 + 2 * E; }

bool dq_supported(int K, int N) {
    // whole K pairs; 32-bit buffer offsets of a matrix (fp8: one byte per element)
    return K > 0 && K % DQ_PK == 0 && N > 0 && (size_t)N * (size_t)K < ((size_t)1 << 31);
}

// The staged kernel: whole stages (128 K for 4-bit codes, 64 K for fp8), at
// least four of them, and scale rows of whole dwords (the window copies).
bool dq_staged_ok(int fmt, int gs, int K) {
    if (K % 128 != 0) return false;
    if (fmt == DQ_MXFP8) return K >= 256;
    if (K < 512) return false;
    return !(fmt == DQ_INT4 && gs == 128 && K % 256 != 0);
}

// Token rows of the staged kernel's tiles: 128 for MXFP8 (three stages) and
// int4 (two stages; int4 widening is VALU-bound, and each widened fragment
// then feeds four token fragments: 5.48 -> 4.75 ms on the fine-grained int4
// prefill layer), 64 for MXFP4 (with 128 rows its registers spill and the
// layer measured 1.6% slower).
static bool dq_wide(int fmt) { return fmt != DQ_MXFP4; }

int dq_tile_rows(int fmt, bool staged) {
    if (!staged) return DQ_BM;
    return dq_wide(fmt) ? 2 * DT_BM : DT_BM;
}

int32_t* dq_remainders(int32_t* tiles, int max_mt) { return tiles + 3 * max_mt + 1; }

hipError_t launch_dq_plan(const int32_t* counts, const int32_t* offsets, int E, int tau, int fmt, bool staged,
                          int32_t* tiles, int max_mt, int rem_max, hipStream_t s) {
    if (E > 256) return hipErrorInvalidValue;
    int32_t* rem = rem_max > 0 ? dq_remainders(tiles, max_mt) : nullptr;
    hipLaunchKernelGGL(dq_plan_kernel, dim3(1), dim3(256), 0, s, counts, offsets, E, tau, dq_tile_rows(fmt, staged),
                       tiles, max_mt, rem_max, rem);
    return hipGetLastError();
}

hipError_t launch_dq_ffn(int mode, int fmt, int gs, bool staged, const void* w0, const void* w1, const void* s0,
                         const void* s1, const void* in, void* out, const int32_t* perm, const int32_t* tiles, int N,
                         int K, int topk, int max_mt, int in_rows, hipStream_t s) {
    if (!dq_supported(K, N) || (fmt == DQ_INT4 && (gs != 64 && gs != 128)) || fmt < 0 || fmt > 2)
        return hipErrorInvalidValue;
    if (staged && (!dq_staged_ok(fmt, gs, K) || N % 4 != 0)) return hipErrorInvalidValue;
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
    if (staged) {
        // one 512-thread block per CU over the (M-tile, N-tile) tasks
        const int nN = mode == 0 ? (N + DT_BN / 2 - 1) / (DT_BN / 2) : (N + DT_BN - 1) / DT_BN;
        const long slots = (long)max_mt * nN;
        const long cap = cu_count();
        const int grid = (int)(slots < cap ? slots : cap);
        const int f = fmt == DQ_MXFP4 ? DT_FP4 : fmt == DQ_MXFP8 ? DT_FP8 : (gs == 128 ? DT_I4G128 : DT_I4G64);
        // the tile height dq_wide gives each format (the plan used the same)
#define DT_LAUNCH(M, F) hipLaunchKernelGGL((dq_tile_kernel<M, F, F != DT_FP4>), dim3(grid), dim3(DT_THREADS), 0, s, a)
#define DT_FMTS(M)                               \
        switch (f) {                             \
            case DT_I4G128: DT_LAUNCH(M, DT_I4G128); break; \
            case DT_I4G64: DT_LAUNCH(M, DT_I4G64); break;   \
            case DT_FP4: DT_LAUNCH(M, DT_FP4); break;       \
            default: DT_LAUNCH(M, DT_FP8); break;           \
        }
        if (mode == 0) { DT_FMTS(0) } else { DT_FMTS(1) }
#undef DT_FMTS
#undef DT_LAUNCH
        return hipGetLastError();
    }
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
