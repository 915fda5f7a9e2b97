// Expert FFN for bf16 groups of up to 64 rows: a skinny MFMA kernel (tokens
// as the 16-wide side of v_mfma_f32_16x16x32_bf16, one to four 16-token tiles
// per weight operand) that streams each active expert's weights once.
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §3.1 (w1/w3 gate and up,
// w2 down, no bias) and §3.3 (each expert streams its weights for the tokens
// the dispatcher gave it; the page's kernel is the 32 x 4096 x 14336 top-2
// case).  The GEMV keeps a pass of 4-8 tokens in registers, so a group of
// 5-64 rows would stream its expert's weights two to sixteen times; the MFMA
// grouped GEMM tiles 64 or 256 rows and leaves most of a tile idle.  Here one
// pass covers up to 64 tokens and the weights stream once:
//
//  * a persistent grid (one 512-thread block per CU) splits the list of work
//    items (active expert, tile of 16 R weight rows) into equal contiguous
//    ranges, one per block;
//  * the eight waves of a block split the item's K: wave w takes the 128-byte
//    lines 8 i + w of every row, so a step of the block reads 1 KiB of each of
//    the tile's rows; a K that is not a multiple of 512 leaves whole lines past
//    the row end, which load as zeros.  Each wave keeps a ring of loads in
//    flight that runs on across item boundaries;
//  * every load instruction reads whole 128-byte lines (8 rows x 128 B, lane
//    8a + b taking piece b ^ a of row a; weights with the nontemporal hint).
//    An MFMA operand needs 16 rows x 64 B per register, i.e. half lines;
//    loading that shape directly left the vector L1 stalling on twice as many
//    line requests and let the nontemporal lines leave L2 before their second
//    half was read.  So the lines go through the wave's own LDS slot and come
//    back in operand layout (lane 16q + n: row n, piece 4s + q); the XOR
//    swizzle keeps both the writes and the reads free of bank conflicts;
//  * the token rows (gathered through the permutation for gate/up) take the
//    same route, from L2, as the A operand of 2 R G MFMAs per 16-token tile;
//    blocks start their K walk at different lines so that the token rows'
//    lines spread over the L2 channels;
//  * the buffer range check turns loads past the last weight row, for token
//    slots past the group, past the row end and past the block's range into
//    zeros, so no load is branched;
//  * at the end of an item each wave parks its 16x16 partial tiles in LDS, a
//    barrier, and the block sums the eight K slices in a fixed order, applies
//    the SwiGLU (gate/up: h in bf16) or stores fp32 rows of y_perm (down);
//  * one launch serves a batch: it finds the largest group M of at most `cap`
//    rows and, when M exceeds the GEMV pass `lo`, runs the variant with
//    ceil(M / 16) token tiles over every group of 1..cap rows.  An item is
//    32 weight rows (R = 2), except gate/up with four tiles: 16 rows (R = 1),
//    which keeps its registers and partial tiles within bounds (three tiles
//    of gate/up keep 32 rows with two steps of loads in flight, 12% faster at
//    128 tokens than 16 rows with three).
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
constexpr int kLine = 128;                  // bytes of a row one wave takes per step
constexpr int kStepK = kWaves * kLine / 2;  // K elements one block step covers (512)
constexpr int kTok = 16;                    // tokens of one token tile
constexpr int kMaxE = 256;
constexpr int kMaxPairs = 48;               // experts one block's range can touch
constexpr uint32_t kOob = 0x80000000u;      // past any buffer: the range check yields 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// weights are read once: nontemporal, so they do not push the token rows out of L2
__device__ __forceinline__ u32x4_t ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

// LDS writes complete, then a workgroup barrier; the asm statements keep the
// compiler from moving LDS accesses across it
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int I>
using ic = std::integral_constant<int, I>;

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(ic<B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Position in the block's stream of (item, step) pairs; wave-uniform.
struct Cursor {
    int idx;      // step index in the block's range
    int i;        // step within the item
    int item;     // items completed since the block's first
    int tile;     // row tile of the expert
    int u;        // expert slot
    int e, c, o;  // expert id, rows of the group, its first dispatch row
};

// Shapes of one variant: TT token tiles, 16 R weight rows per item, G
// matrices sharing the token rows, D steps of loads in flight.
template <int MODE, int TT>
struct Shape {
    static constexpr int G = MODE == 0 ? 2 : 1;
    static constexpr int R = (TT <= 3 || MODE == 1) ? 2 : 1;
    static constexpr int D = (TT <= 2 && MODE == 1) ? 4 : (TT == 3 && MODE == 0) ? 2 : 3;
    static constexpr bool XA_FIRST = TT <= 2;         // all token tiles through LDS at once
    static constexpr int NW = R * G * 2;              // weight load instructions per step
    static constexpr int NT = 2 * TT;                 // token load instructions per step
    static constexpr int NL = NW + NT;
    static constexpr int NP = TT * R * G;             // 16x16 partial tiles per wave
    static constexpr int NB = TT == 1 ? 2 : 1;        // partial buffers (one more barrier per item with one)
    static constexpr int SLOT = 2 * G + (XA_FIRST ? NT : 2);   // 1 KiB loads a wave's LDS slot holds
    // LDS carve (bytes): tables, token-row offsets, partial tiles, transpose slots
    static constexpr int TAB = (4 * kMaxE + 4) * 4;
    static constexpr int ROWS = kMaxPairs * kTok * TT * 4;
    static constexpr int PART = NB * kWaves * NP * 4 * 64 * 4;
    static constexpr int LT = kWaves * SLOT * 64 * 16;
    static constexpr int BYTES = TAB + ROWS + PART + LT;
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }
template <int TT>
constexpr int bytes_tt() { return cmax(Shape<0, TT>::BYTES, Shape<1, TT>::BYTES); }
constexpr int kLdsBytes = cmax(cmax(bytes_tt<1>(), bytes_tt<2>()), cmax(bytes_tt<3>(), bytes_tt<4>()));
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

}  // namespace

struct SkArgs {
    const uint16_t* w0;        // gate (mode 0) or down (mode 1): [E][N][K] bf16
    const uint16_t* w1;        // up (mode 0)
    const uint16_t* in;        // x [in_rows][K] (mode 0) or h [in_rows][K] (mode 1), bf16
    void* out;                 // h bf16 [T*k][N] (mode 0) or y_perm fp32 [T*k][N] (mode 1)
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* perm;       // mode 0: token of dispatch row p = perm[p] / topk
    int N, K, topk, E, in_rows;
    int lo, cap;               // serve groups of 1..cap rows when the largest exceeds lo
};

template <int MODE, int TT>
__device__ __forceinline__ void skinny_body(const SkArgs& a, unsigned char* lds) {
    using SH = Shape<MODE, TT>;
    constexpr int G = SH::G, R = SH::R, D = SH::D, NW = SH::NW, NT = SH::NT, NL = SH::NL;
    constexpr int NP = SH::NP, NB = SH::NB, SLOT = SH::SLOT;
    constexpr int TR = 16 * R;                 // weight rows of one item
    int* s_act = reinterpret_cast<int*>(lds);
    int* s_cnt = s_act + kMaxE;
    int* s_off = s_cnt + kMaxE;
    int* s_ipref = s_off + kMaxE;              // kMaxE + 1
    int* s_tot = s_ipref + kMaxE + 1;          // 2
    uint32_t (*s_rows)[kTok * TT] = reinterpret_cast<uint32_t (*)[kTok * TT]>(lds + SH::TAB);
    float (*s_part)[kWaves][NP][4][64] = reinterpret_cast<float (*)[kWaves][NP][4][64]>(lds + SH::TAB + SH::ROWS);
    u32x4_t (*s_lt)[SLOT][64] = reinterpret_cast<u32x4_t (*)[SLOT][64]>(lds + SH::TAB + SH::ROWS + SH::PART);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.K, N = a.N;
    const int S = (K + kStepK - 1) / kStepK;                 // steps of an item
    const int ntile = (N + TR - 1) / TR;
    const uint32_t rowb = (uint32_t)K * 2u;                  // bytes per row

    // ---- the experts of this launch (1 <= c <= cap) and the item prefix over them
    if (wave == 0) {
        int cnt[4], act[4];
        int na = 0, ni = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            cnt[j] = e < a.E ? a.counts[e] : 0;
            act[j] = cnt[j] > 0 && cnt[j] <= a.cap;
            na += act[j];
            ni += act[j] ? ntile : 0;
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
                p += ntile;
            }
        }
        if (lane == 63) {
            s_tot[0] = ia;
            s_tot[1] = ii;
            s_ipref[ia] = ii;
        }
    }
    __syncthreads();

    const int U = s_tot[0];
    const long n_items = s_tot[1];
    const long ib = n_items * blockIdx.x / gridDim.x;
    const long ie = n_items * (blockIdx.x + 1) / gridDim.x;
    if (ib >= ie) return;
    const int nsteps = (int)(ie - ib) * S;

    // first expert slot of the block's range; slot u0 + q is pair q of s_rows
    int u0;
    {
        int lo = 0, hi = U - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_ipref[mid] <= ib) lo = mid; else hi = mid - 1;
        }
        u0 = lo;
    }
    // token-row byte offsets of the (at most kMaxPairs) experts of the range
    for (int t = tid; t < kMaxPairs * kTok * TT; t += kThreads) {
        const int q = t / (kTok * TT), ts = t % (kTok * TT), u = u0 + q;
        uint32_t off = kOob;
        if (u < U && ts < s_cnt[u]) {
            const int p = s_off[u] + ts;
            const int row = MODE == 0 ? a.perm[p] / a.topk : p;
            off = (uint32_t)row * rowb;
        }
        s_rows[q][ts] = off;
    }
    __syncthreads();

    Cursor cur;
    cur.idx = 0;
    cur.i = 0;
    cur.item = 0;
    cur.u = u0;
    cur.tile = (int)(ib - s_ipref[u0]);
    cur.e = __builtin_amdgcn_readfirstlane(s_act[u0]);
    cur.c = __builtin_amdgcn_readfirstlane(s_cnt[u0]);
    cur.o = __builtin_amdgcn_readfirstlane(s_off[u0]);

    // load shape: lane 8a + b reads piece b ^ a of the line of row (or token) a
    const uint32_t la = (uint32_t)lane >> 3;
    const uint32_t lpiece = (((uint32_t)lane & 7u) ^ la) << 4;
    const uint32_t wlane = la * rowb + lpiece;                       // lane part of a weight offset
    const uint32_t mat_bytes = (uint32_t)N * rowb;
    const uint32_t in_bytes = (uint32_t)a.in_rows * rowb;
    const size_t mat_elems = (size_t)N * K;
    const int rot = (int)((blockIdx.x >> 3) % (unsigned)S);        // this block's first line
    // operand shape: lane 16q + n wants row n, piece 4s + q: LDS slot 8 (n%8) + (piece ^ n%8)
    // of the load of rows 8 (n/8) ..
    const int on = lane & 15, oq = lane >> 4, oa = on & 7, og = on >> 3;
    auto tok_of = [&](int u, int g) { return s_rows[u - u0][8 * g + (int)la] + lpiece; };

    auto advance = [&](Cursor& q) {
        ++q.idx;
        if (++q.i < S) return;
        q.i = 0;
        ++q.item;
        if (++q.tile < ntile) return;
        q.tile = 0;
        if (++q.u < U) {
            q.e = __builtin_amdgcn_readfirstlane(s_act[q.u]);
            q.c = __builtin_amdgcn_readfirstlane(s_cnt[q.u]);
            q.o = __builtin_amdgcn_readfirstlane(s_off[q.u]);
        }
    };

    // ring slot: [0, NW) weights, instruction (h G + m) 2 + g for rows 16 h + 8 g ..;
    // NW + g the token slots 8 g ..
    u32x4_t ring[D][NL];
    uint32_t l_tok[NT];
#pragma unroll
    for (int g = 0; g < NT; ++g) l_tok[g] = tok_of(cur.u, g);
    auto issue = [&](Cursor& q, auto slot) __attribute__((always_inline)) {
        constexpr int SL = decltype(slot)::value;
        int pc = q.i + rot;
        if (pc >= S) pc -= S;
        const uint32_t kb = (uint32_t)(pc * kWaves + wave) * (uint32_t)kLine;
        // past the block's range or past the row end: zeros
        const bool live = q.idx < nsteps && kb < rowb;
        const auto ri = rsrc(a.in, live ? in_bytes : 0u);
#pragma unroll
        for (int g = 0; g < NT; ++g) ring[SL][NW + g] = ld16(ri, l_tok[g] + kb);
        const uint32_t wo = (uint32_t)q.tile * TR * rowb + wlane + kb;
        const size_t eo = (size_t)(live ? q.e : 0) * mat_elems;
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const auto r = rsrc((m == 0 ? a.w0 : a.w1) + eo, live ? mat_bytes : 0u);
#pragma unroll
            for (int h = 0; h < R; ++h)
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    ring[SL][(h * G + m) * 2 + g] = ld16_nt(r, wo + (uint32_t)(16 * h + 8 * g) * rowb);
        }
        const int u = q.u;
        advance(q);
        if (q.u != u && q.u < U && q.u - u0 < kMaxPairs) {
#pragma unroll
            for (int g = 0; g < NT; ++g) l_tok[g] = tok_of(q.u, g);
        }
    };

    floatx4 acc[TT][R][G];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int h = 0; h < R; ++h)
#pragma unroll
            for (int m = 0; m < G; ++m) acc[t][h][m] = floatx4{0.f, 0.f, 0.f, 0.f};
    // lines -> LDS -> operands (the wave's LDS accesses run in order, so a
    // part of its slot is free again once its operands are read); two K
    // pieces of 32 per step
    auto compute = [&](auto slot) __attribute__((always_inline)) {
        constexpr int SL = decltype(slot)::value;
        if constexpr (SH::XA_FIRST) {
            // the token tiles first (slot entries 2G ..), then one 16-row half at a time
            u32x4_t xa[2][TT];
#pragma unroll
            for (int g = 0; g < NT; ++g) s_lt[wave][2 * G + g][lane] = ring[SL][NW + g];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int t = 0; t < TT; ++t) xa[s][t] = s_lt[wave][2 * G + 2 * t + og][8 * oa + ((4 * s + oq) ^ oa)];
#pragma unroll
            for (int h = 0; h < R; ++h) {
#pragma unroll
                for (int j = 0; j < 2 * G; ++j) s_lt[wave][j][lane] = ring[SL][h * 2 * G + j];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int sw = 8 * oa + ((4 * s + oq) ^ oa);
#pragma unroll
                    for (int m = 0; m < G; ++m) {
                        const u32x4_t wb = s_lt[wave][m * 2 + og][sw];
#pragma unroll
                        for (int t = 0; t < TT; ++t)
                            acc[t][h][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, xa[s][t]), __builtin_bit_cast(bf16x8_t, wb),
                                acc[t][h][m], 0, 0, 0);
                    }
                }
            }
        } else {
            // the weights of every half into registers, then one token tile at a time (slot entries 2G, 2G+1)
            u32x4_t wb[R][G][2];
#pragma unroll
            for (int h = 0; h < R; ++h) {
#pragma unroll
                for (int j = 0; j < 2 * G; ++j) s_lt[wave][j][lane] = ring[SL][h * 2 * G + j];
#pragma unroll
                for (int m = 0; m < G; ++m)
#pragma unroll
                    for (int s = 0; s < 2; ++s) wb[h][m][s] = s_lt[wave][m * 2 + og][8 * oa + ((4 * s + oq) ^ oa)];
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                s_lt[wave][2 * G][lane] = ring[SL][NW + 2 * t];
                s_lt[wave][2 * G + 1][lane] = ring[SL][NW + 2 * t + 1];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const u32x4_t xa = s_lt[wave][2 * G + og][8 * oa + ((4 * s + oq) ^ oa)];
#pragma unroll
                    for (int h = 0; h < R; ++h)
#pragma unroll
                        for (int m = 0; m < G; ++m)
                            acc[t][h][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, xa), __builtin_bit_cast(bf16x8_t, wb[h][m][s]),
                                acc[t][h][m], 0, 0, 0);
                }
            }
        }
    };
    // C layout: lane l holds weight row l%16 of its half and tokens 4 (l/16) + v
    // of its tile.  The eight K-slice partials meet in LDS and are summed in
    // wave order.
    auto finish = [&](const Cursor& q) __attribute__((always_inline)) {
        float (*P)[NP][4][64] = s_part[NB == 2 ? (q.item & 1) : 0];
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int h = 0; h < R; ++h)
#pragma unroll
                for (int m = 0; m < G; ++m) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) P[wave][(t * R + h) * G + m][v][lane] = acc[t][h][m][v];
                    acc[t][h][m] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
        lds_barrier();
        // TT x R x 256 outputs over the block's threads
#pragma unroll
        for (int o0 = 0; o0 < TT * R * 256; o0 += kThreads) {
            const int o = o0 + tid;
            if (o < TT * R * 256) {
                const int tt = o / (R * 256), h = (o >> 8) % R, v = (o >> 6) & 3;
                float s[G];
#pragma unroll
                for (int m = 0; m < G; ++m) s[m] = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w)
#pragma unroll
                    for (int m = 0; m < G; ++m) s[m] += P[w][(tt * R + h) * G + m][v][lane];
                const int t = kTok * tt + oq * 4 + v;
                const int n = q.tile * TR + h * 16 + on;
                if (t < q.c && n < N) {
                    const size_t oi = (size_t)(q.o + t) * N + n;
                    if constexpr (MODE == 0)
                        reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(silu(s[0]) * s[1]);
                    else
                        reinterpret_cast<float*>(a.out)[oi] = s[0];
                }
            }
        }
        // one buffer: every wave has read it before any wave writes the next item's
        if constexpr (NB == 1) lds_barrier();
    };

    Cursor L = cur;        // next step whose loads go out
    Cursor C = cur;        // step being multiplied
    static_for<0, D>([&](auto k) { issue(L, k); });
    auto step = [&](auto kk) __attribute__((always_inline)) {
        constexpr int k = decltype(kk)::value;
        // steps past the range multiply zeros; only real item ends finish
        compute(ic<k>{});
        if (C.i == S - 1 && C.idx < nsteps) finish(C);
        advance(C);
        issue(L, ic<k>{});
    };
    for (int n = (nsteps + D - 1) / D; n > 0; --n) static_for<0, D>(step);
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void skinny_kernel(SkArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    __shared__ int s_m;
    // the largest group of at most cap rows picks the variant (or none)
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int big = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            const int c = e < a.E ? a.counts[e] : 0;
            if (c <= a.cap && c > big) big = c;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) big = max(big, __shfl_xor(big, o, 64));
        if (lane == 0) s_m = big;
    }
    __syncthreads();
    const int M = s_m;
    if (M <= a.lo) return;
    if (M <= kTok) skinny_body<MODE, 1>(a, lds);
    else if (M <= 2 * kTok) skinny_body<MODE, 2>(a, lds);
    else if (M <= 3 * kTok) skinny_body<MODE, 3>(a, lds);
    else skinny_body<MODE, 4>(a, lds);
}

bool skinny_supported(int K, int N, int in_rows) {
    // whole 128-byte lines per row: K a multiple of 64
    if (K % 64 != 0 || K <= 0 || N <= 0 || in_rows < 0) return false;
    // 32-bit buffer offsets: a weight matrix with its padded last tile, the inputs
    return (size_t)(N + 32) * (size_t)K * 2 < ((size_t)1 << 31) &&
           (size_t)in_rows * (size_t)K * 2 < ((size_t)1 << 31);
}

hipError_t launch_skinny(int mode, const void* w0, const void* w1, const void* in, int in_rows, void* out,
                         const int32_t* counts, const int32_t* offsets, const int32_t* perm, int N, int K,
                         int topk, int E, int lo, int cap, hipStream_t s) {
    SkArgs a;
    a.w0 = reinterpret_cast<const uint16_t*>(w0);
    a.w1 = reinterpret_cast<const uint16_t*>(w1);
    a.in = reinterpret_cast<const uint16_t*>(in);
    a.out = out;
    a.counts = counts;
    a.offsets = offsets;
    a.perm = perm;
    a.N = N;
    a.K = K;
    a.topk = topk;
    a.E = E;
    a.in_rows = in_rows;
    a.lo = lo;
    a.cap = cap;
    if (E > kMaxE || !skinny_supported(K, N, in_rows) || !counts || !offsets || (mode == 0 && !perm) ||
        lo < 0 || cap <= lo || cap > kSkinnyMaxRows)
        return hipErrorInvalidValue;
    const int n_cu = cu_count();
    // a block's range of ceil(items / grid) items touches at most
    // U / grid + 3 experts (each expert owns >= 1 item): kMaxPairs bounds
    // that for E <= 256 and a grid of >= 8 blocks
    if (n_cu < 8) return hipErrorInvalidValue;
    if (mode == 0)
        hipLaunchKernelGGL(skinny_kernel<0>, dim3(n_cu), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(skinny_kernel<1>, dim3(n_cu), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
