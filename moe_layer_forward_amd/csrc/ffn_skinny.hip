// Expert FFN for bf16 groups a little larger than a GEMV pass: a skinny MFMA
// kernel (tokens as the 16-wide side of v_mfma_f32_16x16x32_bf16).
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §3.1 (w1/w3 gate and up,
// w2 down, no bias) and §3.3 (each expert streams its weights for the tokens
// the dispatcher gave it; the page's kernel is the 32 x 4096 x 14336 top-2
// case).  The GEMV keeps a pass of 4-8 tokens in registers, so a group of
// 5-16 rows would stream its expert's weights two to four times; the MFMA
// grouped GEMM tiles 64 or 256 rows and leaves most of a 16-row tile idle.
// Here one pass covers up to 16 tokens and the weights stream once:
//
//  * a persistent grid (one 512-thread block per CU) walks equal-sized work
//    items (expert, 128-row chunk); each wave owns 16 weight rows and runs a
//    flat stream of (item, K step of 32) steps, 8 steps of loads in flight
//    in a register ring, continuing across item boundaries;
//  * per step a lane loads 16 bytes of its weight row (row l%16, K = 32 g +
//    8 (l/16) ..+7): exactly the B operand of one MFMA; the token rows come
//    the same way as the A operand (token slot l%16 of the pass, gathered
//    through the permutation for gate/up), from L2 - every wave of a block
//    reads the same token fragments;
//  * the buffer range check turns loads past the last weight row, for token
//    slots past the group and past the block's range into zeros, so no load
//    is branched;
//  * gate and up share each token fragment; the SwiGLU epilogue writes h
//    (bf16), the down pass fp32 rows of y_perm; lane l holds 4 tokens of
//    weight row l%16.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kItemRows = 16 * kWaves;      // rows of one work item
constexpr int kPass = 16;                   // tokens of the group (at most)
constexpr int kRing = 8;                    // steps of loads in flight
constexpr int kMaxE = 256;
constexpr int kMaxPairs = 64;               // experts one block's range can touch
constexpr uint32_t kOob = 0x80000000u;      // past any buffer: the range check yields 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
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

// Position in the block's flat stream of (item, K step) steps; wave-uniform.
struct Cursor {
    int idx;      // step index in the block's range
    int u;        // expert slot
    int chunk;    // 128-row chunk
    int g;        // K step of 32
    int c, o, e;  // rows of the group, its first dispatch row, expert id
};

}  // namespace

struct SkArgs {
    const uint16_t* w0;        // gate (mode 0) or down (mode 1): [E][N][K] bf16
    const uint16_t* w1;        // up (mode 0)
    const uint16_t* in;        // x [in_rows][K] (mode 0) or h [in_rows][K] (mode 1), bf16
    void* out;                 // h bf16 [T*k][N] (mode 0) or y_perm fp32 [T*k][N] (mode 1)
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* perm;       // mode 0: token of dispatch row p = perm[p] / topk
    int N, K, topk, E, lo, hi, in_rows;
};

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void skinny_kernel(SkArgs a) {
    constexpr int G = MODE == 0 ? 2 : 1;
    __shared__ int s_act[kMaxE], s_cnt[kMaxE], s_off[kMaxE], s_ipref[kMaxE + 1], s_tot[2];
    __shared__ uint32_t s_rows[kMaxPairs][kPass];   // token-row byte offsets of the block's experts

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.K, N = a.N;
    const int NG = K / 32;                                   // K steps per item (multiple of 16)
    const int nrc = (N + kItemRows - 1) / kItemRows;
    const uint32_t rowb = (uint32_t)K * 2u;                  // bytes per row

    // ---- the experts of this launch (lo < c <= hi) and the item prefix over them
    if (wave == 0) {
        int cnt[4], act[4];
        int na = 0, ni = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            const int c = e < a.E ? a.counts[e] : 0;
            act[j] = c > a.lo && c <= a.hi;
            cnt[j] = c;
            na += act[j];
            ni += act[j] ? nrc : 0;
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
                p += nrc;
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
    const int nsteps = (int)(ie - ib) * NG;

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
    for (int t = tid; t < kMaxPairs * kPass; t += kThreads) {
        const int q = t / kPass, ts = t % kPass, u = u0 + q;
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
    cur.u = u0;
    cur.chunk = (int)(ib - s_ipref[u0]);
    cur.g = 0;
    cur.e = __builtin_amdgcn_readfirstlane(s_act[u0]);
    cur.c = __builtin_amdgcn_readfirstlane(s_cnt[u0]);
    cur.o = __builtin_amdgcn_readfirstlane(s_off[u0]);

    const uint32_t lq = (uint32_t)(lane >> 4);
    const uint32_t wrow = (uint32_t)(wave * 16 + (lane & 15));
    const uint32_t woff_l = wrow * rowb + lq * 16u;          // lane part of a weight offset
    const uint32_t mat_bytes = (uint32_t)N * rowb;
    const uint32_t in_bytes = (uint32_t)a.in_rows * rowb;
    // the token-row offset of this lane for the loads' cursor
    auto arow_of = [&](int u) { return s_rows[u - u0][lane & 15] + lq * 16u; };

    auto advance = [&](Cursor& q) {
        ++q.idx;
        if (++q.g < NG) return;
        q.g = 0;
        if (++q.chunk < nrc) return;
        q.chunk = 0;
        if (++q.u < U) {
            q.e = __builtin_amdgcn_readfirstlane(s_act[q.u]);
            q.c = __builtin_amdgcn_readfirstlane(s_cnt[q.u]);
            q.o = __builtin_amdgcn_readfirstlane(s_off[q.u]);
        }
    };

    u32x4_t xa[kRing], wq[kRing][G];
    uint32_t l_arow = arow_of(cur.u);
    auto issue = [&](Cursor& q, auto slot) {
        constexpr int S = decltype(slot)::value;
        const bool live = q.idx < nsteps;
        const uint32_t ko = (uint32_t)q.g * 64u;
        // past the block's range (or a slot index beyond the experts): zeros
        xa[S] = ld16(rsrc(a.in, live ? in_bytes : 0u), l_arow + ko);
        const uint32_t wo = woff_l + (uint32_t)q.chunk * kItemRows * rowb + ko;
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const uint16_t* w = (m == 0 ? a.w0 : a.w1) + (size_t)(live ? q.e : 0) * N * K;
            wq[S][m] = ld16(rsrc(w, live ? mat_bytes : 0u), wo);
        }
        const int u = q.u;
        advance(q);
        if (q.u != u && q.u < U && q.u - u0 < kMaxPairs) l_arow = arow_of(q.u);
    };

    floatx4 acc[G];
#pragma unroll
    for (int m = 0; m < G; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](auto slot) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int m = 0; m < G; ++m)
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[S]),
                                                             __builtin_bit_cast(bf16x8_t, wq[S][m]),
                                                             acc[m], 0, 0, 0);
    };
    // C layout: lane l holds weight row l%16 of its wave's 16 and tokens 4 (l/16) + v
    auto epilogue = [&](const Cursor& q) {
        const int n = q.chunk * kItemRows + wave * 16 + (lane & 15);
        if (n < N) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = (int)lq * 4 + v;
                if (t < q.c) {
                    const size_t oi = (size_t)(q.o + t) * N + n;
                    if constexpr (MODE == 0)
                        reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(silu(acc[0][v]) * acc[1][v]);
                    else
                        reinterpret_cast<float*>(a.out)[oi] = acc[0][v];
                }
            }
        }
#pragma unroll
        for (int m = 0; m < G; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    };

    Cursor L = cur;        // next step whose loads go out
    Cursor C = cur;        // step being multiplied
    static_for<0, kRing>([&](auto k) { issue(L, k); });
    auto step = [&](auto kk) {
        constexpr int k = decltype(kk)::value;
        compute(ic<k % kRing>{});
        if (C.g == NG - 1) epilogue(C);
        advance(C);
        issue(L, ic<k % kRing>{});
    };
    // nsteps is a multiple of 16 (NG is)
    for (int n = nsteps >> 4; n > 0; --n) static_for<0, 16>(step);
}

bool skinny_supported(int K, int N, int in_rows) {
    if (K % 512 != 0 || K <= 0 || N <= 0 || in_rows < 0) return false;
    // 32-bit buffer offsets: a weight matrix with its padded last chunk, the inputs
    return (size_t)(N + kItemRows) * (size_t)K * 2 < ((size_t)1 << 31) &&
           (size_t)in_rows * (size_t)K * 2 < ((size_t)1 << 31);
}

hipError_t launch_skinny(int mode, const void* w0, const void* w1, const void* in, int in_rows, void* out,
                         const int32_t* counts, const int32_t* offsets, const int32_t* perm, int N, int K,
                         int topk, int E, int lo, int hi, hipStream_t s) {
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
    a.lo = lo;
    a.hi = hi < kPass ? hi : kPass;
    a.in_rows = in_rows;
    if (E > kMaxE || !skinny_supported(K, N, in_rows) || !counts || !offsets || (mode == 0 && !perm))
        return hipErrorInvalidValue;
    static int n_cu = 0;
    if (n_cu == 0) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (n_cu < 1) n_cu = 256;
    }
    // a block's range touches at most ceil(E / n_cu) + 1 experts' first
    // chunks plus the experts it spans; kMaxPairs bounds that for E <= 256
    // and n_cu >= 8
    if (n_cu < 8) return hipErrorInvalidValue;
    if (mode == 0)
        hipLaunchKernelGGL(skinny_kernel<0>, dim3(n_cu), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(skinny_kernel<1>, dim3(n_cu), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
