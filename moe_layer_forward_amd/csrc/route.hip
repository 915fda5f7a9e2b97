// Router logits, softmax over experts and top-k with renormalised gate weights.
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §2.1: the gating network is a
// linear layer followed by softmax; the top-2 expert indices are kept and their
// gate weights renormalised.  §3.2: one gating kernel per token, a warp-level
// shuffle reduction, maximum first then the runner-up.  [P3] (wzjinhao.cn)
// §3.2: softmax(x W + b) with the maximum subtracted first.
//
// gfx950 design: the logits are a skinny [T,d]x[d,E] contraction.  Small
// batches (T*E < 4096) and fp32 activations run on the VALU: a 256-thread
// block owns 1 (or 8) tokens x 4 experts, its threads split K in 4-element
// chunks with the loads of several chunks in flight, and the per-lane partial
// sums are folded with a transposing wave reduction before a cross-wave sum in
// LDS.  Larger bf16 batches run on the matrix cores (router_mfma_kernel; 64 x
// 64 tiles for large batches with many experts; with at most 16 experts the
// logits and the top-k share one launch).  Top-k runs one wave64 per token:
// each lane holds up to 4 logits, and k rounds of a shuffle argmax (value
// descending, expert index ascending on ties) pick the experts.  Selection is made on the fp32 logits (softmax is monotone); the
// weights are the softmax of the selected logits, which equals the full
// softmax renormalised over the selection.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

// Transposing reduction of N per-lane values over the 64 lanes.  Afterwards
// lane l holds the wave total of value index (l >> (6 - log2 N)).
template <int N>
__device__ __forceinline__ float wave_reduce_multi(float (&v)[N], int lane) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N power of two");
    int n = N;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        if (n > 1) {
            const bool up = (lane & o) != 0;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                if (i < n / 2) {
                    float send = up ? v[i] : v[i + n / 2];
                    float keep = up ? v[i + n / 2] : v[i];
                    v[i] = keep + __shfl_xor(send, o, MOE_WAVE);
                }
            }
            n >>= 1;
        } else {
            v[0] += __shfl_xor(v[0], o, MOE_WAVE);
        }
    }
    return v[0];
}

constexpr int RT_EXP = 4;
constexpr int RT_THREADS = 256;

// TT tokens x 4 experts per block; the 256 threads split K in 4-element
// chunks, U chunks of loads are issued before their arithmetic.  TT = 8
// reuses each router row for 8 tokens (many tokens; U = 1 keeps the register
// count low enough for two blocks per CU); TT = 1 gives small batches
// (decode) T x E/4 blocks instead of a handful, with U = 4.
template <int ACT, int TT, int RT_U = (TT == 1 ? 4 : 1)>
__global__ __launch_bounds__(RT_THREADS) void router_logits_kernel(
    const void* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int d, int E) {
    const int t0 = blockIdx.x * TT;
    const int e0 = blockIdx.y * RT_EXP;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int NV = TT * RT_EXP;
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;
    const int ne = min(RT_EXP, E - e0);
    const int nt = min(TT, T - t0);

    for (int k0 = tid * 4; k0 < d; k0 += RT_THREADS * 4 * RT_U) {
        // every load is issued unconditionally (rows clamped into range, K
        // chunks past d re-read chunk 0 and are zeroed afterwards), so all of
        // them are in flight before the first use
        float4 wv[RT_U][RT_EXP];
        using XRaw = typename std::conditional<ACT == DT_F32, float4, uint2>::type;
        XRaw xr[RT_U][TT];
#pragma unroll
        for (int u = 0; u < RT_U; ++u) {
            const int kk = k0 + u * RT_THREADS * 4;
            const int kc = kk < d ? kk : 0;
#pragma unroll
            for (int e = 0; e < RT_EXP; ++e)
                wv[u][e] = *reinterpret_cast<const float4*>(wg + (size_t)(e0 + min(e, ne - 1)) * d + kc);
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const size_t row = (size_t)(t0 + min(t, nt - 1)) * d + kc;
                xr[u][t] = *reinterpret_cast<const XRaw*>(reinterpret_cast<const char*>(x) + row * sizeof(XRaw) / 4);
            }
        }
        // keep the loads above together, ahead of their first use
        __builtin_amdgcn_sched_barrier(0);
        float xv[RT_U][TT][4];
#pragma unroll
        for (int u = 0; u < RT_U; ++u) {
            if (k0 + u * RT_THREADS * 4 >= d) {
#pragma unroll
                for (int e = 0; e < RT_EXP; ++e) wv[u][e] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if constexpr (ACT == DT_F32) {
                    xv[u][t][0] = xr[u][t].x; xv[u][t][1] = xr[u][t].y; xv[u][t][2] = xr[u][t].z; xv[u][t][3] = xr[u][t].w;
                } else {
                    xv[u][t][0] = bf16_lo(xr[u][t].x); xv[u][t][1] = bf16_hi(xr[u][t].x);
                    xv[u][t][2] = bf16_lo(xr[u][t].y); xv[u][t][3] = bf16_hi(xr[u][t].y);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < RT_U; ++u)
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int e = 0; e < RT_EXP; ++e) {
                    float s = acc[t * RT_EXP + e];
                    s = fmaf(xv[u][t][0], wv[u][e].x, s);
                    s = fmaf(xv[u][t][1], wv[u][e].y, s);
                    s = fmaf(xv[u][t][2], wv[u][e].z, s);
                    s = fmaf(xv[u][t][3], wv[u][e].w, s);
                    acc[t * RT_EXP + e] = s;
                }
    }
    // fold the NV partials over the wave: lane l owns output index l >> (6 - log2 NV)
    float r = wave_reduce_multi<NV>(acc, lane);
    constexpr int SH = NV == 32 ? 1 : NV == 16 ? 2 : NV == 8 ? 3 : 4;
    __shared__ float part[RT_THREADS / 64][NV];
    if ((lane & ((1 << SH) - 1)) == 0) part[wave][lane >> SH] = r;
    __syncthreads();
    if (tid < NV) {
        const int t = tid / RT_EXP, e = tid % RT_EXP;
        float s = part[0][tid];
#pragma unroll
        for (int w = 1; w < RT_THREADS / 64; ++w) s += part[w][tid];
        if (t < nt && e < ne) {
            if (bias) s += bias[e0 + e];
            logits[(size_t)(t0 + t) * E + e0 + e] = s;
        }
    }
}

// Router logits on the matrix cores for bf16 activations and larger batches.
// The fp32 router row w is split exactly into three bf16 terms by truncation:
// hi = w with the low 16 bits cleared, mid = (w - hi) likewise, lo = w - hi -
// mid (at most 8 significant bits left, so exact in bf16); each product with a
// bf16 activation is exact in fp32, and v_mfma_f32_16x16x32_bf16 accumulates
// x.hi + x.mid + x.lo in fp32 -- the fp32 contraction, summed in another
// order.  A block owns 16 tokens x 16 experts; its RQ_WAVES waves split K
// into contiguous ranges, and the partial tiles are summed in LDS in wave
// order (deterministic).  A lane loads 8 consecutive K of one token row (A)
// and 8 of one router row (B), as the MFMA operand layouts want.
constexpr int RQ_WAVES = 8;
constexpr int RQ_U = 4;     // K steps of loads in flight

typedef __bf16 rq_bf16x8 __attribute__((ext_vector_type(8)));
typedef float rq_f4 __attribute__((ext_vector_type(4)));
typedef unsigned int rq_u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split3(const float4& a, const float4& b, rq_u4& hi, rq_u4& mid, rq_u4& lo) {
    const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t u = __float_as_uint(w[i]);
        const uint32_t uh = u & 0xffff0000u;
        const float r1 = w[i] - __uint_as_float(uh);
        const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(um);
        h[i] = uh >> 16;
        m[i] = um >> 16;
        l[i] = __float_as_uint(r2) >> 16;      // exact: r2 has <= 8 significant bits
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = h[2 * i] | (h[2 * i + 1] << 16);
        mid[i] = m[2 * i] | (m[2 * i + 1] << 16);
        lo[i] = l[2 * i] | (l[2 * i + 1] << 16);
    }
}

// One wave's 16 x 16 tile (tokens of xrow's block x router rows of wrow's
// block) over K steps [s0, s1) of 32: lane (r, q) loads 8 consecutive K of
// token row r and of router row r at K = 32 step + 8 q.
__device__ __forceinline__ rq_f4 router_k_range(const uint16_t* __restrict__ xrow, const float* __restrict__ wrow,
                                                int s0, int s1, int q, int d) {
    rq_f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int st = s0; st < s1; st += RQ_U) {
        uint4 xa[RQ_U];
        float4 wa[RQ_U][2];
#pragma unroll
        for (int u = 0; u < RQ_U; ++u) {
            const int k = (st + u) * 32 + q * 8;
            const int kc = (st + u < s1 && k < d) ? k : 0;
            xa[u] = *reinterpret_cast<const uint4*>(xrow + kc);
            wa[u][0] = *reinterpret_cast<const float4*>(wrow + kc);
            wa[u][1] = *reinterpret_cast<const float4*>(wrow + kc + 4);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < RQ_U; ++u) {
            const int k = (st + u) * 32 + q * 8;
            const bool ok = st + u < s1 && k < d;
            rq_u4 av = {ok ? xa[u].x : 0u, ok ? xa[u].y : 0u, ok ? xa[u].z : 0u, ok ? xa[u].w : 0u};
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            rq_u4 hi, mid, lo;
            split3(ok ? wa[u][0] : z, ok ? wa[u][1] : z, hi, mid, lo);
            const rq_bf16x8 A = __builtin_bit_cast(rq_bf16x8, av);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(rq_bf16x8, hi), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(rq_bf16x8, mid), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(rq_bf16x8, lo), acc, 0, 0, 0);
        }
    }
    return acc;
}

__global__ __launch_bounds__(64 * RQ_WAVES) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int d, int E) {
    const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int tr = min(t0 + r, T - 1), er = min(e0 + r, E - 1);   // clamped rows: results unused
    // this wave's K range, in steps of 32 (the last step may be partial: d % 8 == 0)
    const int nsteps = (d + 31) / 32;
    const int s0 = nsteps * wave / RQ_WAVES, s1 = nsteps * (wave + 1) / RQ_WAVES;
    const rq_f4 acc = router_k_range(x + (size_t)tr * d, wg + (size_t)er * d, s0, s1, q, d);
    // lane l holds tokens 4(l/16)+v, expert l%16; sum the waves' tiles in order
    __shared__ float part[RQ_WAVES][4][64];
#pragma unroll
    for (int v = 0; v < 4; ++v) part[wave][v][lane] = acc[v];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float sum = part[0][v][lane];
#pragma unroll
            for (int w = 1; w < RQ_WAVES; ++w) sum += part[w][v][lane];
            const int t = t0 + 4 * q + v, e = e0 + r;
            if (t < T && e < E) {
                if (bias) sum += bias[e];
                logits[(size_t)t * E + e] = sum;
            }
        }
    }
}

// Large batches with many experts (T*E >= 2^20, E >= 64): the kernel above
// gives every 16 x 16 tile its own block, so each x row is read once per 16
// experts and each router row once per 16 tokens, and every lane splits the
// router values it multiplies.  Here a 512-thread block owns 64 tokens x 64
// experts and stages K in chunks of 64 in LDS: the x chunk as bf16, the router
// chunk split once per block into the same three bf16 terms.  Wave (wm, we,
// kh) multiplies tokens 32 wm .. +31 with experts 32 we .. +31 over K half kh
// of every chunk on v_mfma_f32_32x32x16_bf16, three MFMAs (hi, mid, lo) per
// 16 K (two waves per SIMD); at the end the kh = 1 waves park their sums in
// LDS and the kh = 0 waves add them (a fixed order: deterministic).  LDS rows
// are 128 bytes with their 16-byte chunks XOR-swizzled by (row/2)&7.
constexpr int RTL_T = 64, RTL_E = 64, RTL_K = 64, RTL_THREADS = 512;

typedef float rtl_f16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int rtl_swz(int row, int ch) { return row * RTL_K + ((ch ^ ((row >> 1) & 7)) << 3); }

__global__ __launch_bounds__(RTL_THREADS) void router_tile_kernel(const uint16_t* __restrict__ x,
                                                                  const float* __restrict__ wg,
                                                                  const float* __restrict__ bias,
                                                                  float* __restrict__ logits, int T, int d, int E) {
    __shared__ __attribute__((aligned(16))) uint16_t sx[2][RTL_T * RTL_K];
    __shared__ __attribute__((aligned(16))) uint16_t sw[2][3][RTL_E * RTL_K];
    __shared__ float spart[4][16][64];                   // the kh = 1 waves' sums
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, we = (wave >> 1) & 1, kh = wave >> 2;
    const int h = lane >> 5, r32 = lane & 31;
    const int t0 = blockIdx.x * RTL_T, e0 = blockIdx.y * RTL_E;
    const int nch = (d + RTL_K - 1) / RTL_K;
    // staging: the x piece tid (row tid/8, 16-byte chunk tid%8) and the router
    // pieces tid + 512 i (row p/16, 4 floats at 4 (p%16)), i < 2; chunks are
    // loaded into registers RTL_D chunks ahead (a ring, the loop unrolled by
    // RTL_D so that every index is static)
    constexpr int RTL_D = 4;
    uint4 xr[RTL_D];
    float4 wr[RTL_D][2];
    auto load = [&](int c, int u) __attribute__((always_inline)) {
        const int k0 = c * RTL_K;
        {
            const int row = tid >> 3, k = k0 + 8 * (tid & 7);
            const int t = min(t0 + row, T - 1);          // clamped rows: their results are not stored
            xr[u] = k < d ? *reinterpret_cast<const uint4*>(x + (size_t)t * d + k) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = tid + RTL_THREADS * i, row = p >> 4, k = k0 + 4 * (p & 15);
            const int e = min(e0 + row, E - 1);
            wr[u][i] = k < d ? *reinterpret_cast<const float4*>(wg + (size_t)e * d + k)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store = [&](int u, int buf) __attribute__((always_inline)) {
        *reinterpret_cast<uint4*>(&sx[buf][rtl_swz(tid >> 3, tid & 7)]) = xr[u];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = tid + RTL_THREADS * i, row = p >> 4, c4 = p & 15;
            const float v[4] = {wr[u][i].x, wr[u][i].y, wr[u][i].z, wr[u][i].w};
            uint32_t hi[4], mid[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t uu = __float_as_uint(v[q]);
                const uint32_t uh = uu & 0xffff0000u;
                const float r1 = v[q] - __uint_as_float(uh);
                const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
                const float r2 = r1 - __uint_as_float(um);
                hi[q] = uh >> 16;
                mid[q] = um >> 16;
                lo[q] = __float_as_uint(r2) >> 16;     // exact: r2 has <= 8 significant bits
            }
            const int o = rtl_swz(row, c4 >> 1) + 4 * (c4 & 1);
            *reinterpret_cast<uint2*>(&sw[buf][0][o]) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
            *reinterpret_cast<uint2*>(&sw[buf][1][o]) = make_uint2(mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16));
            *reinterpret_cast<uint2*>(&sw[buf][2][o]) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
        }
    };
    // one accumulator per bf16 term, so consecutive MFMAs do not wait on each
    // other; summed hi + mid + lo at the end
    rtl_f16 acc3[3];
#pragma unroll
    for (int term = 0; term < 3; ++term)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc3[term][v] = 0.f;
    const int ta = 32 * wm + r32, eb = 32 * we + r32;   // the lane's token (A) and expert (B) rows
    // chunk c sits in LDS buffer c % 2: chunk c + 1 is split and stored while
    // chunk c's MFMAs run, then one barrier
#pragma unroll
    for (int u = 0; u < RTL_D; ++u)
        if (u < nch) load(u, u);
    store(0, 0);
    if (RTL_D < nch) load(RTL_D, 0);
    __syncthreads();
    for (int c0 = 0; c0 < nch; c0 += RTL_D) {
#pragma unroll
        for (int u = 0; u < RTL_D; ++u) {
            const int c = c0 + u;
            if (c >= nch) break;
            const int buf = u & 1;              // c % 2 (RTL_D is even)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int ch = 2 * (2 * kh + s2) + h;
                const rq_bf16x8 A = *reinterpret_cast<const rq_bf16x8*>(&sx[buf][rtl_swz(ta, ch)]);
#pragma unroll
                for (int term = 0; term < 3; ++term) {
                    const rq_bf16x8 B = *reinterpret_cast<const rq_bf16x8*>(&sw[buf][term][rtl_swz(eb, ch)]);
                    acc3[term] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc3[term], 0, 0, 0);
                }
            }
            if (c + 1 < nch) {
                const int un = (u + 1) % RTL_D;  // chunk c + 1's register slot
                store(un, buf ^ 1);
                if (c + 1 + RTL_D < nch) load(c + 1 + RTL_D, un);
            }
            __syncthreads();                    // chunk c + 1 published; chunk c's reads done
        }
    }
    rtl_f16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = (acc3[0][v] + acc3[1][v]) + acc3[2][v];
    if (kh == 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) spart[wave & 3][v][lane] = acc[v];
    }
    __syncthreads();
    if (kh == 1) return;
    // lane l, element v: token 8 (v/4) + 4 h + v%4 of the wave's 32, expert l%32
    const int e = e0 + eb;
    if (e < E) {
        const float bv = bias ? bias[e] : 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = t0 + 32 * wm + 8 * (v >> 2) + 4 * h + (v & 3);
            if (t < T) logits[(size_t)t * E + e] = (acc[v] + spart[wave][v][lane]) + bv;
        }
    }
}

// (value, index) is better than (v2, i2): larger value, or equal value and
// lower expert index.  NaN was mapped to -inf before, so every unchosen expert
// stays comparable and exactly k distinct experts are always selected.
__device__ __forceinline__ bool better(float v, int i, float v2, int i2) {
    return v > v2 || (v == v2 && i < i2);
}

constexpr int TK_MAXPL = 4;   // E <= 256 -> up to 4 logits per lane
constexpr int TK_MAXK = 16;

// Top-k of one token by one wave: lane l holds logits l + 64 i (live when
// < E).  k rounds of a shuffle argmax; the owner retires each winner.  Writes
// the k indices and the softmax of the selected logits (max-subtracted; the
// first selected is the maximum).  selv: this wave's TK_MAXK floats of LDS.
__device__ __forceinline__ void topk_wave(float (&v)[TK_MAXPL], bool (&live)[TK_MAXPL], int lane, int k,
                                          int32_t* __restrict__ idx_row, float* __restrict__ w_row,
                                          float* selv) {
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < TK_MAXPL; ++i)
            if (live[i] && better(v[i], lane + 64 * i, bv, bi)) { bv = v[i]; bi = lane + 64 * i; }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            float ov = __shfl_xor(bv, o, MOE_WAVE);
            int oi = __shfl_xor(bi, o, MOE_WAVE);
            if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
#pragma unroll
        for (int i = 0; i < TK_MAXPL; ++i)
            if (lane + 64 * i == bi) live[i] = false;
        if (lane == 0) {
            idx_row[j] = bi;
            selv[j] = bv;
        }
    }
    if (lane == 0) {
        const float m = selv[0];
        float s = 0.f;
        for (int j = 0; j < k; ++j) s += expf(selv[j] - m);
        const float inv = 1.0f / s;
        for (int j = 0; j < k; ++j) w_row[j] = expf(selv[j] - m) * inv;
    }
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                  int32_t* __restrict__ idx,
                                                  float* __restrict__ w, int T, int E, int k) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    __shared__ float selv[4][TK_MAXK];
    if (t >= T) return;
    float v[TK_MAXPL];
    bool live[TK_MAXPL];
#pragma unroll
    for (int i = 0; i < TK_MAXPL; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < E;
        float x = live[i] ? logits[(size_t)t * E + e] : -INFINITY;
        v[i] = (x != x) ? -INFINITY : x;
    }
    topk_wave(v, live, lane, k, idx + (size_t)t * k, w + (size_t)t * k, selv[wave]);
}

// Router logits and top-k in one launch for bf16 batches with up to 16
// experts (the grid of router_mfma_kernel is then one block per 16 tokens
// anyway): a 1024-thread block owns 16 tokens x all experts.  Its 16 waves
// split into the ceil(E/16) expert tiles (1, 2 or 4; the kernel takes up to 64
// experts, but above 16 every block would split the whole router, which the
// two-launch path spreads over E/16 blocks) times the K ranges that leave;
// each wave runs the 16 x 16 tile of router_mfma_kernel over its K range, the
// partial tiles are summed in K-range order in LDS (deterministic), the logits
// written out, and wave w then selects the top-k of token w with the rule of
// topk_kernel.
constexpr int RK_WAVES = 16;

__global__ __launch_bounds__(64 * RK_WAVES) void router_topk_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ w, int T, int d, int E, int k) {
    __shared__ float part[RK_WAVES][4][64];
    __shared__ float lg[16][64];
    __shared__ float selv[RK_WAVES][TK_MAXK];
    const int t0 = blockIdx.x * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int net = E <= 16 ? 1 : (E <= 32 ? 2 : 4);     // expert tiles
    const int nkr = RK_WAVES / net;                       // K ranges per tile
    const int et = wave % net, kr = wave / net;
    const int tr = min(t0 + r, T - 1), er = min(et * 16 + r, E - 1);   // clamped rows: results unused
    const int nsteps = (d + 31) / 32;
    const int s0 = nsteps * kr / nkr, s1 = nsteps * (kr + 1) / nkr;
    const rq_f4 acc = router_k_range(x + (size_t)tr * d, wg + (size_t)er * d, s0, s1, q, d);
#pragma unroll
    for (int v = 0; v < 4; ++v) part[wave][v][lane] = acc[v];
    __syncthreads();
    // wave e' < net sums tile e' over the K ranges in order: lane (r, q)
    // holds tokens 4q + v of expert 16 e' + r
    if (wave < net) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float sum = part[wave][v][lane];
            for (int j = 1; j < nkr; ++j) sum += part[wave + j * net][v][lane];
            const int t = t0 + 4 * q + v, e = wave * 16 + r;
            if (e < E) {
                if (bias) sum += bias[e];
                lg[4 * q + v][e] = sum;
                if (t < T) logits[(size_t)t * E + e] = sum;
            }
        }
    }
    __syncthreads();
    const int t = t0 + wave;
    if (t >= T) return;
    float v[TK_MAXPL];
    bool live[TK_MAXPL];
    live[0] = lane < E;
    const float xv = live[0] ? lg[wave][lane] : -INFINITY;
    v[0] = (xv != xv) ? -INFINITY : xv;
#pragma unroll
    for (int i = 1; i < TK_MAXPL; ++i) {
        live[i] = false;
        v[i] = -INFINITY;
    }
    topk_wave(v, live, lane, k, idx + (size_t)t * k, w + (size_t)t * k, selv[wave]);
}

hipError_t launch_route(int act, const void* x, const float* wg, const float* b, float* logits,
                        int32_t* idx, float* w, int T, int d, int E, int k, hipStream_t s) {
    if (T == 0) return hipSuccess;
    // few tokens x experts (decode): one token per block for enough blocks
    const bool small = (long)T * E < 4096;
    const int tt = small ? 1 : 8;
    dim3 g1((T + tt - 1) / tt, (E + RT_EXP - 1) / RT_EXP);
    if (act == DT_F32) {
        if (small) hipLaunchKernelGGL((router_logits_kernel<DT_F32, 1>), g1, dim3(RT_THREADS), 0, s, x, wg, b, logits, T, d, E);
        else hipLaunchKernelGGL((router_logits_kernel<DT_F32, 8>), g1, dim3(RT_THREADS), 0, s, x, wg, b, logits, T, d, E);
    } else if (small) {
        hipLaunchKernelGGL((router_logits_kernel<DT_BF16, 1>), g1, dim3(RT_THREADS), 0, s, x, wg, b, logits, T, d, E);
    } else if ((long)T * E >= (1L << 20) && E >= RTL_E) {
        const dim3 g3((T + RTL_T - 1) / RTL_T, (E + RTL_E - 1) / RTL_E);
        hipLaunchKernelGGL(router_tile_kernel, g3, dim3(RTL_THREADS), 0, s, reinterpret_cast<const uint16_t*>(x), wg, b,
                           logits, T, d, E);
    } else if (E <= 16) {
        // logits and top-k in one launch
        hipLaunchKernelGGL(router_topk_kernel, dim3((T + 15) / 16), dim3(64 * RK_WAVES), 0, s,
                           reinterpret_cast<const uint16_t*>(x), wg, b, logits, idx, w, T, d, E, k);
        return hipGetLastError();
    } else {
        const dim3 g2((T + 15) / 16, (E + 15) / 16);
        hipLaunchKernelGGL(router_mfma_kernel, g2, dim3(64 * RQ_WAVES), 0, s,
                           reinterpret_cast<const uint16_t*>(x), wg, b, logits, T, d, E);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, idx, w, T, E, k);
    return hipGetLastError();
}

}  // namespace moe
