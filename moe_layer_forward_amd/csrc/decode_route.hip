// Router, softmax, top-k and dispatch of a decode batch in one kernel.
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §3.2: the per-token
// gating path (linear layer, softmax, top-2) as one fused kernel, so a decode
// step pays one launch for it; §3.3: the token map and expert offsets handed
// to the expert kernels.  [P2] "Colibri不是一只蜂鸟，而是一套为前沿MoE模型量身定制的C语言推理引擎"
// §4.2: the counting-sort dispatcher (histogram, running offsets, placement).
//
// gfx950 design: one 512-thread workgroup for batches with T*E <= 64 (the
// Mixtral-shaped decode batch of 8 tokens x 8 experts).  The eight waves split
// K: each lane owns 4 consecutive K elements per 2048-wide slice and keeps the
// partial dot products of all T*E (token, expert) pairs in registers, so every
// element of x and of the router is read once.  A transposing wave reduction
// leaves pair p's wave total in lane p; the eight wave totals are summed in LDS
// in wave order (deterministic).  Top-k runs one wave per token with the same
// selection rule as the batched kernel (larger logit first, lower expert index
// on ties; weights = softmax over the selection).  The T*k <= 64 assignments
// are then placed by the stable counting sort written out directly: a thread
// per assignment ranks itself among the earlier assignments of its expert.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int DR_THREADS = 512;
constexpr int DR_WAVES = DR_THREADS / 64;
constexpr int DR_PAIRS = 64;        // T * E limit
constexpr int DR_MAXK = 16;

// T tokens x E experts fit the 64 register-held pairs: E <= 8 with T <= 8,
// or E <= 16 with T <= 4
bool route_dispatch_small_supported(int T, int E, int k) {
    return T >= 1 && k >= 1 && k <= E && k <= DR_MAXK && ((E <= 8 && T <= 8) || (E <= 16 && T <= 4));
}

// Transposing reduction of 64 per-lane values: afterwards lane l holds the
// wave total of value l.  Level with N live values and lane bit O: a lane
// keeps the half of its values selected by that bit and adds its partner's
// copy of the same half (compile-time indices throughout).
template <int N, int O>
__device__ __forceinline__ void dr_level(float (&v)[DR_PAIRS], int lane) {
    if constexpr (N > 1) {
        const bool up = (lane & O) != 0;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float send = up ? v[i] : v[i + N / 2];
            const float keep = up ? v[i + N / 2] : v[i];
            v[i] = keep + __shfl_xor(send, O, MOE_WAVE);
        }
        dr_level<N / 2, O / 2>(v, lane);
    }
}

__device__ __forceinline__ float dr_reduce64(float (&v)[DR_PAIRS], int lane) {
    dr_level<DR_PAIRS, 32>(v, lane);
    return v[0];
}

// EM: experts per token held in registers (E <= EM); TM = 64 / EM tokens
template <int ACT, int EM>
__global__ __launch_bounds__(DR_THREADS) void route_dispatch_small_kernel(
    const void* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv, int T, int d, int E,
    int k) {
    constexpr int TM = DR_PAIRS / EM;
    __shared__ float part[DR_WAVES][DR_PAIRS];
    __shared__ float s_lg[DR_PAIRS];
    __shared__ int s_idx[DR_PAIRS];
    __shared__ float s_sel[DR_PAIRS];
    __shared__ int s_cnt[DR_PAIRS];
    __shared__ int s_off[DR_PAIRS + 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    // 1. partial dots of pair p = t * EM + e over this lane's K elements
    float acc[DR_PAIRS];
#pragma unroll
    for (int p = 0; p < DR_PAIRS; ++p) acc[p] = 0.f;
    for (int k0 = tid * 4; k0 < d; k0 += DR_THREADS * 4) {
        float4 r[EM];
#pragma unroll
        for (int e = 0; e < EM; ++e)
            r[e] = *reinterpret_cast<const float4*>(wg + (size_t)(e < E ? e : E - 1) * d + k0);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t < T) {
                float xa[4];
                if constexpr (ACT == DT_F32) {
                    const float4 v =
                        *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + (size_t)t * d + k0);
                    xa[0] = v.x; xa[1] = v.y; xa[2] = v.z; xa[3] = v.w;
                } else {
                    const uint2 v =
                        *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + (size_t)t * d + k0);
                    xa[0] = bf16_lo(v.x); xa[1] = bf16_hi(v.x); xa[2] = bf16_lo(v.y); xa[3] = bf16_hi(v.y);
                }
#pragma unroll
                for (int e = 0; e < EM; ++e) {
                    float sum = acc[t * EM + e];
                    sum = fmaf(xa[0], r[e].x, sum);
                    sum = fmaf(xa[1], r[e].y, sum);
                    sum = fmaf(xa[2], r[e].z, sum);
                    sum = fmaf(xa[3], r[e].w, sum);
                    acc[t * EM + e] = sum;
                }
            }
        }
    }
    const float tot = dr_reduce64(acc, lane);
    part[wave][lane] = tot;
    __syncthreads();
    {
        const int t = tid / EM, e = tid % EM;
        if (tid < DR_PAIRS && t < T && e < E) {
            float sum = part[0][tid];
#pragma unroll
            for (int v = 1; v < DR_WAVES; ++v) sum += part[v][tid];
            if (bias) sum += bias[e];
            s_lg[t * E + e] = sum;
            logits[t * E + e] = sum;
        }
    }
    __syncthreads();

    // 2. top-k, one wave per token (E <= 64: one logit per lane)
    for (int t = wave; t < T; t += DR_WAVES) {
        float v = -INFINITY;
        bool live = lane < E;
        if (live) {
            const float lv = s_lg[t * E + lane];
            v = (lv != lv) ? -INFINITY : lv;
        }
        for (int j = 0; j < k; ++j) {
            float bv = live ? v : -INFINITY;
            int bi = live ? lane : 0x7fffffff;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float ov = __shfl_xor(bv, o, MOE_WAVE);
                const int oi = __shfl_xor(bi, o, MOE_WAVE);
                if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
            }
            if (lane == bi) live = false;
            if (lane == 0) {
                s_idx[t * k + j] = bi;
                s_sel[t * k + j] = bv;
            }
        }
        if (lane == 0) {
            const float m = s_sel[t * k];
            float s = 0.f;
            for (int j = 0; j < k; ++j) s += expf(s_sel[t * k + j] - m);
            const float r = 1.0f / s;
            for (int j = 0; j < k; ++j) {
                idx[t * k + j] = s_idx[t * k + j];
                w[t * k + j] = expf(s_sel[t * k + j] - m) * r;
            }
        }
    }
    __syncthreads();

    // 3. stable counting sort of the n = T*k assignments by expert
    const int n = T * k;
    if (tid < E) {
        int c = 0;
        for (int a = 0; a < n; ++a) c += s_idx[a] == tid;
        s_cnt[tid] = c;
        counts[tid] = c;
    }
    __syncthreads();
    if (tid <= E) {
        int o = 0;
        for (int e = 0; e < tid; ++e) o += s_cnt[e];
        s_off[tid] = o;
        offsets[tid] = o;
    }
    __syncthreads();
    if (tid < n) {
        const int e = s_idx[tid];
        int r = 0;
        for (int a = 0; a < tid; ++a) r += s_idx[a] == e;
        const int p = s_off[e] + r;
        perm[p] = tid;
        inv[tid] = p;
    }
}

hipError_t launch_route_dispatch_small(int act, const void* x, const float* wg, const float* b, float* logits,
                                       int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                                       int32_t* inv, int T, int d, int E, int k, hipStream_t s) {
    if (!route_dispatch_small_supported(T, E, k) || d % 4 != 0) return hipErrorInvalidValue;
#define DR_LAUNCH(A, M)                                                                                   \
    hipLaunchKernelGGL((route_dispatch_small_kernel<A, M>), dim3(1), dim3(DR_THREADS), 0, s, x, wg, b, logits, idx, \
                       w, counts, offsets, perm, inv, T, d, E, k)
    const bool narrow = E <= 8 && T <= 8;
    if (act == DT_F32) {
        if (narrow) DR_LAUNCH(DT_F32, 8); else DR_LAUNCH(DT_F32, 16);
    } else {
        if (narrow) DR_LAUNCH(DT_BF16, 8); else DR_LAUNCH(DT_BF16, 16);
    }
#undef DR_LAUNCH
    return hipGetLastError();
}

}  // namespace moe
