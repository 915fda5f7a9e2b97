// Dispatch: per-expert histogram, exclusive prefix sum and a stable placement
// of the T*k assignments (a = t*k + j) into expert-contiguous order.
//
// [P2] "Colibri不是一只蜂鸟，而是一套为前沿MoE模型量身定制的C语言推理引擎" §4.2:
// a counting-sort dispatcher (count per expert, running offsets, groups of
// token indices).  [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §3.3: a
// token-to-expert map plus per-expert offsets handed to the expert kernels.
// The pages sort on the host; here the whole step is one GPU workgroup so the
// layer never leaves the device.
//
// gfx950 design: one 1024-thread workgroup (16 wave64s).  The histogram uses
// LDS integer atomics (order-independent, so deterministic).  One wave scans
// the E <= 256 bins (4 per lane, a shuffle scan) for the offsets.  Placement walks the assignments
// in chunks of 1024: inside a wave, the rank of an element among equal keys
// comes from 8 ballots on the key bits (peer mask, popcount of lower peers);
// per-(wave, expert) counts go to an LDS table that is scanned wave-major per
// expert.  The result equals a stable counting sort, bit for bit.  The keys of
// DP_PF rounds are loaded together up front, so a round does not wait on its
// own global load.  With plan arguments, wave 0 also writes the grouped
// GEMM's tile lists once the offsets are known (plan.h).
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

constexpr int DP_THREADS = 1024;
constexpr int DP_WAVES = DP_THREADS / 64;
constexpr int DP_MAXE = 256;
constexpr int DP_PF = 8;      // rounds of keys loaded together

__global__ __launch_bounds__(DP_THREADS) void dispatch_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int n, int E, MfmaPlanArgs plan) {
    __shared__ int s_cnt[DP_MAXE];
    __shared__ int s_cursor[DP_MAXE];
    __shared__ int s_wave[DP_WAVES][DP_MAXE];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    for (int e = tid; e < DP_MAXE; e += DP_THREADS) s_cnt[e] = 0;
    for (int i = tid; i < DP_WAVES * DP_MAXE; i += DP_THREADS) (&s_wave[0][0])[i] = 0;
    __syncthreads();

    // 1. histogram
    for (int a = tid; a < n; a += DP_THREADS) {
        const int e = idx[a];
        if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();

    // 2. exclusive scan over the E bins: wave 0, 4 bins per lane, one barrier
    if (wave == 0) {
        int c[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            c[j] = (e < E) ? s_cnt[e] : 0;
            sum += c[j];
        }
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        int run = incl - sum, o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            o[j] = run;
            if (e < E) {
                counts[e] = c[j];
                offsets[e] = run;
                s_cursor[e] = run;
            }
            run += c[j];
        }
        if (lane == 63) offsets[E] = incl;
        if (plan.tiles) mfma_plan_wave(lane, c, o, E, plan);
    }
    __syncthreads();

    // 3. stable placement, 1024 assignments per round
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base0 = 0; base0 < n; base0 += DP_THREADS * DP_PF) {
        int keys[DP_PF];
#pragma unroll
        for (int r = 0; r < DP_PF; ++r) {
            const int a = base0 + r * DP_THREADS + tid;
            keys[r] = a < n ? idx[a] : -1;
        }
#pragma unroll
        for (int r = 0; r < DP_PF; ++r) {
            const int base = base0 + r * DP_THREADS;
            if (base >= n) break;
            const int a = base + tid;
            int key = keys[r];
            if (key < 0 || key >= E) key = -1;
            const bool valid = key >= 0;
            uint64_t peers = __ballot(valid);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const bool bit = valid && ((key >> b) & 1);
                const uint64_t m = __ballot(bit);
                peers &= bit ? m : ~m;
            }
            const int rank = __popcll(peers & lt_mask);
            if (valid && rank == 0) s_wave[wave][key] = __popcll(peers);
            __syncthreads();
            // per expert: exclusive scan over waves, then advance the cursor
            if (tid < E) {
                int run = s_cursor[tid];
#pragma unroll
                for (int w = 0; w < DP_WAVES; ++w) {
                    const int c = s_wave[w][tid];
                    s_wave[w][tid] = run;
                    run += c;
                }
                s_cursor[tid] = run;
            }
            __syncthreads();
            if (valid) {
                const int pos = s_wave[wave][key] + rank;
                perm[pos] = a;
                inv[a] = pos;
            }
            __syncthreads();
            // clear the table for the next round
            for (int i = tid; i < DP_WAVES * DP_MAXE; i += DP_THREADS) (&s_wave[0][0])[i] = 0;
            __syncthreads();
        }
    }
}

hipError_t launch_dispatch(const int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, int T, int k, int E, hipStream_t s, const MfmaPlanArgs* plan) {
    if (plan && (E > DP_MAXE || plan->tile_mode < MFMA_TILES_BOTH || plan->tile_mode > MFMA_TILES_BIG))
        return hipErrorInvalidValue;
    const MfmaPlanArgs p = plan ? *plan : MfmaPlanArgs{nullptr, 0, 0, 0, 0};
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(DP_THREADS), 0, s, idx, counts, offsets, perm,
                       inv, T * k, E, p);
    return hipGetLastError();
}

// The always-on shared expert as one group over all n tokens in token order:
// counts = {n}, offsets = {0, n}, perm = identity, so the expert kernels run
// it exactly as a routed expert that every token picked with one slot.
__global__ __launch_bounds__(256) void identity_group_kernel(int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) perm[i] = i;
    if (i == 0) {
        counts[0] = n;
        offsets[0] = 0;
        offsets[1] = n;
    }
}

hipError_t launch_identity_group(int32_t* counts, int32_t* offsets, int32_t* perm, int n, hipStream_t s) {
    const int blocks = n > 0 ? (n + 255) / 256 : 1;
    hipLaunchKernelGGL(identity_group_kernel, dim3(blocks), dim3(256), 0, s, counts, offsets, perm, n);
    return hipGetLastError();
}

// One-layer-ahead expert prediction, scored: for each token, how many of the
// k experts a prediction chose (pred) the layer then chose (actual).  [P5]
// "一只蜂鸟如何喂饱九头大象" §4.2: the router run one layer ahead picks the
// experts to fetch early, and the share it gets right bounds the time spent
// waiting for the rest.  hist[j] counts the tokens sharing exactly j experts.
// Integer work in one block: per-block LDS counts, then one write per bin.
__global__ __launch_bounds__(256) void topk_overlap_kernel(const int32_t* __restrict__ pred,
                                                           const int32_t* __restrict__ actual,
                                                           int32_t* __restrict__ hist, int T, int k) {
    __shared__ int s_h[17];
    const int tid = threadIdx.x;
    if (tid <= k) s_h[tid] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += 256) {
        int n = 0;
        for (int j = 0; j < k; ++j) {
            const int e = pred[(size_t)t * k + j];
            bool hit = false;
            for (int m = 0; m < k; ++m) hit |= actual[(size_t)t * k + m] == e;
            n += hit;
        }
        atomicAdd(&s_h[n], 1);
    }
    __syncthreads();
    if (tid <= k) hist[tid] = s_h[tid];
}

hipError_t launch_topk_overlap(const int32_t* pred, const int32_t* actual, int32_t* hist, int T, int k,
                               hipStream_t s) {
    hipLaunchKernelGGL(topk_overlap_kernel, dim3(1), dim3(256), 0, s, pred, actual, hist, T, k);
    return hipGetLastError();
}

}  // namespace moe
