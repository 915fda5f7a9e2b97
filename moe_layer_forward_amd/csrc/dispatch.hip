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
// gfx950 design: one 1024-thread workgroup (16 wave64s); wave w owns the
// contiguous chunk [w C, (w+1) C) of the assignments (C a multiple of 64), so
// the waves work independently between two barriers:
//  1. each wave counts the experts of its chunk into its row of a
//     [wave][expert] LDS table (integer atomics: order-independent);
//  2. one thread per expert sums its column (the counts) and wave 0 scans
//     the E <= 256 counts (4 per lane, a shuffle scan) for the offsets; each
//     expert's column then becomes the start of each wave's run of it
//     (offset + the counts of the lower waves);
//  3. each wave walks its chunk in groups of 64 in order: inside a group the
//     lanes holding the same expert find each other with ballots on the key
//     bits (peer mask; only the bits E-1 needs), an assignment lands at its
//     wave's cursor for its expert plus its rank among the lower peers, and
//     the lowest peer advances the cursor (the wave's own LDS operations stay
//     in program order).
// Chunks in wave order, groups in chunk order and ranks in lane order make
// this the stable counting sort, bit for bit.  With plan arguments, wave 0
// also writes the grouped GEMM's tile lists once the offsets are known
// (plan.h).
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

constexpr int DP_THREADS = 1024;
constexpr int DP_WAVES = DP_THREADS / 64;
constexpr int DP_MAXE = 256;

// Peer mask of this lane's key among the wave's valid lanes (same key); keys
// below 2^nbits.
__device__ __forceinline__ uint64_t key_peers(int key, bool valid, int nbits) {
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        if (b >= nbits) break;
        const bool bit = valid && ((key >> b) & 1);
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

// KB: groups of keys a wave holds in registers (all loaded together).  When
// the wave's chunk fits one such batch, the keys stay in registers from the
// counting pass to the placement pass.
template <int KB>
__global__ __launch_bounds__(DP_THREADS) void dispatch_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int n, int E, MfmaPlanArgs plan) {
    __shared__ int s_tab[DP_WAVES][DP_MAXE];
    __shared__ int s_cnt[DP_MAXE];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // this wave's chunk, in groups of 64 (ngc groups, the same for every wave)
    const int C = ((n + DP_WAVES - 1) / DP_WAVES + 63) & ~63;
    const int ngc = C / 64;
    const int c0 = wave * C, c1 = min(n, c0 + C);
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;      // key bits that can differ

    for (int i = tid; i < DP_WAVES * DP_MAXE; i += DP_THREADS) (&s_tab[0][0])[i] = 0;
    __syncthreads();

    int keys[KB];
    // the keys of KB groups from group g0 of the chunk (invalid: -1)
    auto load_keys = [&](int g0) {
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int i = c0 + 64 * (g0 + u) + lane;
            const int key = i < c1 ? idx[i] : -1;
            keys[u] = (key >= 0 && key < E) ? key : -1;
        }
    };

    // 1. per-wave counts (LDS integer atomics: order-independent)
    for (int g0 = 0; g0 < ngc; g0 += KB) {
        load_keys(g0);
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            if (g0 + u >= ngc) break;
            if (keys[u] >= 0) atomicAdd(&s_tab[wave][keys[u]], 1);
        }
    }
    __syncthreads();

    // 2. counts, offsets, and each wave's start in each expert's range
    if (tid < E) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < DP_WAVES; ++w) c += s_tab[w][tid];
        s_cnt[tid] = c;
    }
    __syncthreads();
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
                s_cnt[e] = run;
            }
            run += c[j];
        }
        if (lane == 63) offsets[E] = incl;
        if (plan.tiles) mfma_plan_wave(lane, c, o, E, plan);
    }
    __syncthreads();
    if (tid < E) {
        int run = s_cnt[tid];
#pragma unroll
        for (int w = 0; w < DP_WAVES; ++w) {
            const int c = s_tab[w][tid];
            s_tab[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();

    // 3. placement
    for (int g0 = 0; g0 < ngc; g0 += KB) {
        if (ngc > KB) load_keys(g0);       // else the keys of pass 1 are still here
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            if (g0 + u >= ngc) break;
            const bool valid = keys[u] >= 0;
            const uint64_t peers = key_peers(keys[u], valid, nbits);
            const int rank = __popcll(peers & lt_mask);
            if (valid) {
                const int pos = s_tab[wave][keys[u]] + rank;
                const int i = c0 + 64 * (g0 + u) + lane;
                perm[pos] = i;
                inv[i] = pos;
            }
            // every lane of the group has read the cursor (program order
            // within the wave) before its lowest lane advances it
            if (valid && rank == 0) s_tab[wave][keys[u]] += __popcll(peers);
        }
    }
}

hipError_t launch_dispatch(const int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, int T, int k, int E, hipStream_t s, const MfmaPlanArgs* plan) {
    if (plan && (E > DP_MAXE || plan->tile_mode < MFMA_TILES_BOTH || plan->tile_mode > MFMA_TILES_BIG))
        return hipErrorInvalidValue;
    const MfmaPlanArgs p = plan ? *plan : MfmaPlanArgs{nullptr, 0, 0, 0, 0};
    const int n = T * k;
    // groups of 64 per wave: up to 8 in one batch, else batches of 32
    if (n <= DP_WAVES * 64 * 8)
        hipLaunchKernelGGL(dispatch_kernel<8>, dim3(1), dim3(DP_THREADS), 0, s, idx, counts, offsets, perm, inv, n, E, p);
    else
        hipLaunchKernelGGL(dispatch_kernel<32>, dim3(1), dim3(DP_THREADS), 0, s, idx, counts, offsets, perm, inv, n, E, p);
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
