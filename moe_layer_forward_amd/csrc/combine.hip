// Weighted combine back into token order, and the RMSNorm of the stacked layers.
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §2.1: the experts' outputs are
// merged with the gate weights.  [P4] "Colibri：轻量级MoE推理引擎的C语言实践" §2.3:
// the K slot results are merged back in the original token order.
//
// gfx950 design: a gather-reduce, never float atomics.  Each 256-thread block
// covers 1024 elements of one token: every thread reads its 4-element chunk of
// the token's k rows of y_perm through the inverse permutation (16-byte loads,
// all in flight together), sums them in slot order j = 0..k-1 in fp32 (plus
// the shared-expert row and the residual), and writes the output once.  The result is bit-identical run to run.  HBM-bound: k*d*4 bytes read
// and d*2 (bf16) written per token.
#include "common.h"
#include "kernels.h"

namespace moe {

template <int ACT, int KK>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ yp,
                                                     const int32_t* __restrict__ inv,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ ys,
                                                     const void* __restrict__ res,
                                                     void* __restrict__ y, int T, int d, int k) {
    // block (c, t): token t, elements [1024 c, 1024 c + 1024) -- each thread one
    // 4-element chunk, so all of a thread's k loads are in flight together;
    // consecutive blocks walk along the same rows (tokens beyond the grid's y
    // extent are taken in a stride)
    // KK > 0: k known at compile time, so all k loads of a thread are issued
    // together (a runtime trip count serialises them); KK == 0: any k <= 16
    if constexpr (KK > 0) k = KK;
    const int i = blockIdx.x * 1024 + threadIdx.x * 4;
    if (i >= d) return;
    for (int t = blockIdx.y; t < T; t += gridDim.y) {
        constexpr int NJ = KK > 0 ? KK : 16;
        float4 v[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (KK == 0 && j >= k) break;
            v[j] = *reinterpret_cast<const float4*>(yp + (size_t)inv[(size_t)t * k + j] * d + i);
        }
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (KK == 0 && j >= k) break;
            const float wj = w[(size_t)t * k + j];
            acc.x = fmaf(wj, v[j].x, acc.x);
            acc.y = fmaf(wj, v[j].y, acc.y);
            acc.z = fmaf(wj, v[j].z, acc.z);
            acc.w = fmaf(wj, v[j].w, acc.w);
        }
        if (ys) {
            const float4 q = *reinterpret_cast<const float4*>(ys + (size_t)t * d + i);
            acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
        }
        if constexpr (ACT == DT_F32) {
            if (res) {
                const float4 r = *reinterpret_cast<const float4*>(
                    reinterpret_cast<const float*>(res) + (size_t)t * d + i);
                acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
            }
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)t * d + i) = acc;
        } else {
            if (res) {
                const uint2 r = *reinterpret_cast<const uint2*>(
                    reinterpret_cast<const uint16_t*>(res) + (size_t)t * d + i);
                acc.x += bf16_lo(r.x); acc.y += bf16_hi(r.x); acc.z += bf16_lo(r.y); acc.w += bf16_hi(r.y);
            }
            uint2 o;
            o.x = pack_bf16x2(acc.x, acc.y);
            o.y = pack_bf16x2(acc.z, acc.w);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (size_t)t * d + i) = o;
        }
    }
}

hipError_t launch_combine(int act, const float* yp, const int32_t* inv, const float* w,
                          const float* ys, const void* res, void* y, int T, int d, int k,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (k > 16) return hipErrorInvalidValue;
    const dim3 g((d + 1023) / 1024, T < 65535 ? T : 65535);
#define MOE_COMBINE(A, KC) hipLaunchKernelGGL((combine_kernel<A, KC>), g, dim3(256), 0, s, yp, inv, w, ys, res, y, T, d, k)
#define MOE_COMBINE_K(A)                              \
    switch (k) {                                      \
        case 1: MOE_COMBINE(A, 1); break;             \
        case 2: MOE_COMBINE(A, 2); break;             \
        case 4: MOE_COMBINE(A, 4); break;             \
        case 6: MOE_COMBINE(A, 6); break;             \
        case 8: MOE_COMBINE(A, 8); break;             \
        default: MOE_COMBINE(A, 0); break;            \
    }
    if (act == DT_F32) {
        MOE_COMBINE_K(DT_F32)
    } else {
        MOE_COMBINE_K(DT_BF16)
    }
#undef MOE_COMBINE_K
#undef MOE_COMBINE
    return hipGetLastError();
}

// RMSNorm: out = h / sqrt(mean(h^2) + eps) * gamma, fp32 math.  One block per
// token; each thread takes 8-element chunks (one 16-byte load in bf16), sums
// their squares, and after the block sum scales the same chunks (the second
// read hits the cache).
template <int ACT>
__device__ __forceinline__ void load8(const void* p, size_t i, float (&v)[8]) {
    if constexpr (ACT == DT_F32) {
        const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
        const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
}

template <int ACT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ h,
                                                     const float* __restrict__ gamma, float eps,
                                                     void* __restrict__ out, int d) {
    const int t = blockIdx.x;
    const int nch = d / 8;
    float ss = 0.f;
    for (int c = threadIdx.x; c < nch; c += 256) {
        float v[8];
        load8<ACT>(h, (size_t)t * d + (size_t)c * 8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
    }
    ss = wave_sum(ss);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = part[0] + part[1] + part[2] + part[3];
    const float r = 1.0f / sqrtf(tot / (float)d + eps);
    for (int c = threadIdx.x; c < nch; c += 256) {
        float v[8], g[8];
        load8<ACT>(h, (size_t)t * d + (size_t)c * 8, v);
        if (gamma) {
            load8<DT_F32>(gamma, (size_t)c * 8, g);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) g[i] = 1.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = v[i] * r * g[i];
        const size_t o = (size_t)t * d + (size_t)c * 8;
        if constexpr (ACT == DT_F32) {
            float* q = reinterpret_cast<float*>(out) + o;
            *reinterpret_cast<float4*>(q) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(q + 4) = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            uint4 q;
            q.x = pack_bf16x2(v[0], v[1]);
            q.y = pack_bf16x2(v[2], v[3]);
            q.z = pack_bf16x2(v[4], v[5]);
            q.w = pack_bf16x2(v[6], v[7]);
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + o) = q;
        }
    }
}

hipError_t launch_rmsnorm(int act, const void* h, const float* gamma, float eps, void* out, int T,
                          int d, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (act == DT_F32)
        hipLaunchKernelGGL(rmsnorm_kernel<DT_F32>, dim3(T), dim3(256), 0, s, h, gamma, eps, out, d);
    else
        hipLaunchKernelGGL(rmsnorm_kernel<DT_BF16>, dim3(T), dim3(256), 0, s, h, gamma, eps, out, d);
    return hipGetLastError();
}

}  // namespace moe
