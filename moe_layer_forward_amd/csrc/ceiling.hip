// Measurement helpers, not part of the layer: a plain streaming read of a
// device buffer (the measured HBM ceiling the decode kernels are compared with
// beside the published 8 TB/s) and a loop of independent bf16 MFMAs (the
// measured matrix-core ceiling beside the published 2.5 PFLOP/s, with the
// shader clock it ran at).
//
// One 256-thread block per CU; each wave reads contiguous 8 KB runs (8
// nontemporal 16-byte loads per lane in flight, consecutive lanes on
// consecutive addresses) and folds everything into one XOR per wave so the
// loads cannot be dropped.  Of the shapes tried on MI355X (grid-strided or
// per-wave runs, 1-8 blocks per CU, 4-16 loads in flight, temporal or not)
// this one read fastest: more streams in flight per CU read slower.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_ceiling_kernel(const u32x4_t* __restrict__ p, size_t n16,
                                                           uint32_t* sink) {
    constexpr int U = 8;
    const int lane = threadIdx.x & 63;
    const size_t nw = (size_t)gridDim.x * (blockDim.x / 64);
    const size_t w = (size_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    const size_t per = 64 * U;                       // 16-byte elements per wave run
    const size_t nruns = n16 / per;
    uint32_t acc = 0;
    for (size_t r = w; r < nruns; r += nw) {
        const u32x4_t* q = p + r * per + lane;
        u32x4_t v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = __builtin_nontemporal_load(q + j * 64);
#pragma unroll
        for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    // the ragged tail past the last whole run
    for (size_t i = nruns * per + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x) {
        const u32x4_t v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, MOE_WAVE);
    if (lane == 0) atomicXor(sink, acc);
}

// Eight waves per CU (two per SIMD), each issuing back-to-back independent
// v_mfma_f32_32x32x16_bf16 on 8 accumulators; one result per wave goes to sink
// so nothing is dropped.  Block 0's wave 0 records its shader cycles
// (s_memtime) and 100 MHz ticks (s_memrealtime) over the loop.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512, 1) void mfma_ceiling_kernel(int iters, float* sink, uint64_t* clk) {
    floatx16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
    bf16x8_t a, b;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        a[v] = (__bf16)(float)((threadIdx.x + v) & 7);
        b[v] = (__bf16)(float)((v - (int)threadIdx.x) & 3);
    }
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[i][v];
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 8 + (threadIdx.x >> 6)] = s;
    if (clk && blockIdx.x == 0 && threadIdx.x == 0) {
        clk[0] = t1 - t0;
        clk[1] = r1 - r0;
    }
}

int mfma_ceiling_blocks() {
    static int n_cu = 0;
    if (n_cu == 0) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (n_cu < 1) n_cu = 256;
    }
    return n_cu;
}

hipError_t launch_mfma_ceiling(int iters, float* sink, uint64_t* clk, hipStream_t s) {
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(mfma_ceiling_blocks()), dim3(512), 0, s, iters, sink, clk);
    return hipGetLastError();
}

hipError_t launch_read_ceiling(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
    static int n_cu = 0;
    if (n_cu == 0) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (n_cu < 1) n_cu = 256;
    }
    hipLaunchKernelGGL(read_ceiling_kernel, dim3(n_cu), dim3(256), 0, s,
                       reinterpret_cast<const u32x4_t*>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace moe
