// libmoe_measure.so: measurement helpers, not part of the layer and not linked
// into libmoe.so.  A plain streaming read of a
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
#include <stdarg.h>
#include <stdio.h>

#include "common.h"
#include "devinfo.h"
#include "moe_measure.h"

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

}  // namespace moe

namespace {

int fail(char* err, size_t len, int code, const char* fmt, ...) {
    if (err && len > 0) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(err, len, fmt, ap);
        va_end(ap);
    }
    return code;
}

int launched(char* err, size_t len, const char* what) {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_MEASURE_OK : fail(err, len, MOE_MEASURE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int moe_mfma_ceiling(int32_t iters, float* sink, size_t sink_bytes, uint64_t* clock, int64_t* flops, void* stream,
                     char* err, size_t err_len) {
    if (iters < 1 || iters > (1 << 24))
        return fail(err, err_len, MOE_MEASURE_EINVAL, "iters=%d out of range [1, 2^24]", iters);
    if (!sink) return fail(err, err_len, MOE_MEASURE_EINVAL, "sink is NULL");
    if ((uintptr_t)sink % 16) return fail(err, err_len, MOE_MEASURE_EINVAL, "sink is not 16-byte aligned");
    const int blocks = moe::cu_count();
    if (sink_bytes < (size_t)blocks * 8 * sizeof(float))
        return fail(err, err_len, MOE_MEASURE_EINVAL, "sink_bytes=%zu below %zu", sink_bytes,
                    (size_t)blocks * 8 * sizeof(float));
    if (clock && (uintptr_t)clock % 8) return fail(err, err_len, MOE_MEASURE_EINVAL, "clock is not 8-byte aligned");
    if (flops) *flops = (int64_t)blocks * 8 * iters * 8 * (2LL * 32 * 32 * 16);
    hipLaunchKernelGGL(moe::mfma_ceiling_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters, sink,
                       clock);
    return launched(err, err_len, "mfma ceiling");
}

int moe_read_ceiling(const void* buf, size_t bytes, uint32_t* sink, void* stream, char* err, size_t err_len) {
    if (bytes % 16) return fail(err, err_len, MOE_MEASURE_EINVAL, "bytes=%zu is not a multiple of 16", bytes);
    if (bytes && !buf) return fail(err, err_len, MOE_MEASURE_EINVAL, "buf is NULL");
    if (bytes && (uintptr_t)buf % 16) return fail(err, err_len, MOE_MEASURE_EINVAL, "buf is not 16-byte aligned");
    if (!sink) return fail(err, err_len, MOE_MEASURE_EINVAL, "sink is NULL");
    if ((uintptr_t)sink % 4) return fail(err, err_len, MOE_MEASURE_EINVAL, "sink is not 4-byte aligned");
    if (!bytes) return MOE_MEASURE_OK;
    hipLaunchKernelGGL(moe::read_ceiling_kernel, dim3(moe::cu_count()), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const moe::u32x4_t*>(buf), bytes / 16, sink);
    return launched(err, err_len, "read ceiling");
}

}  // extern "C"
