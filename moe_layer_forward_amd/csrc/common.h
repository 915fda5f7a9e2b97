// Device helpers shared by the gfx950 kernels of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

namespace moe {

enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_INT4 = 2, DT_INT4_TILED = 3 };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// two fp32 -> packed bf16 (lo in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 (same result as f32_to_bf16 for every non-NaN input)
typedef __bf16 moe_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float moe_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((moe_f32x2_t){lo, hi}, moe_bf16x2_t));
}

// IEEE binary16 -> fp32 (hardware conversion).
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}

template <int ACT>
__device__ __forceinline__ float load_act(const void* p, size_t i) {
    if constexpr (ACT == DT_F32) return reinterpret_cast<const float*>(p)[i];
    else return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

template <int ACT>
__device__ __forceinline__ void store_act(void* p, size_t i, float v) {
    if constexpr (ACT == DT_F32) reinterpret_cast<float*>(p)[i] = v;
    else reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}

// Sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}

// silu(g) = g / (1 + e^-g), as g * rcp(1 + 2^(-g log2 e)) with the hardware
// exp2 and reciprocal (each within about 1 ulp in fp32).  For very negative g
// the exponential overflows to +inf and the result is -0.
__device__ __forceinline__ float silu(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// Blocks are dealt round-robin to the 8 XCDs of an MI355X; remap so that
// consecutive logical ids land on the same XCD (and share its L2).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nblocks) {
    const uint32_t nx = 8;
    uint32_t per = nblocks / nx;          // full rounds
    uint32_t full = per * nx;
    if (b >= full) return b;              // ragged tail keeps its id
    return (b % nx) * per + b / nx;
}

}  // namespace moe
