// Global -> LDS copies (buffer_load ... lds) and the waits around them, shared
// by the grouped GEMMs that stage their operands in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int int32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (base, 32-bit range, default format) as four dwords.
__device__ __forceinline__ int32x4_t make_desc(const void* base, uint32_t nbytes) {
    const uint64_t b = (uint64_t)base;
    int32x4_t r;   // wave-uniform by construction: keep it in SGPRs
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane((int)nbytes);
    r.w = 0x00020000;
    return r;
}

// 16 bytes per lane straight from global memory into LDS: lane l of the wave
// lands at lds_addr + 16*l; an offset the range check rejects writes zeros.
// Issued as inline assembly so that the compiler's wait-count pass does not
// model it: the kernel waits for these copies itself (vmcnt + s_barrier),
// which lets LDS fragment reads of one stage proceed while later stages are
// still being filled.  The LDS address reaches the instruction through m0 as
// an input operand bound to that register ("{m0}"), so the compiler itself
// writes m0 and knows it is in use: no live value of its own can sit there.
__device__ __forceinline__ void dma16(const int32x4_t& desc, uint32_t off, uint32_t lds_addr) {
    // the descriptor and the LDS address are wave-uniform; readfirstlane keeps
    // them in scalar registers even where the compiler cannot prove it
    int32x4_t d;
    d.x = __builtin_amdgcn_readfirstlane(desc.x);
    d.y = __builtin_amdgcn_readfirstlane(desc.y);
    d.z = __builtin_amdgcn_readfirstlane(desc.z);
    d.w = __builtin_amdgcn_readfirstlane(desc.w);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(d), "{m0}"(m0)
                 : "memory");
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(size_t)((__attribute__((address_space(3))) const T*)(p)));
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (N <= 63; loads complete in issue order, so every load older than the
// newest N has landed).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace moe
