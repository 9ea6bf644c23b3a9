// Global -> LDS copies for gfx950 kernels that stage tiles through LDS (the projection GEMM and
// the attention kernel), and the waits that go with them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rglru {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A buffer resource as four dwords (base, stride 0, byte range, format word).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, 0x00020000u};
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Four global -> LDS copies of 1 KB (buffer_load_dwordx4 with the LDS bit: lane l's 16 bytes go
// to LDS byte M0 + 16 l), to consecutive 1 KB destinations from lds_addr; off[j] is the lane's
// byte offset in the buffer for copy j.
//
// Written as inline assembly on purpose: the compiler's wait insertion cannot tell the LDS
// stages of a ring apart, and made the fragment reads after each refill wait for that refill to
// land (a memory round trip per step).  Hidden from it, the copies are waited for only where a
// kernel says so: each wave waits for its own copies (wait_vmcnt) before the barrier that
// publishes a stage, and no other vector-memory instruction of the wave is in flight meanwhile.
// The block has no output register (the data goes to LDS); it saves M0, steps it through the
// 1 KB destinations (one wait state after each write before its use) and restores it.  The
// resource words must not have been written by the VALU in the 5 wait states before (see
// guard_vmem_sgprs).
__device__ __forceinline__ void copy4(const u32x4& rs, uint32_t lds_addr, const int (&off)[4]) {
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %6, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %3, %6, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %4, %6, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(lds_addr), "s"(rs)
        : "memory", "scc");
}

// Five wait states after the resource words were last written (they are often built from
// v_readfirstlane results: a buffer instruction reading SGPRs that the VALU wrote needs 5).
__device__ __forceinline__ void guard_vmem_sgprs(const u32x4& a, const u32x4& b) {
    asm volatile("s_nop 4" ::"s"(a), "s"(b));
}

// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Barrier over LDS accesses (each wave has waited for its own copies before it arrives).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace rglru
