// Buffer resources, direct global->LDS DMA and explicit wait helpers for gfx950
// kernels that stage tiles through LDS with their own vmcnt bookkeeping.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace moe {

// A workgroup-uniform pointer, pinned to scalar registers.  Buffer resources
// must live in SGPRs; without this the compiler may keep a base it cannot
// prove uniform in VGPRs and wrap every load in a read-first-lane loop.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

// Raw buffer resource: accesses at byte offsets >= num_records return zero
// without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

constexpr uint32_t kOob = 0x80000000u;   // an offset beyond every resource's range

// 16 bytes per lane from global memory straight into LDS (M0 + 16 * lane);
// no VGPR is written, so nothing is left in flight in registers.  Completion
// is tracked with vmcnt by the caller; the compiler does not count these (the
// compiler's own LDS-DMA builtin makes it wait for every DMA in flight before
// the next LDS read, which would drain the prefetch ring).
// M0 is reserved to the compiler, so the helper saves it, loads the LDS
// address, waits the one wait state gfx9 needs between an M0 write and an
// LDS DMA that reads it (s_nop 0), issues the DMA (which takes M0 at issue)
// and restores M0: whatever the compiler keeps in M0 survives the call.
#define MOE_DMA16(HINT)                                                           \
    do {                                                                         \
        uint32_t saved_m0;                                                       \
        asm volatile("s_mov_b32 %0, m0\n\t"                                       \
                     "s_mov_b32 m0, %3\n\t"                                       \
                     "s_nop 0\n\t"                                                \
                     "buffer_load_dwordx4 %1, %2, 0 offen " HINT "lds\n\t"         \
                     "s_mov_b32 m0, %0"                                           \
                     : "=&s"(saved_m0)                                            \
                     : "v"(voff), "s"(r), "s"(lds)                                \
                     : "memory");                                                 \
    } while (0)

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
    MOE_DMA16("");
}

// As dma16, with the nontemporal hint: the lines are not kept in the
// last-level cache, so streaming a large input once neither evicts nor
// writes back other kernels' lines on the way.
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
    MOE_DMA16("nt ");
}
#undef MOE_DMA16

// s_waitcnt vmcnt(n) (gfx9 encoding; lgkmcnt and expcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace moe
