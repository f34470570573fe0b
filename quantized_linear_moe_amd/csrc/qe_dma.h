// Global -> LDS DMA (global_load_lds) and the explicit waits that go with it.
//
// The copies are issued as inline asm so that the compiler inserts no waits of its
// own; kernels wait with explicit vmcnt counts.  Vector-memory loads retire in issue
// order, so "vmcnt <= n" means every load older than the n most recent ones has landed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qe {

// 16 bytes per lane: lane i writes LDS bytes [lds_base + 16 i, +16)
__device__ inline void dma16(const void* src, uint32_t lds_base) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_base) : "memory");
}

// 4 bytes per lane: lane i writes LDS bytes [lds_base + 4 i, +4)
__device__ inline void dma4(const void* src, uint32_t lds_base) {
    asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_base) : "memory");
}

// LDS byte address of a __shared__ object, as the DMA's M0 operand wants it
template <typename T>
__device__ inline uint32_t lds_addr(T* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)p;
}

}  // namespace qe

#define QE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// vmcnt <= n and every LDS access of this wave completed (lgkmcnt 0)
#define QE_WAIT_VMCNT_LDS(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))
// every LDS access of this wave completed (lgkmcnt 0); vector-memory loads stay in flight
#define QE_WAIT_LDS() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))
// Workgroup barrier without the memory fence of __syncthreads (which also waits for every
// outstanding global load): callers wait for what the barrier must order themselves.
#define QE_WG_BARRIER()                   \
    do {                                  \
        asm volatile("" ::: "memory");    \
        __builtin_amdgcn_s_barrier();     \
        asm volatile("" ::: "memory");    \
    } while (0)
