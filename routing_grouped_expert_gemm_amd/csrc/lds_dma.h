// LDS-DMA primitives of the GEMM kernels (gfx950): global_load_lds with the LDS address in M0,
// vmcnt waits and a barrier that does not drain the DMA stages still in flight.
#pragma once
#include "device_common.h"

namespace mok {

// s_waitcnt with only the vector-memory counter constrained: vmcnt <= n (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
MOK_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS-DMA: every lane copies 16 (or 4) bytes from sbase + voff (sbase uniform) to LDS address
// lds + lane * 16 (or * 4), lds uniform. Issued as inline asm so that the compiler does not
// track these writes: its own bookkeeping would make the first read after a loop back-edge
// wait for every DMA in flight. The K loop orders them with explicit vmcnt waits instead.
// M0 carries the LDS address; nothing else in these kernels uses M0.
MOK_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// L2C (ring data: written by another workgroup during this kernel): the load bypasses the
// CU's L1 (sc0) and reads the XCD's L2, where the producer's stores landed.
template <bool L2C = false>
MOK_DEV void dma_b128(const void* sbase, uint32_t voff, uint32_t lds) {
  if constexpr (L2C)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 sc0"
                 :: "s"(lds), "v"(voff), "s"(sbase) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds), "v"(voff), "s"(sbase) : "memory");
}
template <bool L2C = false>
MOK_DEV void dma_b32(const void* sbase, uint32_t voff, uint32_t lds) {
  if constexpr (L2C)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2 sc0"
                 :: "s"(lds), "v"(voff), "s"(sbase) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(lds), "v"(voff), "s"(sbase) : "memory");
}

// Workgroup barrier for the LDS-DMA K loop. __syncthreads() would also wait for every
// outstanding LDS-DMA (its fence covers LDS, and DMA writes count as LDS writes), draining the
// stages still in flight; the K loop instead waits for exactly the step it needs (wait_vmcnt)
// and then only synchronises. The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
MOK_DEV void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace mok
