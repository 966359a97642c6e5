// LDS-DMA and synchronisation helpers shared by the matrix-core decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpla_device.h"

namespace tpla {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4] = 7
// meaning no wait, lgkmcnt [11:8] = 0).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// One 16-byte-per-lane LDS DMA: lane i's 16 bytes land at LDS byte `lds_base + 16*i` (the
// wave-uniform base goes through M0).  Issued from asm so that the compiler does not treat every
// later LDS read as possibly aliasing it and wait for it (it would insert vmcnt(0) before the
// first read of the tile being computed and serialise the ring); the instruction has no
// destination register -- its data goes to LDS -- and completion is awaited explicitly with
// s_waitcnt vmcnt before the barrier that publishes the tile.
// Source = 64-bit per-lane address:
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
               : "memory", "m0");
}
// Source = wave-uniform 64-bit base (SGPRs) + per-lane 32-bit byte offset:
__device__ __forceinline__ void dma16_sbase(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Workgroup barrier without a memory fence: LDS-DMA loads stay in flight across it (the caller
// has already waited for the ones it needs), and the empty asm keeps the compiler from moving
// memory accesses over it.
__device__ __forceinline__ void raw_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace tpla
