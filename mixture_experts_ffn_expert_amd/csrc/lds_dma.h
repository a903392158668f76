// lds_dma.h -- direct-to-LDS buffer loads (gfx950): a 64-lane
// buffer_load_dwordx4 ... lds writes lane l's 16 bytes at M0 + 16 l, so one
// instruction fills 1 KiB of LDS without passing through registers. Waits
// are the caller's: the load counts in vmcnt until its data is in LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ i32x4_t raw_rsrc(const void* base, uint32_t bytes) {
  const unsigned long long b = (unsigned long long)base;
  i32x4_t r = {(int)(uint32_t)b, (int)(uint32_t)(b >> 32), (int)bytes, 0x00020000};
  return r;
}

__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t m0, uint32_t voff, uint32_t soff) {
  // M0 is an input operand: the compiler places the LDS address there itself
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0)
               : "memory");
}

// Wait until at most N of this wave's vector loads are in flight and all its
// LDS reads are done, then barrier. Memory-clobbering, so no LDS access
// moves across it.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

}  // namespace moe
