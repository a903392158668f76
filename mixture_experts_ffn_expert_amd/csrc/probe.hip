// probe.hip -- measurement micro-kernels: the two ceilings that the GEMM and
// combine figures are read against on the chip at hand, next to the
// datasheet peaks.
//
//  * probe_read_kernel: a streaming read of a device buffer, 16-byte
//    non-temporal loads; each workgroup streams one contiguous share of the
//    buffer, eight 4 KiB steps in flight; each thread writes the XOR of
//    every dword it read (so no load is dead, and the result can be checked
//    against the buffer). Bound: HBM, for a buffer well above the
//    256 MB last-level cache.
//  * probe_mfma_kernel: a register-only loop of v_mfma_f32_32x32x16_bf16 on
//    operands taken from a caller buffer (random bf16 values exercise the
//    multipliers as real data does; the chip lowers its clock under the
//    heavier switching). Each wave runs four independent accumulator chains
//    and cycles through four operand pairs, so consecutive MFMAs never wait
//    on each other and their inputs change from one MFMA to the next.
//
// Both launch kProbeBlocks x kProbeThreads threads (4,096 wavefronts: 16 per
// CU on 256 CUs) and write one 32-bit value per thread.
#include <hip/hip_runtime.h>

#include "device_math.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_t* __restrict__ p,
                                                                  size_t n, uint32_t* out) {
  // workgroup b reads the contiguous 16-byte elements [b * per, (b+1) * per)
  // (the last one also the remainder), 4 KiB per workgroup step, U steps in
  // flight: each wavefront touches one page at a time
  constexpr int U = 8;
  const size_t per = n / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = (blockIdx.x + 1 == gridDim.x) ? n : beg + per;
  uint32_t acc = 0;
  size_t i = beg + threadIdx.x;
  for (; i + (U - 1) * kProbeThreads < end; i += U * kProbeThreads) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&p[i + u * kProbeThreads]);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += kProbeThreads) {
    const u32x4_t a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(const bf16x8_t* __restrict__ ops,
                                                                  uint32_t n_ops, int iters,
                                                                  float* out) {
  const uint32_t tid = blockIdx.x * kProbeThreads + threadIdx.x;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = ops[(tid * 4u + (uint32_t)j) % n_ops];
    b[j] = ops[(tid * 4u + (uint32_t)j + 2u * n_ops / 3u) % n_ops];
  }
  f32x16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s = s + acc[j][r];
  out[tid] = s;
}

hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t s) {
  const u32x4_t* p = static_cast<const u32x4_t*>(buf);
  size_t n = bytes / 16;
  void* args[] = {&p, &n, &out};
  return timed_launch(reinterpret_cast<const void*>(probe_read_kernel), dim3(kProbeBlocks),
                      dim3(kProbeThreads), args, s);
}

hipError_t launch_probe_mfma(const uint16_t* ops, uint32_t n_ops, int iters, float* out,
                             hipStream_t s) {
  const bf16x8_t* p = reinterpret_cast<const bf16x8_t*>(ops);
  void* args[] = {&p, &n_ops, &iters, &out};
  return timed_launch(reinterpret_cast<const void*>(probe_mfma_kernel), dim3(kProbeBlocks),
                      dim3(kProbeThreads), args, s);
}

}  // namespace moe
