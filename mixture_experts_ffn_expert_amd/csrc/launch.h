// launch.h -- internal launchers of the MoE expert-path kernels (not part of
// the C ABI; the C ABI validates its arguments and then calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Packed expert weights: 1 KiB blocks of 16 rows x 32 k (layout in gemm.hip).
constexpr uint32_t kPackBlock = 1024;
__host__ __device__ inline int packed_nkb(int kdim) { return (kdim + 31) / 32; }
// Bytes of one expert's packed matrix: gate-up [2I, kdim] (R = 2I) or plain
// [R, kdim].
__host__ __device__ inline size_t packed_expert_bytes(int R, int kdim, bool gateup) {
  const size_t nkb = (size_t)packed_nkb(kdim);
  if (gateup) return (size_t)((R / 2 + 15) / 16) * nkb * 2 * kPackBlock;
  return (size_t)((R + 15) / 16) * nkb * kPackBlock;
}

// pack.hip
hipError_t launch_pack(const uint16_t* w, int E, int R, int kdim, int gateup, uint16_t* out,
                       hipStream_t s);

// route.hip
size_t route_workspace_bytes(int T, int E, int K);
// The library-held grouping scratch of moe_route_noalloc: its size, and its
// device address on the current device (looked up on the first call per
// device and kept; devices 0 .. kRouteScratchDevices - 1).
constexpr size_t kRouteScratchBytes = (size_t)1 << 20;
constexpr int kRouteScratchDevices = 64;
hipError_t route_scratch(void** out);
hipError_t launch_route(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                        int32_t* offsets, int32_t* sorted, void* ws, hipStream_t s);
hipError_t launch_route_scored(const float* logits, int T, int E, int K, int sigmoid,
                               const float* bias, int n_group, int topk_group, int group_top2,
                               int renorm, int32_t* ids, float* w, int32_t* offsets,
                               int32_t* sorted, void* ws, hipStream_t s);

// gemm.hip
hipError_t launch_gateup_silu(const uint16_t* x, int T, int H, const uint16_t* w_gu, int E, int I,
                              const int32_t* sorted, const int32_t* offsets, int K, uint16_t* act,
                              hipStream_t s);
hipError_t launch_down(const uint16_t* act, int P, int I, const uint16_t* w_d, int E, int H,
                       const int32_t* sorted, const int32_t* offsets, const float* pair_w,
                       uint16_t* expert_out, hipStream_t s);
// Arms kernel timing for the next GEMM launch on this host thread (both null:
// disarm).
void set_gemm_timing(hipEvent_t start, hipEvent_t stop);
// Launch through hipExtLaunchKernel with the armed events (then disarmed), or
// plainly when none are armed.
hipError_t timed_launch(const void* kernel, dim3 grid, dim3 block, void** args, hipStream_t s,
                        size_t shm = 0);
hipError_t launch_logits(const uint16_t* x, int T, int H, const uint16_t* w, int N,
                         const float* bias, float* out, hipStream_t s);

// gemm.hip: the decode expert FFN in one launch (gate-up, SiLU-mul, down);
// ws holds fused_ffn_workspace_ints(P, E, grouped) int32 counters, zero
// before the first launch and zero again after each one that reports no error
int fused_ffn_workspace_ints(int P, int E, bool grouped);
hipError_t launch_fused_ffn(const uint16_t* x, int T, int H, const uint16_t* w_gu,
                            const uint16_t* w_d, int E, int I, const int32_t* sorted,
                            const int32_t* offsets, int K, const float* pair_w, uint16_t* act,
                            uint16_t* expert_out, int* ws, hipStream_t s);

// combine.hip; dtype codes: 0 = f32, 1 = bf16
// measurement micro-kernels (probe.hip): kProbeBlocks x kProbeThreads threads,
// one 32-bit output per thread
constexpr int kProbeBlocks = 1024;
constexpr int kProbeThreads = 256;
constexpr int kProbeMfmaChains = 4;  // MFMAs per wave and loop iteration
hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t s);
hipError_t launch_probe_mfma(const uint16_t* ops, uint32_t n_ops, int iters, float* out,
                             hipStream_t s);

hipError_t launch_combine(const void* eo, int eo_bf16, int T, int K, int H, const float* topk_w,
                          float routed_scale, const void* shared, int sh_bf16,
                          const float* gate_logit, void* out, int out_bf16, hipStream_t s);

// keepquant.hip
hipError_t launch_quantize_q8k(const uint16_t* x, int R, int K, int8_t* qs, float* d,
                               int32_t* bsums, hipStream_t s);
hipError_t launch_quantize_q8_0(const uint16_t* x, int R, int K, int8_t* qs, uint16_t* d,
                                hipStream_t s);
// wtype: GGUF type id (8 = Q8_0, 12 = Q4_K, 13 = Q5_K, 14 = Q6_K); xd points at
// f32 Q8_K scales or f16 Q8_0 scales; xs (Q8_K sums of 16) is unused for Q8_0
hipError_t launch_kq_gateup_silu(const int8_t* xq, const void* xd, const int32_t* xs, int T, int H,
                                 const uint8_t* w_gu, int wtype, int E, int I,
                                 const int32_t* sorted, const int32_t* offsets, int K,
                                 uint16_t* act, hipStream_t s);
hipError_t launch_kq_down(const int8_t* aq, const void* ad, const int32_t* as, int P, int I,
                          const uint8_t* w_d, int wtype, int E, int H, const int32_t* sorted,
                          const int32_t* offsets, const float* pair_w, uint16_t* out,
                          hipStream_t s);

}  // namespace moe
