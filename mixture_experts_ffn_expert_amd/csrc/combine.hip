// combine.hip -- weighted top-k combine with the sigmoid-gated shared term.
//
// Operation: vllm.cpp PR #509 ("MoE combine/gate ops -- SharedExpertGate,
// MoeCombine, MoeCombineGate"), What changed: the weighted sum of a token's
// top-k expert rows plus an optional shared term, the shared term optionally
// scaled by sigmoid of the token's gate logit and rounded through bf16. The
// rework commit fixes the arithmetic recipe that makes the result
// bit-reproducible: every output element is computed by one thread, the k
// rows are added in one fixed sequential order, there is a single rounding at
// the store and no multiply-add contraction; the routed_scale commit adds one
// multiply of the finished routed sum before the shared term. f32 and bf16
// arms only (the review comment: f16 is refused by name, at the C ABI).
//
// Design: HBM-bound streaming. One thread owns 8 consecutive h of one token,
// so each of its K expert rows, its shared row and its output are single
// 16-byte accesses (bf16) and a wavefront covers 1 KiB of each row: fully
// coalesced. The sequential k order and the per-element arithmetic are
// unchanged by the vector width. A thread issues the loads of up to 8 of its
// rows before the first add, so 8 loads per thread are in flight.
#include "device_math.h"
#include "launch.h"

namespace moe {

template <typename Tp>
struct Vec8;

template <>
struct Vec8<uint16_t> {  // bf16
  template <bool NT = false>
  static __device__ __forceinline__ void load(const uint16_t* p, float v[8]) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
    const u32x4_t u = NT ? __builtin_nontemporal_load(q) : *q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float v[8]) {
    u32x4_t u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = f32_to_bf16(v[2 * i]) | (f32_to_bf16(v[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4_t*>(p) = u;
  }
};

template <>
struct Vec8<float> {
  template <bool NT = false>
  static __device__ __forceinline__ void load(const float* p, float v[8]) {
    const f32x4_t* q = reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t a = NT ? __builtin_nontemporal_load(q) : q[0];
    const f32x4_t b = NT ? __builtin_nontemporal_load(q + 1) : q[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float v[8]) {
    f32x4_t a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = v[i];
      b[i] = v[4 + i];
    }
    *reinterpret_cast<f32x4_t*>(p) = a;
    *reinterpret_cast<f32x4_t*>(p + 4) = b;
  }
};

template <typename EO, typename SH, typename OUT, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const EO* __restrict__ eo, int K, int H,
                                                      const float* __restrict__ w, float scale,
                                                      const SH* __restrict__ sh,
                                                      const float* __restrict__ gl,
                                                      OUT* __restrict__ out, long long n_vec) {
#pragma clang fp contract(off)
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_vec) return;
  const int hv = H >> 3;
  const long long t = idx / hv;
  const int h0 = (int)(idx - t * hv) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;  // +0
  // The K rows are loaded KB at a time, all KB loads issued before the first
  // add (a row index past K - 1 re-reads row K - 1 and is not added), then
  // summed in k order.
  constexpr int KB = 8;
  const EO* row = eo + (size_t)t * K * H + h0;
  for (int k0 = 0; k0 < K; k0 += KB) {
    float v[KB][8];
#pragma unroll
    for (int j = 0; j < KB; ++j)
      Vec8<EO>::template load<NT>(row + (size_t)min(k0 + j, K - 1) * H, v[j]);
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (k0 + j >= K) break;
      if (w != nullptr) {
        const float wk = w[(size_t)t * K + k0 + j];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = wk * v[j][i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = acc[i] + v[j][i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = acc[i] * scale;
  if (sh != nullptr) {
    float s[8];
    Vec8<SH>::load(sh + (size_t)t * H + h0, s);
    if (gl != nullptr) {
      const float g = sigmoid_cw(gl[t]);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = round_bf16(g * s[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] + s[i];
  }
  Vec8<OUT>::store(out + (size_t)t * H + h0, acc);
}

template <typename EO, typename SH, typename OUT>
static void launch3(const void* eo, int T, int K, int H, const float* w, float scale,
                    const void* sh, const float* gl, void* out, hipStream_t s) {
  const long long n_vec = (long long)T * (H / 8);
  const long long blocks = (n_vec + 255) / 256;
  // expert_out larger than the 256 MiB last-level cache cannot still be
  // there from the down projection that wrote it: its rows are read with the
  // non-temporal hint (8192 tokens x 8 x 4096: 128 -> 111 us); a smaller one
  // is read through the caches
  const EO* eo_p = static_cast<const EO*>(eo);
  const SH* sh_p = static_cast<const SH*>(sh);
  OUT* out_p = static_cast<OUT*>(out);
  void* args[] = {&eo_p, &K, &H, &w, &scale, &sh_p, &gl, &out_p, const_cast<long long*>(&n_vec)};
  const void* kern = ((size_t)T * K * H * sizeof(EO) > ((size_t)256 << 20))
                         ? reinterpret_cast<const void*>(combine_kernel<EO, SH, OUT, true>)
                         : reinterpret_cast<const void*>(combine_kernel<EO, SH, OUT, false>);
  (void)timed_launch(kern, dim3((unsigned)blocks), dim3(256), args, s);
}

template <typename EO, typename SH>
static void launch2(const void* eo, int T, int K, int H, const float* w, float scale,
                    const void* sh, const float* gl, void* out, int out_bf16, hipStream_t s) {
  if (out_bf16)
    launch3<EO, SH, uint16_t>(eo, T, K, H, w, scale, sh, gl, out, s);
  else
    launch3<EO, SH, float>(eo, T, K, H, w, scale, sh, gl, out, s);
}

template <typename EO>
static void launch1(const void* eo, int T, int K, int H, const float* w, float scale,
                    const void* sh, int sh_bf16, const float* gl, void* out, int out_bf16,
                    hipStream_t s) {
  if (sh_bf16)
    launch2<EO, uint16_t>(eo, T, K, H, w, scale, sh, gl, out, out_bf16, s);
  else
    launch2<EO, float>(eo, T, K, H, w, scale, sh, gl, out, out_bf16, s);
}

hipError_t launch_combine(const void* eo, int eo_bf16, int T, int K, int H, const float* topk_w,
                          float routed_scale, const void* shared, int sh_bf16,
                          const float* gate_logit, void* out, int out_bf16, hipStream_t s) {
  if (eo_bf16)
    launch1<uint16_t>(eo, T, K, H, topk_w, routed_scale, shared, sh_bf16, gate_logit, out,
                      out_bf16, s);
  else
    launch1<float>(eo, T, K, H, topk_w, routed_scale, shared, sh_bf16, gate_logit, out, out_bf16,
                   s);
  return hipGetLastError();
}

}  // namespace moe
