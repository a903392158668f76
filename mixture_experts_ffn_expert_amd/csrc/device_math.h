// device_math.h -- gfx950 device helpers of the MoE expert path: bf16
// storage, a bit-reproducible f32 exp, sigmoid, SiLU, vector types.
//
// Everything here is written for IEEE f32 with each operation rounded on its
// own: the library is built with -ffp-contract=off and the functions below
// also switch contraction off locally, so no multiply-add is ever fused.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 bits -> f32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// f32 -> bf16 bits: the hardware conversion the compiler emits for a float ->
// __bf16 cast on gfx950 (v_cvt_pk_bf16_f32). On every one of the 2^32 f32
// patterns it rounds to nearest even, keeps subnormals, takes values past the
// largest bf16 to infinity, and turns a NaN into sign and top payload bits
// with the quiet bit set, i.e. (bits >> 16) | 0x0040.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// f32 rounded to bf16 and read back as f32 (one narrowing).
__device__ __forceinline__ float round_bf16(float f) {
  return bf16_to_f32(f32_to_bf16(f));
}

// Two f32 values converted to bf16 (as f32_to_bf16) by one
// v_cvt_pk_bf16_f32: lo in the low half, hi in the high half.
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b16x2_t));
}

// e^x in f32: Cody & Waite argument reduction (n = rint(x / ln2),
// r = x - n*ln2 with ln2 split into a 9-bit head, so n*head is exact, and an
// f32 tail) followed by the degree-7 Taylor polynomial of e^r in Horner form
// and a final scaling by 2^n. Each step is a single IEEE f32 operation, so
// the result is reproducible on any IEEE machine. Inputs above 88 give +inf,
// below -87 give +0 (every other result is a normal number), NaN gives NaN.
__device__ __forceinline__ float exp_cw(float x) {
#pragma clang fp contract(off)
  if (x != x) return x + x;                 // NaN stays NaN
  if (x > 88.0f) return __builtin_inff();
  if (x < -87.0f) return 0.0f;
  const float kLog2e = 0x1.715476p+0f;      // f32(1/ln 2)
  const float kLn2Hi = 0x1.63p-1f;          // ln 2 to 9 bits: 0.693359375
  const float kLn2Lo = -0x1.bd0106p-13f;    // f32(ln 2 - head)
  float n = __builtin_rintf(x * kLog2e);
  float t = n * kLn2Hi;
  float r = x - t;
  float t2 = n * kLn2Lo;
  r = r - t2;
  // 1/k! rounded to f32, k = 7 .. 0
  float p = 0x1.a01a02p-13f;
  p = p * r; p = p + 0x1.6c16c2p-10f;
  p = p * r; p = p + 0x1.111112p-7f;
  p = p * r; p = p + 0x1.555556p-5f;
  p = p * r; p = p + 0x1.555556p-3f;
  p = p * r; p = p + 0x1p-1f;
  p = p * r; p = p + 0x1p+0f;
  p = p * r; p = p + 0x1p+0f;
  return __builtin_ldexpf(p, (int)n);
}

// sigmoid(z) = 1 / (1 + e^-z), correctly rounded f32 divide.
__device__ __forceinline__ float sigmoid_cw(float z) {
#pragma clang fp contract(off)
  float d = 1.0f + exp_cw(-z);
  return __fdiv_rn(1.0f, d);
}

// SiLU(g) = g / (1 + e^-g), correctly rounded f32 divide.
__device__ __forceinline__ float silu_cw(float g) {
#pragma clang fp contract(off)
  float d = 1.0f + exp_cw(-g);
  return __fdiv_rn(g, d);
}

}  // namespace moe
