// silu_table.h -- SiLU of a bf16 gate value by table lookup, bit for bit the
// SiLU of device_math.h (silu_cw: Cody & Waite exp, one correctly rounded
// divide).
//
// The gate-up epilogue applies SiLU to the gate after its narrowing to bf16
// (N1 of the numeric contract of vllm.cpp issue #3094, row statement), so the
// argument is one of 65,536 bit patterns, and for most of them silu_cw has a
// closed form:
//  * |g| < 2^-24 (exponent field below 103): e^-g lies within half an ulp of
//    1, so 1 + e^-g rounds to exactly 2 and silu_cw(g) = g / 2 = g * 0.5
//    (exact, subnormals included);
//  * |g| >= 128 finite (exponent field 134..254): for g > 0, e^-g is below
//    e^-87 and silu_cw uses 0, so the result is g; for g < 0, e^-g is past
//    e^88 and silu_cw uses +inf, so the result is g / inf = -0;
//  * infinities and NaNs: +inf -> +inf, -inf -> -inf / inf = NaN, NaN -> NaN.
// The patterns between (exponent fields 103..133, both signs: 2 x 31 x 128 =
// 7,936) are tabulated. The table is built at compile time by a constexpr
// copy of silu_cw whose every step is the same single IEEE f32 operation as
// on the device; the library's CPU tests compare all 7,936 entries with the
// oracle bit for bit.
//
// Plain C++ (no HIP header), so that a host program can include it.
#pragma once

#include <stdint.h>

namespace moe {

constexpr int kSiluExpLo = 103;                // first tabulated exponent field
constexpr int kSiluExps = 31;                  // exponent fields 103 .. 133
constexpr int kSiluHalf = kSiluExps * 128;     // 3,968 patterns per sign
constexpr int kSiluTabFloats = 8192;           // 7,936 entries, padded to 32 KiB
constexpr int kSiluTabBytes = kSiluTabFloats * 4;

constexpr float silu_f32_of(uint32_t u) { return __builtin_bit_cast(float, u); }

// Round to the nearest integer, ties to even, for |x| < 2^22: in
// x + 1.5 * 2^23 the unit in the last place is 1, so the addition rounds x to
// an integer and the subtraction is exact. The same result as rint.
constexpr float silu_ce_rint(float x) { return (x + 12582912.0f) - 12582912.0f; }

// e^x exactly as exp_cw computes it: n = rint(x / ln 2), r = x - n * ln2_hi -
// n * ln2_lo, the degree-7 Taylor polynomial of e^r in Horner form, then
// scaling by 2^n; +inf above 88, +0 below -87. On [-87, 88] the result is a
// normal number and n lies in [-126, 127], so 2^n is a normal float and the
// scaling is one exact multiplication.
constexpr float silu_ce_exp(float x) {
  if (x != x) return x + x;
  if (x > 88.0f) return __builtin_inff();
  if (x < -87.0f) return 0.0f;
  const float kLog2e = 0x1.715476p+0f;
  const float kLn2Hi = 0x1.63p-1f;
  const float kLn2Lo = -0x1.bd0106p-13f;
  const float n = silu_ce_rint(x * kLog2e);
  const float t = n * kLn2Hi;
  float r = x - t;
  const float t2 = n * kLn2Lo;
  r = r - t2;
  float p = 0x1.a01a02p-13f;
  p = p * r; p = p + 0x1.6c16c2p-10f;
  p = p * r; p = p + 0x1.111112p-7f;
  p = p * r; p = p + 0x1.555556p-5f;
  p = p * r; p = p + 0x1.555556p-3f;
  p = p * r; p = p + 0x1p-1f;
  p = p * r; p = p + 0x1p+0f;
  p = p * r; p = p + 0x1p+0f;
  const int e = (int)n;
  return p * silu_f32_of((uint32_t)(e + 127) << 23);
}

constexpr float silu_ce(float g) {
  const float d = 1.0f + silu_ce_exp(-g);
  return g / d;
}

// Entry i < 7,936 is silu_cw of the bf16 pattern with sign i / 3,968,
// exponent field 103 + (i % 3,968) / 128 and mantissa i % 128; the rest is 0.
struct SiluTable {
  float v[kSiluTabFloats];
};

constexpr SiluTable make_silu_table() {
  SiluTable t{};
  for (int i = 0; i < 2 * kSiluHalf; ++i) {
    const uint32_t s = (uint32_t)i / kSiluHalf, rem = (uint32_t)i % kSiluHalf;
    const uint32_t b = (s << 15) | ((kSiluExpLo + rem / 128) << 7) | (rem % 128);
    t.v[i] = silu_ce(silu_f32_of(b << 16));
  }
  return t;
}

// silu_cw of the bf16 gate with bits b (low 16 bits; the rest zero), with
// tab holding the table above. Branch-free: the lookup index is clamped into
// the table, and the closed forms are g * 0.5 (small), g * 1 (positive
// large, +inf, NaN) and g * 0 (negative large: -0; -inf and NaN: NaN).
constexpr float silu_bf16(uint32_t b, const float* tab) {
  const float g = silu_f32_of(b << 16);
  const uint32_t mag = b & 0x7FFFu;
  const uint32_t a = mag - (uint32_t)(kSiluExpLo * 128);  // wraps below the window
  const uint32_t s = b >> 15;
  const bool inw = a < (uint32_t)kSiluHalf;
  const float t = tab[inw ? a + s * (uint32_t)kSiluHalf : 0u];
  const float f = (mag < (uint32_t)(kSiluExpLo * 128)) ? 0.5f : (s ? 0.0f : 1.0f);
  return inw ? t : g * f;
}

}  // namespace moe
