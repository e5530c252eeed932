// FP8 E4M3 ("e4m3fn") encoding and the exact quotient used by the quantizers.
//
// Encoding: round to nearest, ties to an even mantissa, saturating to +-448,
// sign bit taken from the input (OCP 8-bit floating point specification,
// E4M3; the pages name the format only as "FP8").
//
// Everything here is __host__ __device__ so that a host build can sweep every
// float32 bit pattern through exactly the code the kernels run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

namespace fp8mm {

#define FP8MM_HD __host__ __device__ __forceinline__

FP8MM_HD uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

FP8MM_HD float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

FP8MM_HD float bf16_to_f32(uint16_t h) { return bits_f32(uint32_t(h) << 16); }

// E4M3 code of |v| (bit 7 clear), v a float32 magnitude in any range.
//   |v| >= 2^-6 : keep 3 mantissa bits with round-to-nearest-even on the
//                 float32 bit pattern, rebias the exponent (127 -> 7); any
//                 carry moves into the exponent, which is the next code.
//   |v| <  2^-6 : subnormal codes are m * 2^-9, so the code is |v| * 2^9
//                 rounded to the nearest integer, ties to even (0..8; 8 is
//                 the smallest normal code 0x08, so the two ranges meet).
//   Results above 0x7E (448) saturate to 0x7E; NaN maps to 0x7F.
FP8MM_HD uint32_t e4m3_magnitude_code(uint32_t abs_bits) {
  const uint32_t a = abs_bits;
  const uint32_t rounded = a + 0x7FFFFu + ((a >> 20) & 1u);
  const uint32_t normal = (rounded >> 20) - (120u << 3);
  const float sub_f = __builtin_rintf(bits_f32(a) * 512.0f);
  const uint32_t sub = uint32_t(sub_f);
  uint32_t c = a >= 0x3C800000u ? normal : sub;
  c = c > 0x7Eu ? 0x7Eu : c;
  return a > 0x7F800000u ? 0x7Fu : c;
}

// Full code of a float32 whose sign is given separately (sign_src's sign bit).
FP8MM_HD uint32_t e4m3_encode(float mag_src, float sign_src) {
  const uint32_t a = f32_bits(mag_src) & 0x7FFFFFFFu;
  return e4m3_magnitude_code(a) | ((f32_bits(sign_src) >> 24) & 0x80u);
}

// Scales smaller than this take the plain IEEE division path below.
constexpr float kFastDivMinScale = 8.077935669463161e-28f;  // 2^-90

// fl32(x / s) exactly (IEEE round-to-nearest) from r = fl32(1 / s):
// q0 = x*r is within a few ulp of x/s; each FMA step forms the residual
// x - q*s exactly and corrects q by residual*r (Markstein's correction with a
// correctly rounded reciprocal; the second step delivers the correctly
// rounded quotient).  Valid for s >= 2^-90 and |x/s| <= 2^100: then every
// residual is a normal float, or x/s is below 2^-12, where every candidate
// quotient encodes to the same (signed) zero code.
FP8MM_HD float div_by_scale(float x, float s, float r) {
#pragma clang fp contract(off)
  const float q0 = x * r;
  const float e0 = __builtin_fmaf(-q0, s, x);
  const float q1 = __builtin_fmaf(e0, r, q0);
  const float e1 = __builtin_fmaf(-q1, s, x);
  return __builtin_fmaf(e1, r, q1);
}

// Scale of a group from its amax: fl32(amax / 448) [+ eps], 0 -> 1.
FP8MM_HD float scale_from_amax(float amax, float eps, bool add_eps) {
#pragma clang fp contract(off)
  float s = amax / 448.0f;
  if (add_eps) s = s + eps;
  return s == 0.0f ? 1.0f : s;
}

// Per-group constants of the cast.
struct CastScale {
  float s;
  float r;
  bool fast;
};

FP8MM_HD CastScale make_cast_scale(float s) {
  CastScale c;
  c.s = s;
  c.r = 1.0f / s;
  c.fast = s >= kFastDivMinScale;
  return c;
}

FP8MM_HD uint32_t quantize_one(float x, const CastScale& cs) {
  const float y = cs.fast ? div_by_scale(x, cs.s, cs.r) : x / cs.s;
  return e4m3_encode(y, x);
}

}  // namespace fp8mm
