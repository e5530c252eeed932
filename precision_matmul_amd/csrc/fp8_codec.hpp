// Scale and exact quotient of the FP8 E4M3 ("e4m3fn") quantizers.
//
// A group's scale is s = fl32(amax / 448) (+ eps for the per-token recipe),
// and each value becomes the E4M3 code of the correctly rounded float32
// quotient fl32(x / s).  (The encoding itself, round to nearest even with
// saturation to +-448 per the OCP 8-bit floating point specification, is done
// by the hardware conversion in the kernels.)
//
// Everything here is __host__ __device__ so that a host build can check the
// quotient against IEEE division on any float32 input.
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

// Scales smaller than this take the plain IEEE division path below.
constexpr float kFastDivMinScale = 8.077935669463161e-28f;  // 2^-90

// fl32(x / s) from r = fl32(1 / s): q0 = x*r is within one ulp of x/s; the
// FMA forms the residual x - q0*s exactly and corrects q0 by residual*r
// (Markstein's theorem: with a correctly rounded reciprocal one correction
// gives the correctly rounded quotient).  Valid for s >= 2^-90 and quotients
// of at least 2^-12 in magnitude; smaller quotients (where a subnormal
// residual can leave the last bit off) all encode to the zero magnitude, and
// the kernels take the code's sign from x.  tests/host/div_by_scale_check.cpp
// builds this header for the host and checks it over the whole input domain
// of the quantizers: every bf16 x with |x| <= amax, against s = fl32(amax /
// 448) and s = fl32(fl32(amax / 448) + 1e-12) for every positive finite bf16
// amax (2.1e9 pairs): no quotient of magnitude >= 2^-12 differs from IEEE
// division, every smaller one stays below 2^-10, and the fast path is taken
// exactly when s >= 2^-90.
FP8MM_HD float div_by_scale(float x, float s, float r) {
#pragma clang fp contract(off)
  const float q0 = x * r;
  const float e0 = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(e0, r, q0);
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

}  // namespace fp8mm
