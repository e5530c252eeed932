// Host check of the quantizers' quotient (precision_matmul_amd/csrc/fp8_codec.hpp).
//
// The scaling step of the per-token recipe (DiffSynth-Engine PR #160, "per-token
// scaling for fp8 linear", "Highlights") divides each value by its group's
// scale, s = fl32(amax / 448) (+ a small epsilon for the per-token recipe),
// before the round-to-nearest-even cast to E4M3.  The kernels form that
// correctly rounded float32 quotient from the reciprocal and one FMA
// correction (div_by_scale) instead of a division.  This program runs the
// very same header code on the host, over the quantizers' whole input domain:
//   every positive finite bf16 amax (and 0), both scale forms (plain and
//   + 1e-12f), and every bf16 x of either sign with |x| <= amax,
// and compares it with IEEE float division:
//   - quotients of magnitude >= 2^-12 must be bit-identical;
//   - smaller ones must both lie below 2^-10 in magnitude, i.e. encode to the
//     zero magnitude (the smallest E4M3 subnormal is 2^-9, and 2^-10 itself
//     rounds to zero under ties-to-even); the kernels take the code's sign
//     from x itself (an FMA correction can turn -0 into +0);
//   - the fast path must be chosen exactly when s >= 2^-90.
// Exit status 0 when all hold; the counts are printed either way.
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "fp8_codec.hpp"

using fp8mm::bits_f32;
using fp8mm::f32_bits;

static float bf16_value(uint32_t h) { return bits_f32(h << 16); }

int main() {
  long long pairs = 0, differ_big = 0, differ_code = 0, wrong_switch = 0, slow_groups = 0, near_zero = 0;
  for (int form = 0; form < 2; ++form) {
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, differ_big, differ_code, wrong_switch, slow_groups, near_zero)
    for (int a = 0; a < 0x7F80; ++a) {  // bf16 patterns 0 .. largest finite
      const float amax = bf16_value(uint32_t(a));
      const float s = fp8mm::scale_from_amax(amax, 1e-12f, form == 1);
      const fp8mm::CastScale c = fp8mm::make_cast_scale(s);
      if (c.fast != (s >= 0x1p-90f)) ++wrong_switch;
      if (!c.fast) {
        ++slow_groups;
        continue;
      }
      for (int h = 0; h <= a; ++h) {
        for (uint32_t sign = 0; sign <= 0x8000u; sign += 0x8000u) {
          const float x = bf16_value(uint32_t(h) | sign);
          const float ref = x / s;
          const float got = fp8mm::div_by_scale(x, c.s, c.r);
          ++pairs;
          if (fabsf(ref) >= 0x1p-12f) {
            if (f32_bits(got) != f32_bits(ref)) ++differ_big;
          } else {
            ++near_zero;
            if (!(fabsf(got) < 0x1p-10f)) ++differ_code;
          }
        }
      }
    }
  }
  printf("pairs=%lld near_zero=%lld slow_groups=%lld differ_big=%lld differ_code=%lld wrong_switch=%lld\n", pairs,
         near_zero, slow_groups, differ_big, differ_code, wrong_switch);
  return (pairs > 0 && differ_big == 0 && differ_code == 0 && wrong_switch == 0) ? 0 : 1;
}
