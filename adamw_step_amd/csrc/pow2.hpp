// The 1Q grid level 2^x for a double x, rounded once to binary32.
//
// TurboAdam package page, 1Q: a block's levels lie on a logarithmic grid
// between its two fp16 log2 endpoints.  Level k is the exact power 2^x,
// x = lo + (hi - lo)(k - 1)/(L - 2) in double, rounded to nearest binary32.
// That is well defined: 2^x is irrational for every non-integer x, so it
// never lies on a midpoint between two binary32 values, and for an integer
// x it is a power of two.  A double exp2 rounded again to binary32 is not
// the same thing: where 2^x lies within the exp2's error of a midpoint,
// the two roundings can part.
//
// pow2_rn32_dd below decides every x through a double-double evaluation of
// 2^x (relative error below 2^-95) and an exact comparison with the
// midpoints around it.  It uses only IEEE double operations (add, multiply,
// divide, fma, scaling by powers of two), so it gives the same result on the
// host and on the device; the library is built without floating-point
// contraction, and so is the host build the tests use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// a + b = s + e exactly, for |a| >= |b| or a = 0.
__host__ __device__ inline void quick_two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  e = b - (s - a);
}

// a + b = s + e exactly, any a and b (Knuth's TwoSum).
__host__ __device__ inline void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// RN32(2^x), decided through a double-double 2^x.
__host__ __device__ inline __attribute__((always_inline)) float pow2_rn32_dd(double x) {
  if (x != x) return (float)x;
  if (x >= 128.0) return __builtin_inff();   // 2^128 and above round to +inf
  if (x <= -150.0) return 0.0f;              // 2^-150 is the midpoint below 2^-149: even 0
  // x = n + r, |r| <= 1/2, both exact.
  const double n = __builtin_rint(x);
  const double r = x - n;
  // t = r ln2 as a double-double; ln2 = LN2_HI + LN2_LO within 2^-107.
  constexpr double LN2_HI = 0x1.62e42fefa39efp-1, LN2_LO = 0x1.abc9e3b39803fp-56;
  double th, tl;
  {
    const double p = r * LN2_HI;
    quick_two_sum(p, __builtin_fma(r, LN2_HI, -p) + r * LN2_LO, th, tl);
  }
  // e^t = sum over j of t^j / j!; |t| <= 0.347, so the terms past j = 24 add
  // less than 2^-110.  The term and the sum are double-doubles.
  double sh = 1.0, sl = 0.0, ph = 1.0, pl = 0.0;
#pragma unroll 1
  for (int j = 1; j <= 24; ++j) {
    double mh, ml;
    {
      const double p = ph * th;
      quick_two_sum(p, __builtin_fma(ph, th, -p) + (ph * tl + pl * th), mh, ml);
    }
    const double dj = (double)j;
    const double qh = mh / dj;
    const double ql = (__builtin_fma(-qh, dj, mh) + ml) / dj;
    quick_two_sum(qh, ql, ph, pl);
    double s, e;
    two_sum(sh, ph, s, e);
    quick_two_sum(s, e + (sl + pl), sh, sl);
  }
  // V = 2^n (sh + sl); both scalings are exact (no double underflow here).
  const int ni = (int)n;
  const double H = __builtin_ldexp(sh, ni), Lw = __builtin_ldexp(sl, ni);
  const float f = (float)H;
  if (f == __builtin_inff()) {
    // H at or above the overflow threshold 2^128 - 2^103 (the midpoint above
    // the largest binary32): V below it rounds to the largest binary32.
    return (H - 0x1.ffffffp127) + Lw < 0.0 ? 0x1.fffffep127f : f;
  }
  // The midpoints on either side of f: half the gap above f and below it
  // (the gap below a normal power of two is half as wide).  f + up and
  // f - dn are exact doubles, and so is H minus either, as H rounds to f.
  uint32_t bits = __builtin_bit_cast(uint32_t, f);
  const int biased = (int)(bits >> 23);        // f > 0; 0 for subnormals
  const double fd = (double)f;
  const double up = __builtin_ldexp(1.0, (biased == 0 ? -126 : biased - 127) - 24);
  const double dn = (biased > 1 && (bits & 0x7FFFFFu) == 0) ? 0.5 * up : up;
  const double above = (H - (fd + up)) + Lw;   // > 0: V beyond the upper midpoint
  const double below = (H - (fd - dn)) + Lw;   // < 0: V beneath the lower midpoint
  const bool odd = bits & 1u;
  if (above > 0.0 || (above == 0.0 && odd)) bits += 1u;
  else if (below < 0.0 || (below == 0.0 && odd)) bits -= 1u;
  return __builtin_bit_cast(float, bits);
}

}  // namespace pa
