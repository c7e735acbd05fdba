// The gate affinity s = sqrt(softplus(l)) (mastering-deepseek-v4 "MoE +
// Expert-Parallel Overlap (Exp08)", Implemented: Sqrt(Softplus) affinities),
// shared by the top-k router, the hash router and the gate backward.
//
// s = fp32(sqrt(sp)) with sp = softplus(l) from a fixed sequence of fp64
// operations and one rounding to fp32 at the end.  fp64 is accurate far below
// fp32's steps, so s is the correctly rounded affinity except within ~2^-50 of
// an fp32 rounding boundary, and non-decreasing in l like the exact function
// (routing ranks experts by it, so a larger logit never scores lower).  Include
// only from files compiled with contraction off (each operation rounded on
// its own; the fp64 divide and sqrt are correctly rounded).
//   |l| < 2^-14 : sp = ln2 + (l/2 + l*l/8)   (Taylor series at 0; monotone
//                 step by step; the dropped terms are < 2^-63 of sp)
//   otherwise   : sp = max(l,0) + log1p(exp(-|l|)), exp(-a) = 0 for a > 300
//   exp(-a): Cody & Waite 1980 range reduction (ln2 split into a 40-bit head
//            and a tail), degree-13 Taylor polynomial in Horner form, ldexp
//   log1p(u): Goldberg 1991 Thm 4 (w = 1+u; u if w == 1 else
//            log(w)*u/(w-1)); log(w) by frexp into [sqrt(1/2), sqrt(2)) and
//            2*atanh((m-1)/(m+1)) to the f^21 term, plus e*ln2 in two parts
#pragma once

#include <hip/hip_runtime.h>

namespace moe {
namespace aff {

inline constexpr double kInvLn2 = 0x1.71547652b82fep+0;   // 1/ln2
inline constexpr double kLn2Hi = 0x1.62e42fefa4000p-1;    // ln2, 40 significant bits
inline constexpr double kLn2Lo = -0x1.8432a1b0e2634p-43;  // ln2 - kLn2Hi
inline constexpr double kLn2 = 0x1.62e42fefa39efp-1;      // ln2
inline constexpr double kSqrtHalf = 0x1.6a09e667f3bcdp-1; // sqrt(1/2)
inline constexpr double kSmall = 0x1p-14;
inline constexpr double kExpCutoff = 300.0;

// e^-a for 0 <= a <= kExpCutoff
__device__ inline double exp_neg64(double a) {
  const double n = __builtin_rint(a * kInvLn2);
  const double r = (n * kLn2Hi - a) + n * kLn2Lo;
  // 1/i!, i = 13 .. 0
  double p = 0x1.6124613a86d09p-33;
  p = p * r + 0x1.1eed8eff8d898p-29;
  p = p * r + 0x1.ae64567f544e4p-26;
  p = p * r + 0x1.27e4fb7789f5cp-22;
  p = p * r + 0x1.71de3a556c734p-19;
  p = p * r + 0x1.a01a01a01a01ap-16;
  p = p * r + 0x1.a01a01a01a01ap-13;
  p = p * r + 0x1.6c16c16c16c17p-10;
  p = p * r + 0x1.1111111111111p-7;
  p = p * r + 0x1.5555555555555p-5;
  p = p * r + 0x1.5555555555555p-3;
  p = p * r + 0.5;
  p = p * r + 1.0;
  p = p * r + 1.0;
  return __builtin_ldexp(p, -static_cast<int>(n));
}

// log1p(u) for 0 <= u <= 1
__device__ inline double log1p_unit64(double u) {
  const double w = u + 1.0;
  if (w == 1.0) return u;
  int e;
  double m = __builtin_frexp(w, &e);
  if (m < kSqrtHalf) {
    m = m * 2.0;
    e = e - 1;
  }
  const double f = (m - 1.0) / (m + 1.0);
  const double f2 = f * f;
  // 2/(2j+1), j = 10 .. 0
  double q = 0x1.8618618618618p-4;
  q = q * f2 + 0x1.af286bca1af28p-4;
  q = q * f2 + 0x1.e1e1e1e1e1e1ep-4;
  q = q * f2 + 0x1.1111111111111p-3;
  q = q * f2 + 0x1.3b13b13b13b14p-3;
  q = q * f2 + 0x1.745d1745d1746p-3;
  q = q * f2 + 0x1.c71c71c71c71cp-3;
  q = q * f2 + 0x1.2492492492492p-2;
  q = q * f2 + 0x1.999999999999ap-2;
  q = q * f2 + 0x1.5555555555555p-1;
  q = q * f2 + 2.0;
  const double ed = static_cast<double>(e);
  const double logw = ed * kLn2Hi + (f * q + ed * kLn2Lo);
  return (logw * u) / (w - 1.0);
}

__device__ inline double softplus64(float lf) {
  const double l = static_cast<double>(lf);
  const double a = __builtin_fabs(l);
  if (a < kSmall) return kLn2 + (l * 0.5 + (l * l) * 0.125);
  const double pos = l > 0.0 ? l : 0.0;
  if (a > kExpCutoff) return pos;
  return pos + log1p_unit64(exp_neg64(a));
}

__device__ inline float affinity_spec(float l) {
  return static_cast<float>(__builtin_sqrt(softplus64(l)));
}

}  // namespace aff
}  // namespace moe
