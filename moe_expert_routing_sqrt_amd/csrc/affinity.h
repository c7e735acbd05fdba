// The fixed fp32 operation sequence for the gate affinity
// s = sqrt(softplus(l)) (mastering-deepseek-v4 "MoE + Expert-Parallel Overlap
// (Exp08)", Implemented: Sqrt(Softplus) affinities), shared by the top-k and
// the hash routers.  Include only from files compiled with contraction off,
// correctly rounded divide and sqrt, and fp32 denormals kept:
//   softplus(l) = max(l,0) + log1p(exp(-|l|))
//   exp(-a): Cody & Waite 1980 range reduction (ln2 split in two), degree-7
//            Taylor polynomial in Horner form, ldexp; 0 for a > 87
//   log1p(u): Goldberg 1991 Thm 4 (w = 1+u; u if w == 1 else
//            log(w)*u/(w-1)); log(w) by frexp into [sqrt(1/2), sqrt(2)) and
//            2*atanh((m-1)/(m+1)) to the f^11 term, plus e*ln2 in two parts
#pragma once

#include <hip/hip_runtime.h>

namespace moe {
namespace aff {

inline constexpr float kInvLn2 = 1.44269502162933349609375f;
inline constexpr float kLn2Hi = 0.693359375f;
inline constexpr float kLn2Lo = -0.000212194441701285541057586669922f;
inline constexpr float kSqrtHalf = 0.707106769084930419921875f;
inline constexpr float kExpCutoff = 87.0f;

__device__ inline float exp_neg_spec(float a) {
  const float ac = a > kExpCutoff ? 0.0f : a;
  const float n = __builtin_rintf(ac * kInvLn2);
  const float r = (n * kLn2Hi - ac) + n * kLn2Lo;
  float p = 1.0f / 5040.0f;
  p = p * r + 1.0f / 720.0f;
  p = p * r + 1.0f / 120.0f;
  p = p * r + 1.0f / 24.0f;
  p = p * r + 1.0f / 6.0f;
  p = p * r + 1.0f / 2.0f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  const float res = ldexpf(p, -static_cast<int>(n));
  return a > kExpCutoff ? 0.0f : res;
}

__device__ inline float log1p_spec(float u) {
  const float w = u + 1.0f;
  if (w == 1.0f) return u;
  int e;
  float m = frexpf(w, &e);
  if (m < kSqrtHalf) {
    m = m * 2.0f;
    e = e - 1;
  }
  const float f = (m - 1.0f) / (m + 1.0f);
  const float f2 = f * f;
  float q = 2.0f / 11.0f;
  q = q * f2 + 2.0f / 9.0f;
  q = q * f2 + 2.0f / 7.0f;
  q = q * f2 + 2.0f / 5.0f;
  q = q * f2 + 2.0f / 3.0f;
  q = q * f2 + 2.0f;
  const float logm = f * q;
  const float ef = static_cast<float>(e);
  const float logw = ef * kLn2Hi + (logm + ef * kLn2Lo);
  return (logw * u) / (w - 1.0f);
}

__device__ inline float affinity_spec(float l) {
  const float pos = l > 0.0f ? l : 0.0f;
  const float sp = pos + log1p_spec(exp_neg_spec(fabsf(l)));
  return sqrtf(sp);
}

}  // namespace aff
}  // namespace moe
