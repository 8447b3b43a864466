// pow_pair.hpp -- pole powers p^x = exp(lam x) as fp32 pairs (hi + lo).
//
// The carried modal state is decayed once per chunk, s <- p^C s + e.  With
// p^C rounded to fp32 (relative error d up to 2^-24), a token j chunks back
// is weighted by (p^C)^j (1 + d)^j: with chunks of a few tokens, or one per
// decode step, a slow mode (|lam| ~ 1e-3 keeps a token for thousands of
// steps) drifts by j d, a bias that does not average out.  Multiplying by
// hi + lo, lo the remainder of an fp64 exp, makes each decay exact to second
// order; what remains is the unbiased rounding of s itself.
#pragma once
#include <hip/hip_runtime.h>

namespace hyena {

// exp(lam x): .x the fp32 rounding, .y the rest
__device__ __forceinline__ float2 pow_pair(float lam, float x) {
  const double e = exp(static_cast<double>(lam) * static_cast<double>(x));
  const float hi = static_cast<float>(e);
  return make_float2(hi, static_cast<float>(e - static_cast<double>(hi)));
}

// complex mode lam = a + i b (b in radians per token): exp(a x) (cos b x,
// sin b x), each component as hi (returned) + lo (in `lo`)
__device__ __forceinline__ float2 cpow_pair(float a, float b, float x, float2& lo) {
  const double m = exp(static_cast<double>(a) * static_cast<double>(x));
  const double ang = static_cast<double>(b) * static_cast<double>(x);
  const double re = m * cos(ang), im = m * sin(ang);
  const float2 hi = make_float2(static_cast<float>(re), static_cast<float>(im));
  lo = make_float2(static_cast<float>(re - static_cast<double>(hi.x)),
                   static_cast<float>(im - static_cast<double>(hi.y)));
  return hi;
}

// An fp64 value as an fp32 pair: .x its rounding, .y the rest.
__device__ __forceinline__ float2 split_pair(double e) {
  const float hi = static_cast<float>(e);
  return make_float2(hi, static_cast<float>(e - static_cast<double>(hi)));
}

}  // namespace hyena
