// device_math.h -- small numeric helpers for the gfx950 semi-CRF kernels.
//
// The streaming messages are kept in exp space as float64 values relative
// to a per-label log reference (see chain.hip).  These helpers convert
// between log values held in float64 and exp-space float64 values using the
// hardware base-2 transcendentals (v_exp_f32 / v_log_f32) on the fractional
// part and an exact power-of-two scaling (v_ldexp_f64) for the integer part,
// so the result has the full float64 exponent range and float32-level
// relative precision in the mantissa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace semicrf {

constexpr double kLog2e = 1.4426950408889634074;
constexpr double kLn2 = 0.69314718055994530942;

// exp(y) for float64 y: 2^floor(y*log2e) * 2^frac.  NaN propagates; 0
// below the float64 range, +inf above it.
__device__ __forceinline__ double exp_wide(double y) {
  const double z = y * kLog2e;
  if (z != z) return z;
  if (z <= -1075.0) return 0.0;
  if (z >= 1024.0) return __builtin_huge_val();
  const double n = floor(z);
  const float f = static_cast<float>(z - n);  // in [0, 1]
  const float m = __builtin_amdgcn_exp2f(f);  // 2^f in [1, 2]
  return ldexp(static_cast<double>(m), static_cast<int>(n));
}

// log(x) for float64 x >= 0: exponent exactly, mantissa via v_log_f32.
// log(0) = -inf.
__device__ __forceinline__ double log_wide(double x) {
  int e;
  const double m = frexp(x, &e);  // x = m * 2^e, m in [0.5, 1)
  const float l2 = __builtin_amdgcn_logf(static_cast<float>(m));  // log2(m)
  return (static_cast<double>(e) + static_cast<double>(l2)) * kLn2;
}

// exp(y) in float32 for y <= ~88 (probabilities and bounded ratios).
__device__ __forceinline__ float exp_f32(double y) {
  return __builtin_amdgcn_exp2f(static_cast<float>(y * kLog2e));
}

// Integer log2 magnitude of a positive float64 (frexp exponent), used to
// decide exact power-of-two rebasing.
__device__ __forceinline__ int exponent_of(double x) {
  int e;
  (void)frexp(x, &e);
  return e;
}

}  // namespace semicrf
