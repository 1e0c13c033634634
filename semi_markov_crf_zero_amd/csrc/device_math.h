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
constexpr double kLn2Lo = 2.3190468138462996e-17;  // ln 2 minus its float64 rounding

// exp(y) for float64 y: 2^floor(y*log2e) * 2^frac.  NaN propagates; 0
// below the float64 range, +inf above it (the exponent is clamped to
// [-1100, 1100] and ldexp saturates).  No branch: selects only.
__device__ __forceinline__ double exp_wide(double y) {
  const double z = y * kLog2e;
  const double zc = fmin(fmax(z, -1100.0), 1100.0);  // (a NaN z becomes -1100 here)
  const double n = floor(zc);
  const float f = static_cast<float>(zc - n);  // in [0, 1]
  const float m = __builtin_amdgcn_exp2f(f);   // 2^f in [1, 2]
  const double r = ldexp(static_cast<double>(m), static_cast<int>(n));
  return z != z ? z : r;
}

// log(x) for float64 x >= 0: exponent exactly, mantissa via v_log_f32.
// log(0) = -inf.
__device__ __forceinline__ double log_wide(double x) {
  int e;
  const double m = frexp(x, &e);  // x = m * 2^e, m in [0.5, 1)
  const float l2 = __builtin_amdgcn_logf(static_cast<float>(m));  // log2(m)
  return (static_cast<double>(e) + static_cast<double>(l2)) * kLn2;
}

// log(x) + q ln 2 for float64 x > 0 and an integer-valued q (0 gives -inf,
// +inf and NaN pass through): x = m 2^e with m in [2^-1/2, 2^1/2);
// log m = 2 atanh(s), s = (m - 1) / (m + 1), |s| <= 0.172, by its series
// sum_k s^(2k+1) / (2k+1) through k = 11 (the next term is below 1e-18 of
// the sum); (e + q) ln 2 with a two-part ln 2, so a large q costs no
// accuracy.  About a third of the instructions of the library logarithm.
// The coefficients come from constant memory through scalar registers
// (as literals the compiler would hold them in vector registers).
__constant__ double kAtanhSeries[12] = {1.0,        1.0 / 3.0,  1.0 / 5.0,  1.0 / 7.0,
                                        1.0 / 9.0,  1.0 / 11.0, 1.0 / 13.0, 1.0 / 15.0,
                                        1.0 / 17.0, 1.0 / 19.0, 1.0 / 21.0, 1.0 / 23.0};
__device__ __forceinline__ double log_plus(double x, double q) {
  if (!(x > 0.0 && x < __builtin_huge_val())) return x == 0.0 ? -__builtin_huge_val() : x + x;
  int ex;
  double m = frexp(x, &ex);  // [1/2, 1)
  if (m < 0.70710678118654752440) {
    m *= 2.0;
    ex -= 1;
  }
  const double f = m - 1.0;  // exact
  const double s = f / (2.0 + f);
  const double z = s * s;
  double p = kAtanhSeries[11];
#pragma unroll
  for (int k = 10; k >= 0; --k) p = fma(p, z, kAtanhSeries[k]);
  const double qe = (double)ex + q;
  return fma(qe, kLn2, fma(qe, kLn2Lo, 2.0 * s * p));
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

// exp(s) = ep * 2^n and exp(-s) = em * 2^-n with ep, em in [2^-1/2, 2^1/2]
// and n = rint(s / ln 2): the reduced argument r = s - n ln 2 is formed with
// a two-part ln 2 (so it is accurate to a float64 rounding of r, whatever n),
// then exp(+-r) in float64 from one shared series.  |s| >= 1e9 (no such cumulative score arises
// from finite float32 emissions at the supported sizes) and NaN give NaN.
__device__ __forceinline__ void exp_split(double s, double &ep, double &em, int &n) {
  if (!(fabs(s) < 1e9)) {
    ep = em = __builtin_nan("");
    n = 0;
    return;
  }
  const double k = rint(s * kLog2e);
  const double r = fma(-k, kLn2Lo, fma(-k, kLn2, s));
  n = static_cast<int>(k);
  // exp(+-r) = E(r) +- O(r), the even and odd parts of the exponential
  // series, |r| <= ln2/2: terms through r^14 (the first omitted one is below
  // 1e-17 of the result), in z = r^2 by Horner's rule
  const double z = r * r;
  double e = 1.0 / 87178291200.0;  // 1/14!
  e = fma(e, z, 1.0 / 479001600.0);  // 1/12!
  e = fma(e, z, 1.0 / 3628800.0);    // 1/10!
  e = fma(e, z, 1.0 / 40320.0);      // 1/8!
  e = fma(e, z, 1.0 / 720.0);        // 1/6!
  e = fma(e, z, 1.0 / 24.0);         // 1/4!
  e = fma(e, z, 0.5);                // 1/2!
  e = fma(e, z, 1.0);
  double o = 1.0 / 6227020800.0;     // 1/13!
  o = fma(o, z, 1.0 / 39916800.0);   // 1/11!
  o = fma(o, z, 1.0 / 362880.0);     // 1/9!
  o = fma(o, z, 1.0 / 5040.0);       // 1/7!
  o = fma(o, z, 1.0 / 120.0);        // 1/5!
  o = fma(o, z, 1.0 / 6.0);          // 1/3!
  o = fma(o, z, 1.0);
  o *= r;
  ep = e + o;
  em = e - o;
}

// Row rotation (within each row of 16 lanes) by DPP; lanes whose source would
// be invalid keep their own value, so no register is left undefined.
__device__ __forceinline__ int dpp_ror_i(int v, int by) {
  switch (by) {
    case 8: return __builtin_amdgcn_update_dpp(v, v, 0x128, 0xf, 0xf, false);
    case 4: return __builtin_amdgcn_update_dpp(v, v, 0x124, 0xf, 0xf, false);
    case 2: return __builtin_amdgcn_update_dpp(v, v, 0x122, 0xf, 0xf, false);
    default: return __builtin_amdgcn_update_dpp(v, v, 0x121, 0xf, 0xf, false);
  }
}

// Wave-wide maximum of an int (all 64 lanes call): row rotations by DPP,
// then the four row maxima through scalar reads.
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_ror_i(v, 8));
  v = max(v, dpp_ror_i(v, 4));
  v = max(v, dpp_ror_i(v, 2));
  v = max(v, dpp_ror_i(v, 1));
  const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// One DPP lane permutation of a float64 (both halves moved alike), for the
// aligned-group reductions: 0xB1 quad_perm [1,0,3,2] (lane ^ 1), 0x4E
// quad_perm [2,3,0,1] (lane ^ 2), 0x141 row_half_mirror (the other quad of
// 8), 0x140 row_mirror (the other half of 16).  Every lane has a source.
__device__ __forceinline__ double dpp_f64(double v, int ctrl) {
  const long long b = __builtin_bit_cast(long long, v);
  int lo = (int)(b & 0xffffffffLL), hi = (int)(b >> 32);
  switch (ctrl) {
    case 0xB1:
      lo = __builtin_amdgcn_update_dpp(lo, lo, 0xB1, 0xf, 0xf, false);
      hi = __builtin_amdgcn_update_dpp(hi, hi, 0xB1, 0xf, 0xf, false);
      break;
    case 0x4E:
      lo = __builtin_amdgcn_update_dpp(lo, lo, 0x4E, 0xf, 0xf, false);
      hi = __builtin_amdgcn_update_dpp(hi, hi, 0x4E, 0xf, 0xf, false);
      break;
    case 0x141:
      lo = __builtin_amdgcn_update_dpp(lo, lo, 0x141, 0xf, 0xf, false);
      hi = __builtin_amdgcn_update_dpp(hi, hi, 0x141, 0xf, 0xf, false);
      break;
    default:
      lo = __builtin_amdgcn_update_dpp(lo, lo, 0x140, 0xf, 0xf, false);
      hi = __builtin_amdgcn_update_dpp(hi, hi, 0x140, 0xf, 0xf, false);
      break;
  }
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

// v(l) + v(l ^ S) in every lane l, for S = 8, 16 or 32: a row rotation by 8
// (DPP) within each row of 16, or gfx950's lane swaps between the two rows of
// each row pair (S = 16) or the two halves of the wave (S = 32).  Both lanes
// of a pair add the same two values, so both hold the same sum.
template <int S>
__device__ __forceinline__ double lane_swap_add(double v) {
  static_assert(S == 8 || S == 16 || S == 32, "lane distance 8, 16 or 32");
  const long long b = __builtin_bit_cast(long long, v);
  const unsigned lo = (unsigned)(b & 0xffffffffLL), hi = (unsigned)((unsigned long long)b >> 32);
  unsigned plo, phi;  // the partner lane's halves
  if constexpr (S == 8) {
    plo = (unsigned)__builtin_amdgcn_update_dpp((int)lo, (int)lo, 0x128, 0xf, 0xf, false);
    phi = (unsigned)__builtin_amdgcn_update_dpp((int)hi, (int)hi, 0x128, 0xf, 0xf, false);
    return v + __builtin_bit_cast(double, ((unsigned long long)phi << 32) | plo);
  } else {
    // swap(x, x): the first result holds the lane's own value in the lower
    // row (half) of each pair and the partner's in the upper one, the second
    // the other way round
    if constexpr (S == 16) {
      const auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
      const auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
      const double u = __builtin_bit_cast(double, ((unsigned long long)rh[0] << 32) | rl[0]);
      const double w = __builtin_bit_cast(double, ((unsigned long long)rh[1] << 32) | rl[1]);
      return u + w;
    } else {
      const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
      const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
      const double u = __builtin_bit_cast(double, ((unsigned long long)rh[0] << 32) | rl[0]);
      const double w = __builtin_bit_cast(double, ((unsigned long long)rh[1] << 32) | rl[1]);
      return u + w;
    }
  }
}

__device__ __forceinline__ int dpp_i(int v, int ctrl) {
  switch (ctrl) {
    case 0xB1: return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xf, 0xf, false);
    case 0x4E: return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xf, 0xf, false);
    case 0x141: return __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false);
    default: return __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false);
  }
}

// Maximum (float64) and minimum (int) over aligned groups of ng consecutive
// lanes, ng a power of two up to 64; every lane of a group receives the
// result.  All 64 lanes of the wave must call with the same ng.  Within rows
// of 16 by DPP; across rows (ng = 32, 64) through the four row results read
// into scalars (v_readlane), not an LDS permute.
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __builtin_bit_cast(long long, v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffLL), lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ double group_max(double v, int ng) {
  if (ng >= 2) v = fmax(v, dpp_f64(v, 0xB1));
  if (ng >= 4) v = fmax(v, dpp_f64(v, 0x4E));
  if (ng >= 8) v = fmax(v, dpp_f64(v, 0x141));
  if (ng >= 16) v = fmax(v, dpp_f64(v, 0x140));
  if (ng >= 32) {
    const double r0 = readlane_f64(v, 0), r1 = readlane_f64(v, 16);
    const double r2 = readlane_f64(v, 32), r3 = readlane_f64(v, 48);
    const double lo = fmax(r0, r1), hi = fmax(r2, r3);
    v = ng >= 64 ? fmax(lo, hi) : ((threadIdx.x & 32) ? hi : lo);
  }
  return v;
}

__device__ __forceinline__ int group_min_i(int v, int ng) {
  if (ng >= 2) v = min(v, dpp_i(v, 0xB1));
  if (ng >= 4) v = min(v, dpp_i(v, 0x4E));
  if (ng >= 8) v = min(v, dpp_i(v, 0x141));
  if (ng >= 16) v = min(v, dpp_i(v, 0x140));
  if (ng >= 32) {
    const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    const int lo = min(r0, r1), hi = min(r2, r3);
    v = ng >= 64 ? min(lo, hi) : ((threadIdx.x & 32) ? hi : lo);
  }
  return v;
}

// Workgroup barrier that orders LDS only: vector-memory loads and stores in
// flight stay in flight across it (a plain __syncthreads waits for them).
// Global memory written before it is not guaranteed visible after it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Tie tolerance of the Viterbi decisions: a candidate within
// 1e-11 (|max| + 1) of the maximum ties with it (segmentations that differ
// only in the order of segment lengths inside a run of one label score the
// same in real arithmetic and differ by rounding only).
__device__ __forceinline__ double viterbi_tie_eps(double best) { return 1e-11 * (fabs(best) + 1.0); }

// Wait for every outstanding vector-memory access of the wave (loads and
// stores): s_waitcnt vmcnt(0), other counters untouched.  Placed before a
// loop whose only vector-memory accesses are prefetch loads, it lets the
// compiler wait for each of those by count.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Exponent used for "no value" in the integer maxima below (any real
// exponent of a float64, plus a label reference, is far above it).
constexpr int kNoExp = -(1 << 30);

}  // namespace semicrf
