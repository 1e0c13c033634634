// chain256.hip -- streaming semi-CRF sweep for 64 < C <= 256 labels, K <= 64
// (speech scale: C = 256, K = 64), one chain per compute unit.
//
// Same recurrences, exp-space entries with integer references, checkpoint
// records and row outputs as chain.hip (see its header for the equations
// and the power-of-two arithmetic; method: "Streaming Structured Inference
// with Flash-SemiCRF", abstract and technical summary sections 2.A-2.C).
// What limits a step at these shapes is operand traffic: the ring (K x C
// entries), the weights exp(dur) (K x C) and exp(trans) (C x C = 65536) are
// all read every step, and the contraction needs every label's input in
// every output's thread.  Together they exceed the compute unit's register
// file and LDS in float64, so this engine keeps them in float32:
//   * 8 waves x 64 lanes; K-sum role: label c = 32w + i is held by the lane
//     pair (2i, 2i+1) of wave w; lane q of the pair holds durations
//     k = 32q + 1 .. 32q + 32 of that label in 32 float32 ring registers (a
//     circular buffer whose head moves back by one register per step, in
//     blocks of 32 steps instantiated for their place so every ring index
//     is a compile-time constant, as in chain64.hip).  The ring's shift by
//     one position is one DPP move (lane 2i's oldest entry to lane 2i+1).
//     exp(dur) (float32) of the lane's durations is read from LDS with
//     immediate offsets from one base address.
//   * contraction role: wave w sums over its own 32 labels (inputs c'), and
//     lane l of the wave produces the partial sums of outputs 4l .. 4l+3
//     with 32 x 4 weights exp(trans) in float32, 24 x 4 of them in
//     registers and the rest read from LDS.  The inputs a[c'] =
//     x[c'] 2^(E[c'] - Bw), scaled to the wave's largest exponent Bw, are
//     the wave's own values: they reach every lane through scalar registers
//     (v_readlane), so no input travels through LDS.  Each wave publishes
//     its 256 partial sums and Bw; one barrier per step; each label's lane
//     pair reads the 8 partials of its label and combines them in float64
//     at the step scale B = max Bw (exact power-of-two scalings):
//     exp(m) = d 2^B.
//   * float32: the ring entries (relative to the label's integer reference,
//     rebased by an exact power of two when a new entry leaves 2^+-32), the
//     K-sum's products and partial sums, the contraction's products and
//     sums, exp(dur) and exp(trans).  float64: the references and scales
//     (integers), the combination of the partial sums, the rows x 2^E and
//     d 2^B, the score splits and every output.  The rounding this adds is
//     a relative error of order 1e-7 per step that does not compound
//     through the recursion (each step's messages are averages of the
//     previous ones); measured on the speech workload (T = 4096) it moves
//     log Z by 2e-10 relative and the segment-start posteriors by 8e-8.  A
//     float32 ring bounds the parameters: an older entry exceeds the newest
//     by at most exp(-dur[k-1][c] - trans[c][c]), and a K-sum of 64 entries
//     up to 2^32 times that, times exp(dur), must stay below 2^127, so
//     2 |dur| + |trans| must stay below about 60 nats.
//   * the parallel-in-time verification accepts a chunk start whose
//     direction matches its predecessor's end to float32 rounding (pit.hip).
//   * rows: lane 0 of a pair stores o (alpha / v), lane 1 stores m (u /
//     beta) of each step; the scores of the next positions are loaded two
//     steps ahead into registers and split there.
#include <stdio.h>
#include <stdlib.h>

#include <utility>

#include "device_math.h"
#include "internal.h"
#include "pitcheck.h"

namespace semicrf {

namespace {

constexpr int kW = 8;            // waves
constexpr int kNT = 64 * kW;     // threads
constexpr int kA = 32;           // durations per lane
constexpr int kDmax = 2 * kA;    // durations per label (two lanes)
constexpr int kLab = 256;        // labels, padded with zero weights
constexpr int kLw = kLab / kW;   // labels (contraction inputs) per wave
constexpr int kR = 4;            // contraction outputs per lane
constexpr int kWr = 24;          // inputs whose weights a lane holds in registers
constexpr int kWl = kLw - kWr;   // inputs whose weights it reads from LDS
constexpr int kPq = 2;           // score prefetch distance (steps); divides kA
constexpr int kRebase = 32;      // rebase bound of the float32 ring, log2 units
constexpr int kTabN = 32;

// Constants of the exponential split and of the logarithm (read from LDS
// where they are used; as literals the compiler keeps them in registers
// across the step loop).
__constant__ double kTab256[kTabN] = {
    1.4426950408889634074,   // 0: log2 e
    0.69314718055994530942,  // 1: ln 2
    2.3190468138462996e-17,  // 2: ln 2 minus its float64 rounding
    1.0 / 87178291200.0,     // 3: 1/14!
    1.0 / 479001600.0,       // 4: 1/12!
    1.0 / 3628800.0,         // 5: 1/10!
    1.0 / 40320.0,           // 6: 1/8!
    1.0 / 720.0,             // 7: 1/6!
    1.0 / 24.0,              // 8: 1/4!
    1.0 / 6227020800.0,      // 9: 1/13!
    1.0 / 39916800.0,        // 10: 1/11!
    1.0 / 362880.0,          // 11: 1/9!
    1.0 / 5040.0,            // 12: 1/7!
    1.0 / 120.0,             // 13: 1/5!
    1.0 / 6.0,               // 14: 1/3!
    1e9,                     // 15: bound of the split's argument
    // 16..27: 1/(2k+1), k = 0..11 (the series of atanh)
    1.0, 1.0 / 3.0, 1.0 / 5.0, 1.0 / 7.0, 1.0 / 9.0, 1.0 / 11.0, 1.0 / 13.0, 1.0 / 15.0,
    1.0 / 17.0, 1.0 / 19.0, 1.0 / 21.0, 1.0 / 23.0,
    0.70710678118654752440,  // 28: sqrt(1/2)
    0.0, 0.0, 0.0};

struct S256 {
  float *dr;     // [kDmax][kLab]: exp(dur[k-1][c]) (0 past K and C)
  float *wl;     // [kW][kWl][64][kR]: exp(trans) of the inputs 32w + kWr + i
  float *part;   // [2][kW][kLab]: partial sums of the contraction, by step parity
  int *bw;       // [2][kW]: the waves' scales
  double *tab;   // [kTabN]
  double *zb;    // [kLab]: log Z inputs (the chain's last step)
  int *zbw;      // [kW]
};

constexpr size_t kLdsBytes = (size_t)kDmax * kLab * 4 + (size_t)kW * kWl * 64 * kR * 4 +
                             (size_t)2 * kW * kLab * 4 +
                             (size_t)2 * kW * 4 + (size_t)kTabN * 8 + (size_t)kLab * 8 +
                             (size_t)kW * 4;

__device__ __forceinline__ S256 carve256(unsigned char *base) {
  S256 m;
  size_t off = 0;
  m.dr = reinterpret_cast<float *>(base + off); off += (size_t)kDmax * kLab * 4;
  m.wl = reinterpret_cast<float *>(base + off); off += (size_t)kW * kWl * 64 * kR * 4;
  m.part = reinterpret_cast<float *>(base + off); off += (size_t)2 * kW * kLab * 4;
  m.tab = reinterpret_cast<double *>(base + off); off += (size_t)kTabN * 8;
  m.zb = reinterpret_cast<double *>(base + off); off += (size_t)kLab * 8;
  m.bw = reinterpret_cast<int *>(base + off); off += (size_t)2 * kW * 4;
  m.zbw = reinterpret_cast<int *>(base + off);
  return m;
}

__device__ __forceinline__ int pslot(int pos, int K) {
  const int s = pos % K;
  return s < 0 ? s + K : s;
}

// The table, through an offset the compiler cannot see (0): its loads stay
// where they are used instead of being hoisted out of the step loop.
__device__ __forceinline__ const double *table_here(const double *tab) {
  int z = 0;
  asm volatile("" : "+s"(z));
  return tab + z;
}

// exp(s) = ep 2^n and exp(-s) = em 2^-n, ep, em in [2^-1/2, 2^1/2]: the same
// reduction and series as exp_split (device_math.h), term for term, with
// the constants read from the table.
__device__ __forceinline__ void exp_split_t(double s, double &ep, double &em, int &n,
                                            const double *tab0) {
  const double *tab = table_here(tab0);
  if (!(fabs(s) < tab[15])) {
    ep = em = __builtin_nan("");
    n = 0;
    return;
  }
  const double k = rint(s * tab[0]);
  const double r = fma(-k, tab[2], fma(-k, tab[1], s));
  n = static_cast<int>(k);
  const double z = r * r;
  double e = tab[3];
  e = fma(e, z, tab[4]);
  e = fma(e, z, tab[5]);
  e = fma(e, z, tab[6]);
  e = fma(e, z, tab[7]);
  e = fma(e, z, tab[8]);
  e = fma(e, z, 0.5);
  e = fma(e, z, 1.0);
  double o = tab[9];
  o = fma(o, z, tab[10]);
  o = fma(o, z, tab[11]);
  o = fma(o, z, tab[12]);
  o = fma(o, z, tab[13]);
  o = fma(o, z, tab[14]);
  o = fma(o, z, 1.0);
  o *= r;
  ep = e + o;
  em = e - o;
}

// Natural logarithm of x > 0 plus E ln 2 (as chain64.hip): x = m 2^e with m
// in [2^-1/2, 2^1/2); log m = 2 atanh(s), s = (m - 1) / (m + 1), by its
// series through s^23.  0 gives -inf, anything else outside (0, inf) NaN.
__device__ __forceinline__ double log_t(double x, int E, const double *tab0) {
  const double *tab = table_here(tab0);
  if (!(x > 0.0 && x < __builtin_huge_val()))
    return x == 0.0 ? -__builtin_huge_val() : __builtin_nan("");
  int ex;
  double m = frexp(x, &ex);  // [1/2, 1)
  if (m < tab[28]) {
    m *= 2.0;
    ex -= 1;
  }
  const double f = m - 1.0;  // exact
  const double s = f / (2.0 + f);
  const double z = s * s;
  double p = tab[27];
#pragma unroll
  for (int k = 10; k >= 0; --k) p = fma(p, z, tab[16 + k]);
  const double q = (double)(ex + E);
  return fma(q, tab[1], fma(q, tab[2], 2.0 * s * p));
}

__device__ __forceinline__ void split256(double s, bool fwd, double &fx, double &fy, int &n,
                                         const double *tab) {
  double ep, em;
  exp_split_t(s, ep, em, n, tab);
  fx = fwd ? ep : em;
  fy = fwd ? em : ep;
}

// A DPP lane permutation of a float64 (every lane has a source, or is
// overwritten by the caller).
template <int CTRL>
__device__ __forceinline__ double dpp_mov_f64(double v) {
  const long long b = __builtin_bit_cast(long long, v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(b & 0xffffffffLL), CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), CTRL, 0xf, 0xf, true);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

// Sum over the lane pair of a label: both lanes add the same two values, so
// they end with the same bits.
__device__ __forceinline__ double gsum2(double v) { return v + dpp_mov_f64<0xB1>(v); }

// Largest value over the wave (uniform): within rows of 16 by DPP, then
// over the four rows.
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, true));   // quad_perm 1,0,3,2
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, true));   // quad_perm 2,3,0,1
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xf, 0xf, true));  // row_ror:4
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, true));  // row_ror:8
  const int m0 = __builtin_amdgcn_readlane(v, 0), m1 = __builtin_amdgcn_readlane(v, 16);
  const int m2 = __builtin_amdgcn_readlane(v, 32), m3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(m0, m1), max(m2, m3));
}

// The value of the lane before (row_shr:1; the first lane of each row of 16,
// a lane 0 of a pair, gets 0 and is overwritten by the caller).
__device__ __forceinline__ float shr1_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x111, 0xf, 0xf, true));
}

// r[i] *= 2^-n[lane] for 16 ring registers, in place, on the lanes of
// `mask` (none: skipped); with CL also capped at 2^120.  One asm statement,
// so that the rebase is no branch in the compiler's view (a branch makes it
// merge the ring's two versions with a copy of every register).  The cap
// (K < 64 only) touches registers past the label's K durations: weight 0,
// no longer bounded by the newest entry, and scaled up by every downward
// rebase until they leave the ring; capped, they stay finite, so 0 times
// them stays 0.  With K = 64 every register holds a live duration.
template <bool CL>
__device__ __forceinline__ void rescale16(float *r, int negn, unsigned long long mask);

template <>
__device__ __forceinline__ void rescale16<false>(float *r, int negn, unsigned long long mask) {
  unsigned long long save;
  asm volatile(
      "s_and_saveexec_b64 %[sv], %[m]\n\t"
      "s_cbranch_execz .Lrescale%=\n\t"
      "v_ldexp_f32 %[a0], %[a0], %[n]\n\t"
      "v_ldexp_f32 %[a1], %[a1], %[n]\n\t"
      "v_ldexp_f32 %[a2], %[a2], %[n]\n\t"
      "v_ldexp_f32 %[a3], %[a3], %[n]\n\t"
      "v_ldexp_f32 %[a4], %[a4], %[n]\n\t"
      "v_ldexp_f32 %[a5], %[a5], %[n]\n\t"
      "v_ldexp_f32 %[a6], %[a6], %[n]\n\t"
      "v_ldexp_f32 %[a7], %[a7], %[n]\n\t"
      "v_ldexp_f32 %[a8], %[a8], %[n]\n\t"
      "v_ldexp_f32 %[a9], %[a9], %[n]\n\t"
      "v_ldexp_f32 %[a10], %[a10], %[n]\n\t"
      "v_ldexp_f32 %[a11], %[a11], %[n]\n\t"
      "v_ldexp_f32 %[a12], %[a12], %[n]\n\t"
      "v_ldexp_f32 %[a13], %[a13], %[n]\n\t"
      "v_ldexp_f32 %[a14], %[a14], %[n]\n\t"
      "v_ldexp_f32 %[a15], %[a15], %[n]\n"
      ".Lrescale%=:\n\t"
      "s_mov_b64 exec, %[sv]"
      : [a0] "+v"(r[0]), [a1] "+v"(r[1]), [a2] "+v"(r[2]), [a3] "+v"(r[3]), [a4] "+v"(r[4]),
        [a5] "+v"(r[5]), [a6] "+v"(r[6]), [a7] "+v"(r[7]), [a8] "+v"(r[8]), [a9] "+v"(r[9]),
        [a10] "+v"(r[10]), [a11] "+v"(r[11]), [a12] "+v"(r[12]), [a13] "+v"(r[13]),
        [a14] "+v"(r[14]), [a15] "+v"(r[15]), [sv] "=&s"(save)
      : [n] "v"(negn), [m] "s"(mask)
      : "scc");
}

template <>
__device__ __forceinline__ void rescale16<true>(float *r, int negn, unsigned long long mask) {
  unsigned long long save;
  asm volatile(
      "s_and_saveexec_b64 %[sv], %[m]\n\t"
      "s_cbranch_execz .Lrescale%=\n\t"
      "v_ldexp_f32 %[a0], %[a0], %[n]\n\t"
      "v_min_f32 %[a0], 0x7b800000, %[a0]\n\t"
      "v_ldexp_f32 %[a1], %[a1], %[n]\n\t"
      "v_min_f32 %[a1], 0x7b800000, %[a1]\n\t"
      "v_ldexp_f32 %[a2], %[a2], %[n]\n\t"
      "v_min_f32 %[a2], 0x7b800000, %[a2]\n\t"
      "v_ldexp_f32 %[a3], %[a3], %[n]\n\t"
      "v_min_f32 %[a3], 0x7b800000, %[a3]\n\t"
      "v_ldexp_f32 %[a4], %[a4], %[n]\n\t"
      "v_min_f32 %[a4], 0x7b800000, %[a4]\n\t"
      "v_ldexp_f32 %[a5], %[a5], %[n]\n\t"
      "v_min_f32 %[a5], 0x7b800000, %[a5]\n\t"
      "v_ldexp_f32 %[a6], %[a6], %[n]\n\t"
      "v_min_f32 %[a6], 0x7b800000, %[a6]\n\t"
      "v_ldexp_f32 %[a7], %[a7], %[n]\n\t"
      "v_min_f32 %[a7], 0x7b800000, %[a7]\n\t"
      "v_ldexp_f32 %[a8], %[a8], %[n]\n\t"
      "v_min_f32 %[a8], 0x7b800000, %[a8]\n\t"
      "v_ldexp_f32 %[a9], %[a9], %[n]\n\t"
      "v_min_f32 %[a9], 0x7b800000, %[a9]\n\t"
      "v_ldexp_f32 %[a10], %[a10], %[n]\n\t"
      "v_min_f32 %[a10], 0x7b800000, %[a10]\n\t"
      "v_ldexp_f32 %[a11], %[a11], %[n]\n\t"
      "v_min_f32 %[a11], 0x7b800000, %[a11]\n\t"
      "v_ldexp_f32 %[a12], %[a12], %[n]\n\t"
      "v_min_f32 %[a12], 0x7b800000, %[a12]\n\t"
      "v_ldexp_f32 %[a13], %[a13], %[n]\n\t"
      "v_min_f32 %[a13], 0x7b800000, %[a13]\n\t"
      "v_ldexp_f32 %[a14], %[a14], %[n]\n\t"
      "v_min_f32 %[a14], 0x7b800000, %[a14]\n\t"
      "v_ldexp_f32 %[a15], %[a15], %[n]\n\t"
      "v_min_f32 %[a15], 0x7b800000, %[a15]\n"
      ".Lrescale%=:\n\t"
      "s_mov_b64 exec, %[sv]"
      : [a0] "+v"(r[0]), [a1] "+v"(r[1]), [a2] "+v"(r[2]), [a3] "+v"(r[3]), [a4] "+v"(r[4]),
        [a5] "+v"(r[5]), [a6] "+v"(r[6]), [a7] "+v"(r[7]), [a8] "+v"(r[8]), [a9] "+v"(r[9]),
        [a10] "+v"(r[10]), [a11] "+v"(r[11]), [a12] "+v"(r[12]), [a13] "+v"(r[13]),
        [a14] "+v"(r[14]), [a15] "+v"(r[15]), [sv] "=&s"(save)
      : [n] "v"(negn), [m] "s"(mask)
      : "scc");
}

// Everything one lane carries through a segment of the sweep.
struct Sweep256 {
  S256 sm;
  const double *S;  // cumulative scores of this sequence
  double *row1, *row2;
  const float *drl;   // this lane's exp(dur) column in LDS (duration 32q + 1)
  const float4 *wll;  // this lane's LDS weights: inputs 32w + kWr ..
  int T, C, w, lane, cl, q, isig, t0, nrun, rt0;
  bool fwd, label, rows, lz_tail;
  float Wt[kWr][kR];  // exp(trans): input label 32w + i, output 4 lane + r
  // ring (float32): register (h + j) mod kA = entry of duration 32q + 1 + j
  // of the coming step, h = -(steps done) mod kA
  float r[kA];
  int R;
  double x;  // the coming step's row exp(o) = x 2^E
  int E;
  double fy;  // the coming step's position: its split for the entry
  int fn;
  double sq[kPq];  // scores of the positions 1 .. kPq steps after the coming one
  double o_end, m_end;  // the segment's last o and m (its end record)
  double z_end;
  int zB;
  int done;
  bool ended;
};

__device__ __forceinline__ double score_at(const Sweep256 &c, int step) {
  const int p = min(max(c.t0 + c.isig * step, 0), c.T);
  return c.S[(size_t)p * c.C + (c.label ? c.cl : 0)];
}

// Step base + I + 1 of the segment.  I is the step's place in a block of kA
// steps, so the ring head (-I mod kA), the prefetch slot and the LDS parity
// are compile-time constants.  Whole blocks that end before the segment's
// last step run unpredicated (PRED false); the last, partial block skips
// the steps past the end (PRED true).
template <int I, bool PRED, bool CL>
__device__ __forceinline__ void step256(Sweep256 &c, int base) {
  const int step = base + I + 1;
  if (PRED && (step > c.nrun || c.ended)) return;
  constexpr int par = I & 1;             // LDS parity of this step
  constexpr int iq = I % kPq;            // prefetch slot: the next position's score
  constexpr int H = (kA - I) % kA;       // head of this step's ring
  constexpr int H1 = (H + kA - 1) % kA;  // head of the next step's
  // the next position's score; its slot is refilled kPq steps ahead
  const double s_next = c.sq[iq];
  c.sq[iq] = score_at(c, step + 1 + kPq);
  // 1. the wave's scale and its labels' contraction inputs a = x 2^(E - Bw)
  const int xe = c.x > 0.0 ? c.E + exponent_of(c.x) : kNoExp;
  const int bw = wave_max_i(xe);
  const double a64 = ldexp(c.x, c.E - bw);
  if (PRED && step == c.nrun && c.lz_tail) {
    // log Z of the chain, in this chunk's frame: sum of x 2^E over the labels
    // (only in the last block: an exit the whole blocks cannot take would
    // keep the ring's old version alive through every step)
    if (c.q == 0) c.sm.zb[c.cl] = c.label ? a64 : 0.0;
    if (c.lane == 0) c.sm.zbw[c.w] = bw;
    __syncthreads();
    if (threadIdx.x == 0) {
      int B = kNoExp;
      for (int w = 0; w < kW; ++w) B = max(B, c.sm.zbw[w]);
      double z = 0.0;
      for (int w = 0; w < kW; ++w) {
        double zw = 0.0;
        for (int i = 0; i < kLw; ++i) zw += c.sm.zb[w * kLw + i];
        z += ldexp(zw, c.sm.zbw[w] - B);
      }
      c.z_end = z;
      c.zB = B;
    }
    if (c.rows && c.label && c.q == 0)
      c.row1[(size_t)(c.t0 + c.isig * step - c.rt0) * c.C + c.cl] = log_t(c.x, c.E, c.sm.tab);
    c.done = step;
    c.ended = true;
    return;
  }
  // 2. this lane's partial sums over the wave's 32 inputs for its 4 outputs
  // (float32); the inputs come from lanes 2i through scalar registers
  {
    const float a32 = (float)a64;
    const int ab = __builtin_bit_cast(int, a32);
    float acc[kR] = {0.0f, 0.0f, 0.0f, 0.0f};
    // the LDS weights in quarters, each loaded while register-weight terms
    // run (a bound on the registers their loads hold); products and sums in
    // float32, one accumulator per output
    constexpr int kNh = 4, kH = kWl / kNh, kRh = kWr / kNh;
    float4 wv[kH];
#pragma unroll
    for (int hh = 0; hh < kNh; ++hh) {
#pragma unroll
      for (int i = 0; i < kH; ++i) wv[i] = c.wll[(hh * kH + i) * 64];
#pragma unroll
      for (int i = hh * kRh; i < (hh + 1) * kRh; ++i) {
        const float ai = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, 2 * i));
#pragma unroll
        for (int r = 0; r < kR; ++r) acc[r] = fmaf(ai, c.Wt[i][r], acc[r]);
      }
#pragma unroll
      for (int i = 0; i < kH; ++i) {
        const int ii = kWr + hh * kH + i;
        const float ai = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, 2 * ii));
        acc[0] = fmaf(ai, wv[i].x, acc[0]);
        acc[1] = fmaf(ai, wv[i].y, acc[1]);
        acc[2] = fmaf(ai, wv[i].z, acc[2]);
        acc[3] = fmaf(ai, wv[i].w, acc[3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float4 pv;
    pv.x = acc[0];
    pv.y = acc[1];
    pv.z = acc[2];
    pv.w = acc[3];
    *reinterpret_cast<float4 *>(c.sm.part + (par * kW + c.w) * kLab + kR * c.lane) = pv;
    if (c.lane == 0) c.sm.bw[par * kW + c.w] = bw;
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  // 3. the ring of the next step but its newest entry: lane 2i's oldest
  // entry (register H1) moves to lane 2i+1, lane 2i's register H1 waits for
  // this step's entry; the K-sum over it.  Independent of this step's entry,
  // so it fills the latency of the dependent chain below (partials ->
  // entry -> next row) instead of delaying the barrier.
  c.r[H1] = c.q == 0 ? 0.0f : shr1_f32(c.r[H1]);
  float sa0 = 0.0f, sa1 = 0.0f;
#pragma unroll
  for (int j = 0; j < kA; j += 2) {
    sa0 = fmaf(c.drl[j * kLab], c.r[(H1 + j) % kA], sa0);
    sa1 = fmaf(c.drl[(j + 1) * kLab], c.r[(H1 + j + 1) % kA], sa1);
  }
  const double gk = gsum2((double)sa0 + (double)sa1);
  // 4. this label's contraction: the 8 waves' partials at the step scale B
  int bws[kW];
  {
    const int4 b0 = *reinterpret_cast<const int4 *>(c.sm.bw + par * kW);
    const int4 b1 = *reinterpret_cast<const int4 *>(c.sm.bw + par * kW + 4);
    bws[0] = b0.x; bws[1] = b0.y; bws[2] = b0.z; bws[3] = b0.w;
    bws[4] = b1.x; bws[5] = b1.y; bws[6] = b1.z; bws[7] = b1.w;
  }
  int B = bws[0];
#pragma unroll
  for (int i = 1; i < kW; ++i) B = max(B, bws[i]);
  double dq = 0.0;
#pragma unroll
  for (int j = 0; j < kW / 2; ++j) {
    const int wsrc = (kW / 2) * c.q + j;
    const int bsel = c.q == 0 ? bws[j] : bws[kW / 2 + j];
    dq += ldexp((double)c.sm.part[(par * kW + wsrc) * kLab + c.cl], bsel - B);
  }
  const double d = gsum2(dq);
  // 5. the entry exp(m -+ S) / 2^R = d fy 2^(B -+ n - R), its rebase
  const double y = d * c.fy;
  const int sh = B - c.isig * c.fn - c.R;
  // When a label of the wave leaves the bound, every label of the wave
  // rebases at once by its own exponent (an exact power of two either way):
  // the labels drift alike, so they reach the bound again together and the
  // wave runs the rescale about once every few steps instead of whenever any
  // one of its 32 labels crosses.
  int n = 0;
  const int ey = c.label ? exponent_of(y) + sh : 0;
  if (__any(ey > kRebase || ey < -kRebase)) n = ey;
  c.R += n;
  const float e = c.label ? (float)ldexp(y, sh - n) : 0.0f;
  {  // the label's registers into the new reference (lanes that rebase)
    const unsigned long long m = __ballot(n != 0);
    rescale16<CL>(c.r, -n, m);
    rescale16<CL>(c.r + 16, -n, m);
  }
  c.r[H1] = c.q == 0 ? e : c.r[H1];  // the new entry: duration 1 of the next step
  // 6. the rows of this step: lane 0 of the pair o = log(x 2^E), lane 1
  // m = log(d 2^B)
  if (c.rows && c.label) {
    const double lv = log_t(c.q == 0 ? c.x : d, c.q == 0 ? c.E : B, c.sm.tab);
    double *dst = c.q == 0 ? c.row1 : c.row2;
    dst[(size_t)(c.t0 + c.isig * step - c.rt0) * c.C + c.cl] = lv;
  }
  if (PRED && step == c.nrun) {  // the segment's last step: its record's o and m
    c.o_end = log_t(c.x, c.E, c.sm.tab);
    c.m_end = log_t(d, B, c.sm.tab);
  }
  // 7. the next step's row: its K-sum (taken before the rebase: exact
  // power-of-two correction) plus the new entry's term, times exp(+-S)
  double fx1, fy1;
  int n1;
  split256(s_next, c.fwd, fx1, fy1, n1, c.sm.tab);
  c.x = c.label ? (ldexp(gk, -n) + (double)c.sm.dr[c.cl] * (double)e) * fx1 : 0.0;
  c.E = c.R + c.isig * n1;
  c.fy = fy1;
  c.fn = n1;
  c.done = step;
}

template <bool PRED, bool CL, int... Is>
__device__ __forceinline__ void block256(Sweep256 &c, int base,
                                         std::integer_sequence<int, Is...>) {
  (step256<Is, PRED, CL>(c, base), ...);
}

}  // namespace

// One workgroup per (direction, sequence, chunk), as k_sweep (chain.hip):
// the same launch grid, start states, records ([K][C] ring by slot, then R,
// o, m), verification hand-off, log Z of the tail chunk and replay windows.
// CL: K < 64 (ring registers past K exist; see rescale16).
template <bool CL, bool REP>
__global__ __launch_bounds__(kNT) void k_sweep256(ChainShape sh, const float *__restrict__ trans,
                                                  const float *__restrict__ dur, Escaled es,
                                                  const int32_t *__restrict__ lengths,
                                                  PitBufs pb, int iter) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int nck = sh.B * sh.nchunk;
  const bool replay = iter == -1;
  bool fwd;
  int b, jc;
  if (REP) {  // the in-order repair: one workgroup per (direction, sequence)
    fwd = (int)blockIdx.x < sh.B;
    b = fwd ? blockIdx.x : blockIdx.x - sh.B;
    jc = 0;
  } else if (replay) {
    const int nf = sh.B * sh.rnf;
    fwd = (int)blockIdx.x < nf;
    const int nj = fwd ? sh.rnf : sh.rnb;
    const int rem = fwd ? blockIdx.x : blockIdx.x - nf;
    b = rem / nj;
    jc = sh.rj0 + rem % nj;
  } else {
    fwd = (int)blockIdx.x < nck;
    const int rem = fwd ? blockIdx.x : blockIdx.x - nck;
    b = rem / sh.nchunk;
    jc = rem % sh.nchunk;
  }
  const size_t base = (fwd ? 0 : (size_t)nck) + (size_t)b * sh.nchunk;  // this chain's flags
  const size_t idx = base + jc;
  if (!REP && iter == 0) {  // the parallel-in-time state, before any verification reads it
    if (threadIdx.x == 0) {
      pb.redo[idx] = 1;
      pb.corr_i[idx] = 0;
      pb.corr_f[idx] = 0.0;
    }
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < sh.nchunk; i += kNT) pb.nbad[i] = 0;
  }
  const int L = lengths[b];
  const int tid = threadIdx.x, C = sh.C, K = sh.K, T = sh.T;
  if (L < 1 || L > T || jc >= sh.nchunk) return;
  if (jc * sh.delta >= L) return;
  const int nvalid = (L + sh.delta - 1) / sh.delta;
  __shared__ PitMaxArg red[kNT / 64];  // scratch of the repair's checks
  __shared__ double redd[kNT / 64];
  if constexpr (REP) {
    // nothing to repair unless the last parallel check found a chunk of
    // this chain inconsistent
    if (pb.nbad[kPitParallelIters - 1] == 0) return;
    int marked = 0;
    for (int j = tid; j < nvalid; j += kNT) marked |= pb.redo[base + j];
    if (!pit_any<kNT>(marked != 0, red)) return;
  } else {
    if (iter > 0 && (pb.nbad[iter - 1] == 0 || pb.redo[idx] == 0)) return;
  }
  const size_t ob = (size_t)b * (T + 1) * C;
  const size_t cks = ck_stride(C, K);
  const size_t kc = (size_t)K * C;
  const int isig = fwd ? 1 : -1;
  const bool rows = pb.row_a != nullptr;
  const size_t orow = (size_t)b * pb.row_stride * C;

  Sweep256 c;
  c.sm = carve256(lds);
  if (tid < kTabN) c.sm.tab[tid] = kTab256[tid];
  // exp(dur) table: durations past K and labels past C are 0
  for (int i = tid; i < kDmax * kLab; i += kNT) {
    const int k = i / kLab + 1, l = i % kLab;
    c.sm.dr[i] = (k <= K && l < C) ? (float)exp((double)dur[(size_t)(k - 1) * C + l]) : 0.0f;
  }
  c.S = es.S + ob;
  c.row1 = rows ? (fwd ? pb.row_a : pb.row_v) + orow : nullptr;  // alpha / v
  c.row2 = rows ? (fwd ? pb.row_u : pb.row_b) + orow : nullptr;  // u / beta
  c.T = T;
  c.C = C;
  c.w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  c.lane = tid & 63;
  c.cl = kLw * c.w + (c.lane >> 1);  // this lane's label (K-sum role)
  c.q = c.lane & 1;                  // its duration half
  c.isig = isig;
  c.rt0 = pb.row_t0;
  c.fwd = fwd;
  c.label = c.cl < C;
  c.drl = c.sm.dr + (size_t)kA * c.q * kLab + c.cl;
  const int cl = c.cl, q = c.q;
  const bool label = c.label;
  // exp(trans) of the contraction role: input 32w + i, output 4 lane + r
  // (forward: previous label -> label; backward: label -> next label),
  // formed by loops (one copy of the exponential's code) through LDS and
  // then taken into registers at compile-time indices
  auto wgt = [&](int i, int r) {
    const int ci = kLw * c.w + i, co = kR * c.lane + r;
    return (ci < C && co < C) ? (float)exp((double)(fwd ? trans[(size_t)ci * C + co]
                                                        : trans[(size_t)co * C + ci]))
                              : 0.0f;
  };
  float *stage = c.sm.wl;  // [kWr / 8][8][kR] per lane, in rounds of 8 inputs
  constexpr int kRound = 8;
#pragma unroll 1
  for (int i0 = 0; i0 < kWr; i0 += kRound) {
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j < kRound * kR; ++j)
      stage[(size_t)j * kNT + tid] = wgt(i0 + j / kR, j % kR);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWr; ++i)
      if (i >= i0 && i < i0 + kRound)
#pragma unroll
        for (int r = 0; r < kR; ++r) c.Wt[i][r] = stage[(size_t)((i - i0) * kR + r) * kNT + tid];
  }
  __syncthreads();
  c.wll = reinterpret_cast<const float4 *>(c.sm.wl) + (size_t)c.w * kWl * 64 + c.lane;
#pragma unroll 1
  for (int i = 0; i < kWl; ++i) {
    float4 v;
    v.x = wgt(kWr + i, 0);
    v.y = wgt(kWr + i, 1);
    v.z = wgt(kWr + i, 2);
    v.w = wgt(kWr + i, 3);
    reinterpret_cast<float4 *>(c.sm.wl)[((size_t)c.w * kWl + i) * 64 + c.lane] = v;
  }
  __syncthreads();  // the tables
  const int nval = max(0, min(kA, K - kA * q));  // valid ring registers of this lane
  // stores the ring (head h) whose newest position is tref as a record, with
  // R, o, m: each register to the slot of its entry
  auto save_ring = [&](double *__restrict__ dst, int tref, int h, double o, double m) {
    if (label) {
      const int s_first = pslot(tref - isig * kA * q, K);
      double *dl = dst + cl;
#pragma unroll
      for (int p = 0; p < kA; ++p) {
        const int j = (p - h) & (kA - 1);  // the register's entry: duration 32q + 1 + j
        if (j < nval) {
          int sl = s_first - isig * j;
          sl += sl < 0 ? K : 0;
          sl -= sl >= K ? K : 0;
          dl[(size_t)sl * C] = (double)c.r[p];
        }
      }
      if (q == 0) {
        dst[kc + cl] = (double)c.R;
        dst[kc + C + cl] = o;
        dst[kc + 2 * C + cl] = m;
      }
    }
  };

  // one chunk, p0 .. p1, from its start record (or, at iteration 0, from
  // its exact or neutral start after the burn-in)
  auto sweep_chunk = [&](const int jc) __attribute__((always_inline)) {
    const int p0 = jc * sh.delta;
    const int p1 = min(p0 + sh.delta, L);
    double *rec_start = (fwd ? pb.ck_fwd : pb.ck_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
    double *rec_end = (fwd ? pb.end_fwd : pb.end_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
    const int tstart = fwd ? p0 : p1;
    const bool tail = fwd ? (p1 == L) : (p0 == 0);
    const bool exact = fwd ? (jc == 0) : (p1 == L);
    const int wb = (iter == 0 && !exact) ? min(sh.burn, fwd ? p0 : L - p1) : 0;
    const int tb = fwd ? p0 - wb : p1 + wb;  // where the sweep starts
    for (int seg = wb > 0 ? 0 : 1; seg < 2; ++seg) {
      const bool main = seg == 1;
      c.t0 = main ? tstart : tb;
      c.nrun = main ? p1 - p0 : wb;
      c.rows = rows && main;
      c.lz_tail = main && tail;
      // ---- the start state, head 0
      c.R = 0;
      if (iter == 0 && (!main || wb == 0)) {
        if (exact) {
          // entry u[0] - S[0] = 0 forward; beta[L] + S[L] = S[L] backward
          double v = 1.0;
          if (!fwd) {
            double em;
            exp_split_t(c.S[(size_t)L * C + (label ? cl : 0)], v, em, c.R, c.sm.tab);
          }
          if (!label) {
            c.R = 0;
            v = 0.0;
          }
  #pragma unroll
          for (int j = 0; j < kA; ++j) c.r[j] = (q == 0 && j == 0) ? (float)v : 0.0f;
        } else {
          // neutral start: every entry of the window (positions inside [0, L]) is 1
  #pragma unroll
          for (int j = 0; j < kA; ++j) {
            const int pos = c.t0 - isig * (kA * q + j);
            c.r[j] = (label && kA * q + 1 + j <= K && pos >= 0 && pos <= L) ? 1.0f : 0.0f;
          }
        }
        if (main) {
          save_ring(rec_start, c.t0, 0, exact ? -__builtin_huge_val() : __builtin_nan(""),
                    exact ? 0.0 : __builtin_nan(""));
          if (exact && q == 0 && label && rows)  // u[0] = 0 forward, beta[L] = 0 backward
            c.row2[(size_t)(tstart - c.rt0) * C + cl] = 0.0;
        }
      } else {
        // the chunk's start record (written by the burn-in segment just now, or
        // by an earlier sweep); each lane reads back the slots it wrote itself
        if (wb > 0) {
          __threadfence_block();
          __syncthreads();
        }
  #pragma unroll
        for (int j = 0; j < kA; ++j) {
          const int k = kA * q + 1 + j;
          c.r[j] = (label && k <= K)
                       ? (float)rec_start[(size_t)pslot(c.t0 - isig * (k - 1), K) * C + cl]
                       : 0.0f;
        }
        c.R = label ? (int)rec_start[kc + cl] : 0;
        if (replay && rows && q == 0 && label &&
            (fwd ? jc == sh.rj0 : (jc == sh.rj0 + sh.rnb - 1 || p1 == L))) {
          c.row1[(size_t)(tstart - c.rt0) * C + cl] = rec_start[kc + C + cl];
          c.row2[(size_t)(tstart - c.rt0) * C + cl] = rec_start[kc + 2 * C + cl];
        }
      }
      // the scores of the first steps: position 1 split now, 2 .. kPq + 1 queued
  #pragma unroll
      for (int j = 0; j < kPq; ++j) c.sq[j] = score_at(c, 2 + j);
      {  // the first step's row: K-sum over the whole start ring (its newest
         // entry included), times exp(+-S) of position 1
        float sa0 = 0.0f, sa1 = 0.0f;
  #pragma unroll
        for (int j = 0; j < kA; j += 2) {
          sa0 = fmaf(c.drl[j * kLab], c.r[j], sa0);
          sa1 = fmaf(c.drl[(j + 1) * kLab], c.r[j + 1], sa1);
        }
        const double g1 = gsum2((double)sa0 + (double)sa1);
        double fx;
        split256(score_at(c, 1), fwd, fx, c.fy, c.fn, c.sm.tab);
        c.x = label ? g1 * fx : 0.0;
        c.E = c.R + isig * c.fn;
      }
      // ---- the steps, in blocks of kA
      c.z_end = 0.0;
      c.zB = 0;
      c.done = 0;
      c.ended = false;
      c.o_end = c.m_end = 0.0;
      const int nfull = (c.nrun - 1) / kA;  // whole blocks before the last step's
      for (int blk = 0; blk < nfull; ++blk)
        block256<false, CL>(c, blk * kA, std::make_integer_sequence<int, kA>{});
      block256<true, CL>(c, nfull * kA, std::make_integer_sequence<int, kA>{});
      if (c.ended) {
        if (!replay && tid == 0) pb.lz_part[(fwd ? 0 : sh.B) + b] = log_t(c.z_end, c.zB, c.sm.tab);
      } else {
        // the ring after the segment: its record (with the last step's o, m);
        // the position and head pass through an empty asm statement so that
        // the record's addresses are formed here, not before the step loop
        // (where they would stay live through it)
        int h = (kA - c.nrun % kA) % kA, tref = c.t0 + isig * c.nrun;
        asm volatile("" : "+v"(h), "+v"(tref));
        if (!main)
          save_ring(rec_start, tref, h, c.o_end, c.m_end);
        else if (!replay)
          save_ring(rec_end, tref, h, c.o_end, c.m_end);
      }
      // (the next segment reuses the LDS step buffers: wait for all)
      __syncthreads();
    }
  };
  if constexpr (REP) {
    // the chain's chunks in order, past its exact one: a marked chunk is
    // swept from its replaced start, then its successor is checked against
    // the new end (forced to take it if the successor is marked too: its own
    // end belongs to an older start)
    for (int s = 1; s < nvalid; ++s) {
      const int j = fwd ? s : nvalid - 1 - s;
      if (pb.redo[base + j] == 0) continue;
      sweep_chunk(j);
      if (s + 1 < nvalid) {
        const int jn = fwd ? j + 1 : j - 1;
        __threadfence_block();  // the end record, for every thread of the check
        __syncthreads();
        pit_check<kNT>(sh, pb, fwd, b, jn, -1, pb.redo[base + jn] != 0, red, redd);
      }
    }
  } else {
    sweep_chunk(jc);
  }
}

size_t sweep256_lds_bytes(int K) {
  (void)K;  // the exp(dur) table always has kDmax rows
  return kLdsBytes;
}

bool sweep256_applies(int C, int K) {
  return C > 64 && C <= kLab && K >= 1 && K <= kDmax && sweep256_lds_bytes(K) <= kMaxDynLds;
}

hipError_t launch_sweep_256(const ChainShape &sh, const float *trans, const float *dur,
                            const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                            int with_bwd, int iter, hipStream_t st) {
  const size_t lds = sweep256_lds_bytes(sh.K);
  const bool cl = sh.K < kDmax, rep = iter == kPitRepair;
  const void *f = cl ? (rep ? (const void *)k_sweep256<true, true>
                            : (const void *)k_sweep256<true, false>)
                     : (rep ? (const void *)k_sweep256<false, true>
                            : (const void *)k_sweep256<false, false>);
  if (!sweep256_applies(sh.C, sh.K) || !lds_fits(f, lds)) return hipErrorInvalidConfiguration;
  const int nd = with_bwd ? 2 : 1;
  const int grid = rep ? nd * sh.B : iter < 0 ? sh.B * (sh.rnf + sh.rnb) : nd * sh.B * sh.nchunk;
#define SEMICRF_SWEEP256(CLV, REPV)                                                             \
  hipLaunchKernelGGL((k_sweep256<CLV, REPV>), dim3(grid), dim3(kNT), lds, st, sh, trans, dur, es, \
                     lengths, pb, iter)
  if (cl) {
    if (rep)
      SEMICRF_SWEEP256(true, true);
    else
      SEMICRF_SWEEP256(true, false);
  } else {
    if (rep)
      SEMICRF_SWEEP256(false, true);
    else
      SEMICRF_SWEEP256(false, false);
  }
#undef SEMICRF_SWEEP256
  return hipGetLastError();
}

}  // namespace semicrf
