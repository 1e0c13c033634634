// chain64.hip -- streaming semi-CRF sweep for 32 < C <= 64 labels, K <= 256,
// with the ring of the K newest entries held in registers.
//
// Same recurrences, exp-space entries with integer references, checkpoint
// records and row outputs as chain.hip (see its header for the equations and
// the exact power-of-two arithmetic; method: "Streaming Structured Inference
// with Flash-SemiCRF", abstract and technical summary sections 2.A-2.C).
// At these shapes (extreme scale: C = 64, K = 256) one chain fills a compute
// unit, so the time of one step is the throughput.  A ring in LDS is read
// whole every step (K x 64 float64 = 128 KB, about 1000 cycles of LDS
// bandwidth alone); here it lives in the register file, laid out so that a
// step needs almost no traffic between waves:
//   * 8 waves x 64 lanes = 64 labels x 8 lanes.  Lane q (0..7) of label c
//     holds durations k = 32q + 1 .. 32q + 32 of that label: 32 float64 ring
//     registers next to their weights exp(dur[k-1][c]), and exp(trans) of
//     the 8 input labels 8q .. 8q + 7 of the contraction into c.  A wave owns
//     8 whole labels.
//   * the K-sum of a label is 32 multiply-adds per lane and a sum over its 8
//     lanes (a DPP butterfly whose every lane ends with the same bits); so
//     is the contraction.  The ring's shift by one position is one DPP move:
//     the oldest entry of lane q goes to lane q + 1 of the same label, the
//     new entry to lane 0.
//   * the 32 registers form a circular buffer: the entry of duration
//     32q + 1 + j in register (h + j) mod 32, the head h moving back by one
//     per step, so the shift moves one register, not 32.  The step loop runs
//     in blocks of 32 steps whose bodies are instantiated for their place in
//     the block (a template), so the head and every ring register index are
//     compile-time constants; the steps are predicated, so a block's control
//     flow is a plain sequence.
//   * one barrier per step, the only exchange between waves: each label's
//     row (exp(o) = x 2^E), its exponent and a = x 2^(E-B) with the carried
//     step scale B go to LDS; after the barrier every lane reads those of its
//     8 input labels (broadcast reads).  The 8 lanes of a label together
//     hold all 64, so a max over them gives every wave the same new step
//     scale (the largest exponent over all labels, carried while it stays
//     within a span; when it moves, a is formed anew from x and E).  Then
//     the lane's share of the contraction.  The new
//     entry, its rebase (R[c] += n, the label's registers rescaled by 2^-n
//     exactly) and the next K-sum stay within the label's 8 lanes.
//   * rows: lane q keeps the raw values (x, E, d, B) of the steps s with
//     s - 1 = q (mod 8); every 8 steps all lanes take their logarithms and
//     store them together.  The constants of the logarithm and of the score
//     split live in LDS and are read where they are used (as literals the
//     compiler keeps them in registers across the loop and the ring spills).
//   * a chunk with a burn-in runs it as a first segment of the same loop; its
//     end state is the chunk's start record, from which the chunk's own
//     positions run as the second segment.
#include <stdio.h>
#include <stdlib.h>

#include <utility>

#include "device_math.h"
#include "internal.h"
#include "pitcheck.h"

namespace semicrf {

namespace {

constexpr int kW = 8;         // waves, 8 labels each
constexpr int kG = 8;         // lanes per label
constexpr int kA = 32;        // durations per lane
constexpr int kNT = 64 * kW;
constexpr int kLab = 64;      // labels, padded with zero weights
constexpr int kPf = 8;        // steps per score-prefetch block
constexpr int kRebase = 512;  // rebase bound, log2 units (as chain.hip)
constexpr int kSpan = 256;    // step-scale span, log2 units (as chain.hip)
// x and E of the labels in LDS by blocks of 8 (one block per input share):
// block q at q * 10 doubles / q * 12 ints, so the 16-byte reads of the 8
// blocks fall on distinct banks
constexpr int kXS = 10, kES = 12;

// Constants of the exponential split and of the logarithm (read from LDS
// where they are used).
constexpr int kTabN = 32;
__constant__ double kTab64[kTabN] = {
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

struct S64 {
  double *xr;         // [2][8][kXS]: x of each label (block, index), by step parity
  double *ar;         // [2][8][kXS]: a = x 2^(E-B) with the carried step scale B
  double *pfx, *pfy;  // [2][kPf][64]: split scores
  double *tab;        // [kTabN]
  double *rx, *rd;    // [kPf][64]: x and d of the last kPf steps (rows, end record)
  int *er;            // [2][8][kES]: E of each label
  int *xe;            // [2][8][kES]: exponent of x 2^E of each label
  int *pfn;           // [2][kPf][64]
  int *re;            // [kPf][64]: E of the last kPf steps
  int *rb;            // [kPf]: their step scales
};

constexpr size_t kLdsBytes = (size_t)2 * 2 * kG * kXS * 8 + (size_t)2 * 2 * kPf * kLab * 8 +
                             (size_t)kTabN * 8 + (size_t)2 * kPf * kLab * 8 +
                             (size_t)2 * 2 * kG * kES * 4 + (size_t)2 * kPf * kLab * 4 +
                             (size_t)kPf * kLab * 4 + (size_t)kPf * 4;

__device__ __forceinline__ S64 carve64(unsigned char *base) {
  S64 m;
  size_t off = 0;
  m.xr = reinterpret_cast<double *>(base + off); off += (size_t)2 * kG * kXS * 8;
  m.ar = reinterpret_cast<double *>(base + off); off += (size_t)2 * kG * kXS * 8;
  m.pfx = reinterpret_cast<double *>(base + off); off += (size_t)2 * kPf * kLab * 8;
  m.pfy = reinterpret_cast<double *>(base + off); off += (size_t)2 * kPf * kLab * 8;
  m.tab = reinterpret_cast<double *>(base + off); off += (size_t)kTabN * 8;
  m.rx = reinterpret_cast<double *>(base + off); off += (size_t)kPf * kLab * 8;
  m.rd = reinterpret_cast<double *>(base + off); off += (size_t)kPf * kLab * 8;
  m.er = reinterpret_cast<int *>(base + off); off += (size_t)2 * kG * kES * 4;
  m.xe = reinterpret_cast<int *>(base + off); off += (size_t)2 * kG * kES * 4;
  m.pfn = reinterpret_cast<int *>(base + off); off += (size_t)2 * kPf * kLab * 4;
  m.re = reinterpret_cast<int *>(base + off); off += (size_t)kPf * kLab * 4;
  m.rb = reinterpret_cast<int *>(base + off);
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

// Natural logarithm of x > 0 plus E ln 2: x = m 2^e with m in [2^-1/2,
// 2^1/2); log m = 2 atanh(s), s = (m - 1) / (m + 1), |s| <= 0.172, by its
// series sum_k s^(2k+1) / (2k+1) through k = 11 (the next term is below
// 1e-18 of the sum).  0 gives -inf, anything else outside (0, inf) NaN.
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

__device__ __forceinline__ void split64(double s, bool fwd, double &fx, double &fy, int &n,
                                        const double *tab) {
  double ep, em;
  exp_split_t(s, ep, em, n, tab);
  fx = fwd ? ep : em;
  fy = fwd ? em : ep;
}

// A DPP lane permutation of a float64 without an "old" operand (every lane
// has a source, or is overwritten by the caller), so no copy is made.
template <int CTRL>
__device__ __forceinline__ double dpp_mov_f64(double v) {
  const long long b = __builtin_bit_cast(long long, v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(b & 0xffffffffLL), CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), CTRL, 0xf, 0xf, true);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

// Sum over the 8 lanes of a label (aligned groups of 8: lane ^ 1, lane ^ 2,
// the other quad): a butterfly whose every step adds the same two values in
// every lane, so all 8 lanes end with the same bits.
__device__ __forceinline__ double gsum8(double v) {
  v += dpp_mov_f64<0xB1>(v);
  v += dpp_mov_f64<0x4E>(v);
  v += dpp_mov_f64<0x141>(v);
  return v;
}

// Largest value over the 8 lanes of a label (every lane gets it).
__device__ __forceinline__ int gmax8_i(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, true));
  return v;
}

// The value of the lane before (row_shr:1; the first lane of each row of 16,
// a lane 0 of a label, gets 0 and is overwritten by the caller).
__device__ __forceinline__ double shr1_f64(double v) { return dpp_mov_f64<0x111>(v); }

// r[i] *= 2^-n[lane] for 16 ring registers, in place, on the lanes of
// `mask` (none: skipped).  Written as one asm statement so that the rare
// rebase is no branch in the compiler's view: a branch there makes it merge
// the ring's two versions with a copy of every register.
__device__ __forceinline__ void rescale16(double *r, int negn, unsigned long long mask) {
  unsigned long long save;
  asm volatile(
      "s_and_saveexec_b64 %[sv], %[m]\n\t"
      "s_cbranch_execz .Lrescale%=\n\t"
      "v_ldexp_f64 %[a0], %[a0], %[n]\n\t"
      "v_ldexp_f64 %[a1], %[a1], %[n]\n\t"
      "v_ldexp_f64 %[a2], %[a2], %[n]\n\t"
      "v_ldexp_f64 %[a3], %[a3], %[n]\n\t"
      "v_ldexp_f64 %[a4], %[a4], %[n]\n\t"
      "v_ldexp_f64 %[a5], %[a5], %[n]\n\t"
      "v_ldexp_f64 %[a6], %[a6], %[n]\n\t"
      "v_ldexp_f64 %[a7], %[a7], %[n]\n\t"
      "v_ldexp_f64 %[a8], %[a8], %[n]\n\t"
      "v_ldexp_f64 %[a9], %[a9], %[n]\n\t"
      "v_ldexp_f64 %[a10], %[a10], %[n]\n\t"
      "v_ldexp_f64 %[a11], %[a11], %[n]\n\t"
      "v_ldexp_f64 %[a12], %[a12], %[n]\n\t"
      "v_ldexp_f64 %[a13], %[a13], %[n]\n\t"
      "v_ldexp_f64 %[a14], %[a14], %[n]\n\t"
      "v_ldexp_f64 %[a15], %[a15], %[n]\n"
      ".Lrescale%=:\n\t"
      "s_mov_b64 exec, %[sv]"
      : [a0] "+v"(r[0]), [a1] "+v"(r[1]), [a2] "+v"(r[2]), [a3] "+v"(r[3]), [a4] "+v"(r[4]),
        [a5] "+v"(r[5]), [a6] "+v"(r[6]), [a7] "+v"(r[7]), [a8] "+v"(r[8]), [a9] "+v"(r[9]),
        [a10] "+v"(r[10]), [a11] "+v"(r[11]), [a12] "+v"(r[12]), [a13] "+v"(r[13]),
        [a14] "+v"(r[14]), [a15] "+v"(r[15]), [sv] "=&s"(save)
      : [n] "v"(negn), [m] "s"(mask)
      : "scc");
}

// Everything one lane carries through a segment of the sweep: constants,
// the ring registers and the loop state (one object, split into registers
// once the step bodies are inlined).
struct Sweep64 {
  S64 sm;
  const double *S;  // cumulative scores of this sequence
  double *row1, *row2;
  int T, C, K, w, lane, cl, q, isig, t0, nrun, rt0;
  bool fwd, label, rows, lz_tail;
  double Dr[kA], Wt[kG], D1;
  // ring: register (h + j) mod kA = entry of duration 32q + 1 + j of the
  // coming step, h = -(steps done) mod kA
  double r[kA];
  int R, Bm;
  double x;  // the coming step's row exp(o) = x 2^E
  int E;
  double pf_s;
  double z_end;
  int done;     // steps done (the last one may be the chain's last, log Z)
  int flushed;  // steps whose rows are stored
  bool ended;
};

// The rows of steps flushed+1 .. done (all within one block of kPf steps,
// staged in LDS by the lanes 0 of the labels): lane q takes step
// (block start) + q, its logarithms and its stores; the chain's last step
// (log Z) has no second row.
__device__ __forceinline__ void flush_rows(Sweep64 &c) {
  const int s = (c.flushed / kPf) * kPf + 1 + c.q;
  if (c.rows && c.label && s > c.flushed && s <= c.done) {
    const int i = (s - 1) % kPf;
    const size_t tr = (size_t)(c.t0 + c.isig * s - c.rt0) * c.C + c.cl;
    c.row1[tr] = log_t(c.sm.rx[i * kLab + c.cl], c.sm.re[i * kLab + c.cl], c.sm.tab);
    if (!(c.ended && s == c.done))
      c.row2[tr] = log_t(c.sm.rd[i * kLab + c.cl], c.sm.rb[i], c.sm.tab);
  }
  c.flushed = c.done;
}

// Step base + I + 1 of the segment.  I is the step's place in a block of kA
// steps, so the ring head (-I mod kA), the prefetch slot and every LDS
// parity are compile-time constants.  Whole blocks that end before the
// segment's last step run unpredicated (PRED false): their control flow is
// one sequence, with no merge of the ring's versions; the last, partial
// block skips the steps past the end (PRED true).
template <int I, bool PRED>
__device__ __forceinline__ void step64(Sweep64 &c, int base) {
  const int step = base + I + 1;
  if (PRED && (step > c.nrun || c.ended)) return;
  constexpr int ipf = I % kPf, buf = (I / kPf) & 1;
  constexpr int ipf1 = (I + 1) % kPf, buf1 = ((I + 1) / kPf) & 1;  // the next step's slot
  constexpr int par = I & 1;             // LDS parity of this step
  constexpr int H = (kA - I) % kA;       // head of this step's ring
  constexpr int H1 = (H + kA - 1) % kA;  // head of the next step's
  const bool next_blk = step - 1 - ipf + kPf < c.nrun;
  if (ipf == 0 && next_blk)  // lane q: label cl at step + kPf + q
    c.pf_s = c.S[(size_t)min(max(c.t0 + c.isig * (step + kPf + c.q), 0), c.T) * c.C +
                 (c.label ? c.cl : 0)];
  // 1. this step's row exp(o) = x 2^E (formed in the step before), its
  // exponent and a = x 2^(E-B) with the carried scale B, published; the row
  // values kept for the row outputs
  if (c.q == 0) {
    const int lb = c.cl >> 3, li = c.cl & 7;
    c.sm.xr[(par * kG + lb) * kXS + li] = c.x;
    c.sm.ar[(par * kG + lb) * kXS + li] = ldexp(c.x, c.E - c.Bm);
    c.sm.er[(par * kG + lb) * kES + li] = c.E;
    c.sm.xe[(par * kG + lb) * kES + li] = c.x > 0.0 ? c.E + exponent_of(c.x) : kNoExp;
    c.sm.rx[ipf * kLab + c.cl] = c.x;
    c.sm.re[ipf * kLab + c.cl] = c.E;
  }
  __syncthreads();
  // the reads of this lane's 8 input labels (block q) first: their latency
  // hides behind the K-sum below
  double a[kG];
  int xev[kG];
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    a[i] = c.sm.ar[(par * kG + c.q) * kXS + i];
    xev[i] = c.sm.xe[(par * kG + c.q) * kES + i];
  }
  __builtin_amdgcn_sched_barrier(0);
  // 2. the ring of the next step but its newest entry: the oldest entry of
  // each lane (register H1) moves to the next lane of the label, lane 0's
  // register H1 waits for this step's entry; the K-sum over it.  Nothing
  // here depends on this step's entry, so these multiply-adds run beside
  // the chain below.
  c.r[H1] = c.q == 0 ? 0.0 : shr1_f64(c.r[H1]);
  double sa[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int j = 0; j < kA; ++j) sa[j & 3] = fma(c.Dr[j], c.r[(H1 + j) % kA], sa[j & 3]);
  const double gk = gsum8((sa[0] + sa[1]) + (sa[2] + sa[3]));
  // 3. the step scale B: the largest exponent over all labels -- over the 8
  // blocks the label's 8 lanes hold, the same in every lane and every wave
  // -- kept while it stays within the span (then the published a hold);
  // when it moves, a = x 2^(E-B) anew from the raw values (the same bits
  // the publisher would have formed)
  int mxl = kNoExp;
#pragma unroll
  for (int i = 0; i < kG; ++i) mxl = max(mxl, xev[i]);
  const int gmx = __builtin_amdgcn_readfirstlane(gmax8_i(mxl));
  if (gmx - c.Bm > kSpan || gmx - c.Bm < -kSpan) {
    c.Bm = gmx;
#pragma unroll
    for (int i = 0; i < kG; ++i)
      a[i] = ldexp(c.sm.xr[(par * kG + c.q) * kXS + i],
                   c.sm.er[(par * kG + c.q) * kES + i] - c.Bm);
  }
  if (PRED && step == c.nrun && c.lz_tail) {
    // log Z of the chain, in this chunk's frame: the sum of a over all labels
    // (only in the last block: an exit that the whole blocks cannot take would
    // keep the ring's old version alive through every step)
    double z = 0.0;
#pragma unroll
    for (int i = 0; i < kG; ++i) z += a[i];
    c.z_end = gsum8(z);
    c.done = step;
    c.ended = true;
    return;
  }
  // 4. the contraction into this lane's label: exp(m) = d 2^B
  double dp0 = 0.0, dp1 = 0.0;
#pragma unroll
  for (int i = 0; i < kG; i += 2) {
    dp0 = fma(a[i], c.Wt[i], dp0);
    dp1 = fma(a[i + 1], c.Wt[i + 1], dp1);
  }
  const double d = gsum8(dp0 + dp1);
  // 5. the new entry exp(m -+ S) / 2^R = d fy 2^(B -+ n - R), its rebase
  const int o = (buf * kPf + ipf) * kLab + c.cl;
  const double fy = c.sm.pfy[o];
  const int nq = c.isig * c.sm.pfn[o];
  const double y = d * fy;
  const int sh = c.Bm - nq - c.R;
  int n = 0;
  if (c.label) {
    const int ey = exponent_of(y) + sh;
    n = (ey > kRebase || ey < -kRebase) ? ey : 0;
    c.R += n;
  }
  const double e = c.label ? ldexp(y, sh - n) : 0.0;
  {  // the label's registers into the new reference (lanes that rebase)
    const unsigned long long m = __ballot(n != 0);
    rescale16(c.r, -n, m);
    rescale16(c.r + 16, -n, m);
  }
  c.r[H1] = c.q == 0 ? e : c.r[H1];  // the new entry: duration 1 of the next step
  if (c.q == 0) c.sm.rd[ipf * kLab + c.cl] = d;
  if (c.lane == 0) c.sm.rb[ipf] = c.Bm;
  c.done = step;
  if (ipf == kPf - 1 && next_blk) {  // the next block's scores, split
    double px, py;
    int pn;
    split64(c.pf_s, c.fwd, px, py, pn, c.sm.tab);
    const int po = ((buf ^ 1) * kPf + c.q) * kLab + c.cl;
    c.sm.pfx[po] = px;
    c.sm.pfy[po] = py;
    c.sm.pfn[po] = pn;
  }
  // 6. the next step's row: its K-sum (taken before the rebase: exact
  // power-of-two correction) plus the new entry's term, times exp(+-S)
  {
    const int o1 = (buf1 * kPf + ipf1) * kLab + c.cl;
    c.x = c.label ? (ldexp(gk, -n) + c.D1 * e) * c.sm.pfx[o1] : 0.0;
    c.E = c.R + c.isig * c.sm.pfn[o1];
  }
  if (ipf == kPf - 1 && c.rows) flush_rows(c);  // (the wave's own labels: no barrier)
}

template <bool PRED, int... Is>
__device__ __forceinline__ void block64(Sweep64 &c, int base, std::integer_sequence<int, Is...>) {
  (step64<Is, PRED>(c, base), ...);
}

}  // namespace

// One workgroup per (direction, sequence, chunk), as k_sweep (chain.hip):
// the same launch grid, start states, records ([K][C] ring by slot, then R,
// o, m), verification hand-off, log Z of the tail chunk and replay windows.
template <bool REP>
__global__ __launch_bounds__(kNT) void k_sweep64(ChainShape sh, const float *__restrict__ trans,
                                                 const float *__restrict__ dur, Escaled es,
                                                 const int32_t *__restrict__ lengths, PitBufs pb,
                                                 int iter) {
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

  Sweep64 c;
  c.sm = carve64(lds);
  if (tid < kTabN) c.sm.tab[tid] = kTab64[tid];
  c.S = es.S + ob;
  c.row1 = rows ? (fwd ? pb.row_a : pb.row_v) + orow : nullptr;  // alpha / v
  c.row2 = rows ? (fwd ? pb.row_u : pb.row_b) + orow : nullptr;  // u / beta
  c.T = T;
  c.C = C;
  c.K = K;
  c.w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  c.lane = tid & 63;
  c.cl = kG * c.w + (c.lane >> 3);  // this lane's label
  c.q = c.lane & (kG - 1);          // its duration block and input-label block
  c.isig = isig;
  c.rt0 = pb.row_t0;
  c.fwd = fwd;
  c.label = c.cl < C;
  const int cl = c.cl, q = c.q;
  const bool label = c.label;
  // per-lane constants: exp(dur) of this lane's durations; exp(trans) of its
  // 8 input labels 8q.. into cl (forward: previous label c' -> cl;
  // backward: cl -> next label c')
#pragma unroll
  for (int j = 0; j < kA; ++j) {
    const int k = kA * q + 1 + j;
    c.Dr[j] = (label && k <= K) ? exp((double)dur[(size_t)(k - 1) * C + cl]) : 0.0;
  }
  c.D1 = label ? exp((double)dur[cl]) : 0.0;
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    const int cp = kG * q + i;
    c.Wt[i] =
        (label && cp < C)
            ? exp((double)(fwd ? trans[(size_t)cp * C + cl] : trans[(size_t)cl * C + cp]))
            : 0.0;
  }
  __syncthreads();  // the table
  // valid ring registers of this lane
  const int nval = max(0, min(kA, K - kA * q));
  // stores the ring (head h) whose newest position is tref as a record, with
  // R, o, m: each register to the slot of its entry, so no register is
  // indexed at run time
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
          dl[(size_t)sl * C] = c.r[p];
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
          for (int j = 0; j < kA; ++j) c.r[j] = (q == 0 && j == 0) ? v : 0.0;
        } else {
          // neutral start: every entry of the window (positions inside [0, L]) is 1
  #pragma unroll
          for (int j = 0; j < kA; ++j) {
            const int pos = c.t0 - isig * (kA * q + j);
            c.r[j] = (label && kA * q + 1 + j <= K && pos >= 0 && pos <= L) ? 1.0 : 0.0;
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
                       ? rec_start[(size_t)pslot(c.t0 - isig * (k - 1), K) * C + cl] : 0.0;
        }
        c.R = label ? (int)rec_start[kc + cl] : 0;
        if (replay && rows && q == 0 && label &&
            (fwd ? jc == sh.rj0 : (jc == sh.rj0 + sh.rnb - 1 || p1 == L))) {
          c.row1[(size_t)(tstart - c.rt0) * C + cl] = rec_start[kc + C + cl];
          c.row2[(size_t)(tstart - c.rt0) * C + cl] = rec_start[kc + 2 * C + cl];
        }
      }
      {  // the first block's scores (later blocks: every lane, a block ahead)
        const int np = min(kPf, c.nrun) * kLab;
        for (int i = tid; i < np; i += kNT) {
          double fx, fy;
          int n;
          const int lab = i % kLab;
          const int tq = min(max(c.t0 + isig * (1 + i / kLab), 0), T);
          split64(c.S[(size_t)tq * C + (lab < C ? lab : 0)], fwd, fx, fy, n, c.sm.tab);
          c.sm.pfx[i] = fx;
          c.sm.pfy[i] = fy;
          c.sm.pfn[i] = n;
        }
      }
      vm_drain();
      __syncthreads();
      {  // the first step's row: K-sum over the whole start ring (its newest
         // entry included), times exp(+-S) of position 1
        double sa[4] = {0.0, 0.0, 0.0, 0.0};
  #pragma unroll
        for (int j = 0; j < kA; ++j) sa[j & 3] = fma(c.Dr[j], c.r[j], sa[j & 3]);
        const double g1 = gsum8((sa[0] + sa[1]) + (sa[2] + sa[3]));
        c.x = label ? g1 * c.sm.pfx[cl] : 0.0;
        c.E = c.R + isig * c.sm.pfn[cl];
      }
      // ---- the steps, in blocks of kA (the logs of the rows every kPf steps,
      // those of the record and log Z values after the loop)
      c.Bm = -(1 << 29);
      c.pf_s = 0.0;
      c.z_end = 0.0;
      c.done = c.flushed = 0;
      c.ended = false;
      const int nfull = (c.nrun - 1) / kA;  // whole blocks before the last step's
      for (int blk = 0; blk < nfull; ++blk)
        block64<false>(c, blk * kA, std::make_integer_sequence<int, kA>{});
      block64<true>(c, nfull * kA, std::make_integer_sequence<int, kA>{});
      if (c.rows) flush_rows(c);  // the rows of the last steps
      if (c.ended) {
        if (!replay && tid == 0) pb.lz_part[(fwd ? 0 : sh.B) + b] = log_t(c.z_end, c.Bm, c.sm.tab);
      } else {
        // the ring after the segment: its record (the last step's x, E, d,
        // staged by the label's lane 0 of this wave)
        const int il = (c.nrun - 1) % kPf;
        const double o = log_t(c.sm.rx[il * kLab + cl], c.sm.re[il * kLab + cl], c.sm.tab),
                     m = log_t(c.sm.rd[il * kLab + cl], c.Bm, c.sm.tab);
        const int h = (kA - c.nrun % kA) % kA;
        if (!main)
          save_ring(rec_start, c.t0 + isig * c.nrun, h, o, m);
        else if (!replay)
          save_ring(rec_end, c.t0 + isig * c.nrun, h, o, m);
      }
      // (the next segment's start rewrites the score buffers: wait for all)
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

size_t sweep64_lds_bytes(int K) {
  (void)K;  // the ring is in registers
  return kLdsBytes;
}

bool sweep64_applies(int C, int K) {
  return C > 32 && C <= kLab && K >= 1 && K <= kG * kA && sweep64_lds_bytes(K) <= kMaxDynLds;
}

hipError_t launch_sweep_64(const ChainShape &sh, const float *trans, const float *dur,
                           const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                           int with_bwd, int iter, hipStream_t st) {
  const size_t lds = sweep64_lds_bytes(sh.K);
  const bool rep = iter == kPitRepair;
  const void *f = rep ? (const void *)k_sweep64<true> : (const void *)k_sweep64<false>;
  if (!sweep64_applies(sh.C, sh.K) || !lds_fits(f, lds)) return hipErrorInvalidConfiguration;
  const int nd = with_bwd ? 2 : 1;
  if (rep) {
    hipLaunchKernelGGL(k_sweep64<true>, dim3(nd * sh.B), dim3(kNT), lds, st, sh, trans, dur, es,
                       lengths, pb, iter);
  } else {
    const int grid = iter < 0 ? sh.B * (sh.rnf + sh.rnb) : nd * sh.B * sh.nchunk;
    hipLaunchKernelGGL(k_sweep64<false>, dim3(grid), dim3(kNT), lds, st, sh, trans, dur, es,
                       lengths, pb, iter);
  }
  return hipGetLastError();
}

}  // namespace semicrf
