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
// bandwidth alone); here it lives in the register file instead:
//   * 8 waves, lane = label c (labels padded to 64 with zero weights).  Wave
//     w owns durations k = 32w + 1 .. 32w + 32 of label `lane`: 32 float64
//     registers form a circular buffer, the entry of duration 32w + 1 + j in
//     register (h + j) mod 32, next to the weights exp(dur[k-1][c]).  A
//     step moves the head h back by one and overwrites the register that
//     held the oldest entry -- no register moves.  The step loop runs in
//     blocks of 32 steps whose bodies are instantiated for their place in
//     the block (a template), so the head and every ring register index are
//     compile-time constants; the steps are predicated, so a block's control
//     flow is a plain sequence.  The entry leaving wave w (duration 32w + 32)
//     enters wave w + 1 through a one-row hand-off in LDS.
//   * one barrier per step, software-pipelined: the interval between two
//     barriers holds, in every wave, (1) the previous step's entry from the
//     contraction partials -- its d, rebase and entry, computed redundantly
//     and bit-identically in all waves; (2) this step's row from the K-sum
//     partials: x, the step scale, a; (3) this wave's share of the C x C
//     contraction (8 input labels 8w..8w+7 read from its own lanes, exp(trans)
//     from LDS); (4) its K-sum partial of the next step (32 multiply-adds on
//     registers).  So the K-sum of step t+1 runs beside the contraction of
//     step t; only wave 0's newest term, duration 1, waits for the entry of
//     step t and is added in the next interval.
//   * a rebase (R[c] += n) is known to every wave in the interval after the
//     step that makes it: the partials computed before it are corrected
//     exactly (2^-n), and each wave rescales its registers and the hand-off
//     entry by 2^-n.
//   * rows: wave w keeps the raw values (x, E, d, B) of the steps s with
//     s - 1 = w (mod 8) in registers; every 8 steps all waves take their
//     logarithms and store them together.
//   * registers: the 32 ring entries and 32 weights take 128 of the 256
//     registers a wave has at 512 threads; exp(trans) and the constants of the
//     logarithm and of the score split live in LDS, read where they are used
//     (kept as literals, the compiler holds them in registers across the loop
//     and the ring spills).
//   * a chunk with a burn-in runs it as a first segment of the same loop; its
//     end state is the chunk's start record, from which the chunk's own
//     positions run as the second segment.
#include <stdio.h>
#include <stdlib.h>

#include <utility>

#include "device_math.h"
#include "internal.h"

namespace semicrf {

namespace {

constexpr int kW = 8;                 // waves
constexpr int kA = 32;                // durations per wave
constexpr int kNT = 64 * kW;
constexpr int kLanes = 64;            // labels padded to a wave
constexpr int kPf = kW;               // positions per score-prefetch block (one per wave)
constexpr int kRebase = 512;          // rebase bound, log2 units (as chain.hip)
constexpr int kSpan = 256;            // step-scale span, log2 units (as chain.hip)

// Constants of the exponential split and of the logarithm, kept in LDS and
// read where they are used: as literals the compiler keeps them in registers
// across the whole step loop, where the ring needs every register.
constexpr int kTabN = 32;
__constant__ double kTab64[kTabN] = {
    1.4426950408889634074,  // 0: log2 e
    0.69314718055994530942, // 1: ln 2
    2.3190468138462996e-17, // 2: ln 2 minus its float64 rounding
    1.0 / 87178291200.0,    // 3: 1/14!
    1.0 / 479001600.0,      // 4: 1/12!
    1.0 / 3628800.0,        // 5: 1/10!
    1.0 / 40320.0,          // 6: 1/8!
    1.0 / 720.0,            // 7: 1/6!
    1.0 / 24.0,             // 8: 1/4!
    1.0 / 6227020800.0,     // 9: 1/13!
    1.0 / 39916800.0,       // 10: 1/11!
    1.0 / 362880.0,         // 11: 1/9!
    1.0 / 5040.0,           // 12: 1/7!
    1.0 / 120.0,            // 13: 1/5!
    1.0 / 6.0,              // 14: 1/3!
    1e9,                    // 15: bound of the split's argument
    // 16..27: 1/(2k+1), k = 0..11 (the series of atanh)
    1.0, 1.0 / 3.0, 1.0 / 5.0, 1.0 / 7.0, 1.0 / 9.0, 1.0 / 11.0, 1.0 / 13.0, 1.0 / 15.0,
    1.0 / 17.0, 1.0 / 19.0, 1.0 / 21.0, 1.0 / 23.0,
    0.70710678118654752440,  // 28: sqrt(1/2)
    0.0, 0.0, 0.0};

struct S64 {
  double *part;      // [2][kW][64]: K-sum partials of a step, by the step's parity
  double *dotp;      // [2][kW][64]: contraction partials
  double *hand;      // [2][kW][64]: each wave's oldest entry, for the next wave
  double *pfx, *pfy; // [2][kPf][64] split scores
  int *pfn;          // [2][kPf][64]
  double *tab;       // [kTabN]: kTab64
  double *wtr;       // [kW][kW][64]: exp(trans) of wave w's 8 input labels, per output label
};

constexpr size_t kRowBytes = (size_t)2 * kW * kLanes * 8;

__device__ __forceinline__ S64 carve64(unsigned char *base) {
  S64 m;
  size_t off = 0;
  m.part = reinterpret_cast<double *>(base + off); off += kRowBytes;
  m.dotp = reinterpret_cast<double *>(base + off); off += kRowBytes;
  m.hand = reinterpret_cast<double *>(base + off); off += kRowBytes;
  m.pfx = reinterpret_cast<double *>(base + off); off += (size_t)2 * kPf * kLanes * 8;
  m.pfy = reinterpret_cast<double *>(base + off); off += (size_t)2 * kPf * kLanes * 8;
  m.pfn = reinterpret_cast<int *>(base + off); off += (size_t)2 * kPf * kLanes * 4;
  m.tab = reinterpret_cast<double *>(base + off); off += (size_t)kTabN * 8;
  m.wtr = reinterpret_cast<double *>(base + off);
  return m;
}

__device__ __forceinline__ int pslot(int pos, int K) {
  const int s = pos % K;
  return s < 0 ? s + K : s;
}

// Score of position t, label c (clamped into [0, T]; lanes past C read
// label 0), split in the order the direction uses it.
__device__ __forceinline__ double raw64(const Escaled &es, size_t ob, int t, int T, int C, int c) {
  const int tc = t < 0 ? 0 : (t > T ? T : t);
  return es.S[ob + (size_t)tc * C + (c < C ? c : 0)];
}

// exp(s) = ep 2^n and exp(-s) = em 2^-n, ep, em in [2^-1/2, 2^1/2]: the same
// reduction and series as exp_split (device_math.h), term for term, with
// the constants read from the table.
__device__ __forceinline__ void exp_split_t(double s, double &ep, double &em, int &n,
                                            const double *__restrict__ tab) {
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
__device__ __forceinline__ double log_t(double x, int E, const double *__restrict__ tab) {
  if (!(x > 0.0 && x < __builtin_huge_val())) return x == 0.0 ? -__builtin_huge_val() : __builtin_nan("");
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
                                        const double *__restrict__ tab) {
  double ep, em;
  exp_split_t(s, ep, em, n, tab);
  fx = fwd ? ep : em;
  fy = fwd ? em : ep;
}

// Everything one wave carries through a segment of the sweep: constants,
// the ring registers and the loop state (one object, split into registers
// once the step bodies are inlined).
struct Sweep64 {
  S64 sm;
  const double *S;  // cumulative scores of this sequence
  double *row1, *row2;
  int T, C, K, w, lane, isig, t0, nrun, rt0;
  bool fwd, label, has_dur, rows, lz_tail;
  double Dr[kA], D1;
  // ring: register (h + j) mod kA = entry of duration 32w + 1 + j, h = -(steps done) mod kA
  double r[kA];
  double e_first;  // the start state's newest entry
  int R, Bm;
  double x_p, fy_p;  // the previous step's x and exp(-+S) mantissa
  int E_p, nq_p, B_p;
  double pf_s;
  double r_x, r_d;  // this wave's pending row
  int r_t, r_E, r_B, r_mode;
  double z_end;
  bool ended;
};

__device__ __forceinline__ void flush_row(Sweep64 &c) {
  if (c.r_mode != 0 && c.label) {
    const size_t tr = (size_t)(c.r_t - c.rt0) * c.C + c.lane;
    c.row1[tr] = log_t(c.r_x, c.r_E, c.sm.tab);
    if (c.r_mode == 2) c.row2[tr] = log_t(c.r_d, c.r_B, c.sm.tab);
  }
  c.r_mode = 0;
}

// The entry of the step before (its contraction partials at parity `par`,
// bit-identical in every wave): d, the rebase n (R moves by it) and the
// entry e = exp(m -+ S) / 2^R = d * fy * 2^(B -+ n - R).
__device__ __forceinline__ void prev_entry(Sweep64 &c, int par, double &e, int &n, double &d) {
  d = 0.0;
#pragma unroll
  for (int q = 0; q < kW; ++q) d += c.sm.dotp[(par * kW + q) * kLanes + c.lane];
  const double y = d * c.fy_p;
  const int sh = c.B_p - c.nq_p - c.R;
  n = 0;
  if (c.label) {
    const int ey = exponent_of(y) + sh;
    n = (ey > kRebase || ey < -kRebase) ? ey : 0;
    c.R += n;
  }
  e = c.label ? ldexp(y, sh - n) : 0.0;
}

__device__ __forceinline__ void rebase_ring(Sweep64 &c, int n) {
  if (c.has_dur && __any(n != 0)) {
#pragma unroll
    for (int j = 0; j < kA; ++j) c.r[j] = ldexp(c.r[j], -n);
  }
}

// Step base + I + 1 of the segment (nothing past the segment's end or its
// last step).  I is the step's place in a block of kA steps, so the ring
// head (-I mod kA), the prefetch slot and every LDS parity are compile-time
// constants.  The steps are predicated, not left early: a block has no exit
// but its end, which keeps its control flow a plain sequence.
template <int I>
__device__ __forceinline__ void step64(Sweep64 &c, int base) {
  const int step = base + I + 1;
  if (step > c.nrun || c.ended) return;
  constexpr int ipf = I % kPf, buf = (I / kPf) & 1;
  constexpr int par = (I + 1) & 1;            // parity of this step
  constexpr int H = (kA - I) % kA;            // head of this step's ring
  constexpr int H1 = (H + kA - 1) % kA;       // head of the next step's
  const int t = c.t0 + c.isig * step;
  const bool next_blk = step - 1 - ipf + kPf < c.nrun;
  if (ipf == 0 && next_blk)  // wave w loads position w of the next block
    c.pf_s = c.S[(size_t)min(max(c.t0 + c.isig * (step + kPf + c.w), 0), c.T) * c.C +
                 (c.label ? c.lane : 0)];
  const int o = (buf * kPf + ipf) * kLanes + c.lane;
  const double fx = c.sm.pfx[o], fy = c.sm.pfy[o];
  const int nq = c.isig * c.sm.pfn[o];
  double psum = 0.0;
#pragma unroll
  for (int q = 0; q < kW; ++q) psum += c.sm.part[(par * kW + q) * kLanes + c.lane];
  // 1. the previous step's entry and rebase
  double e = c.e_first, d = 0.0;
  int n = 0;
  if (step > 1) {
    prev_entry(c, par ^ 1, e, n, d);
    if (c.rows && (I + kW - 1) % kW == c.w) {  // the row of the step before
      c.r_t = t - c.isig;
      c.r_x = c.x_p;
      c.r_E = c.E_p;
      c.r_d = d;
      c.r_B = c.B_p;
      c.r_mode = 2;
    }
  }
  rebase_ring(c, n);
  // 2. this step's row (every wave alike)
  const double x = (ldexp(psum, -n) + c.D1 * e) * fx;
  const int E = c.R + nq;
  const int ex = (c.label && x > 0.0) ? E + exponent_of(x) : kNoExp;
  if (__any(ex - c.Bm > kSpan) || !__any(ex - c.Bm >= -kSpan)) c.Bm = wave_max_i(ex);
  const double a = ldexp(x, E - c.Bm);  // exp(o) / 2^Bm
  c.x_p = x;
  c.E_p = E;
  c.B_p = c.Bm;
  if (step == c.nrun && c.lz_tail) {
    // log Z of the chain, in this chunk's frame: sum of a (fixed-order butterfly)
    double z = c.label ? a : 0.0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    c.z_end = z;
    if (ipf == 0 && step > 1) flush_row(c);  // (the flush this step would make)
    if (c.rows && ipf == c.w) {              // alpha / v of the last position
      c.r_t = t;
      c.r_x = x;
      c.r_E = E;
      c.r_mode = 1;
    }
    c.ended = true;
    return;
  }
  // 3. this wave's share of the contraction
  {
    const int lo = __double2loint(a), hi = __double2hiint(a);
    double dp0 = 0.0, dp1 = 0.0;
#pragma unroll
    for (int q = 0; q < kW; q += 2) {
      const int l0 = kW * c.w + q;
      const double a0 = __hiloint2double(__builtin_amdgcn_readlane(hi, l0),
                                         __builtin_amdgcn_readlane(lo, l0));
      const double a1 = __hiloint2double(__builtin_amdgcn_readlane(hi, l0 + 1),
                                         __builtin_amdgcn_readlane(lo, l0 + 1));
      const double *wq = c.sm.wtr + (c.w * kW + q) * kLanes + c.lane;
      dp0 = fma(a0, wq[0], dp0);
      dp1 = fma(a1, wq[kLanes], dp1);
    }
    c.sm.dotp[(par * kW + c.w) * kLanes + c.lane] = dp0 + dp1;
  }
  // 4. the ring of the next step: wave 0 completes this step's ring with e
  // (duration 1, register H); the head moves to H1, whose register (the
  // oldest entry, which leaves) takes the entry handed over by the wave
  // before (wave 0: 0 -- the coming entry is added apart); this wave's K-sum
  // partial of the next step
  double ks = 0.0;
  if (c.has_dur) {
    double hv = 0.0;
    if (c.w > 0) hv = ldexp(c.sm.hand[(par * kW + c.w - 1) * kLanes + c.lane], -n);
    if (c.w == 0) c.r[H] = e;
    c.r[H1] = hv;
    double sa[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < kA; ++j) sa[j & 3] = fma(c.Dr[j], c.r[(H1 + j) % kA], sa[j & 3]);
    ks = (sa[0] + sa[1]) + (sa[2] + sa[3]);
    c.sm.hand[((par ^ 1) * kW + c.w) * kLanes + c.lane] = c.r[(H1 + kA - 1) % kA];
  }
  c.sm.part[((par ^ 1) * kW + c.w) * kLanes + c.lane] = ks;
  if (ipf == kPf - 1 && next_blk) {  // the next block's scores, split
    double px, py;
    int pn;
    split64(c.pf_s, c.fwd, px, py, pn, c.sm.tab);
    const int po = ((buf ^ 1) * kPf + c.w) * kLanes + c.lane;
    c.sm.pfx[po] = px;
    c.sm.pfy[po] = py;
    c.sm.pfn[po] = pn;
  }
  c.fy_p = fy;
  c.nq_p = nq;
  if (ipf == 0 && step > 1) flush_row(c);  // every wave holds one row here
  __syncthreads();
}

template <int... Is>
__device__ __forceinline__ void block64(Sweep64 &c, int base, std::integer_sequence<int, Is...>) {
  (step64<Is>(c, base), ...);
}

}  // namespace

// One workgroup per (direction, sequence, chunk), as k_sweep (chain.hip):
// the same launch grid, start states, records ([K][C] ring by slot, then R,
// o, m), verification hand-off, log Z of the tail chunk and replay windows.
// A chunk with a burn-in runs it as a first segment of the same loop, whose
// end state is the chunk's start record; the chunk's own positions follow
// from that record.
__global__ __launch_bounds__(kNT) void k_sweep64(ChainShape sh, const float *__restrict__ trans,
                                                 const float *__restrict__ dur, Escaled es,
                                                 const int32_t *__restrict__ lengths, PitBufs pb,
                                                 int iter) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int nck = sh.B * sh.nchunk;
  const bool replay = iter < 0;
  bool fwd;
  int b, jc;
  if (replay) {
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
  const size_t idx = (fwd ? 0 : (size_t)nck) + (size_t)b * sh.nchunk + jc;
  if (iter == 0) {  // the parallel-in-time state, before any verification reads it
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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // w: wave-uniform
  const bool label = lane < C;
  if (L < 1 || L > T || jc >= sh.nchunk) return;
  const int p0 = jc * sh.delta;
  if (p0 >= L) return;
  const int p1 = min(p0 + sh.delta, L);
  if (iter > 0 && (pb.nbad[iter - 1] == 0 || pb.redo[idx] == 0)) return;
  const size_t ob = (size_t)b * (T + 1) * C;
  const size_t cks = ck_stride(C, K);
  const size_t kc = (size_t)K * C;
  double *rec_start = (fwd ? pb.ck_fwd : pb.ck_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  double *rec_end = (fwd ? pb.end_fwd : pb.end_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  const int isig = fwd ? 1 : -1;
  const int tstart = fwd ? p0 : p1;
  const bool tail = fwd ? (p1 == L) : (p0 == 0);
  const bool rows = pb.row_a != nullptr;
  const size_t orow = (size_t)b * pb.row_stride * C;
  const int s_dur0 = kA * w + 1;  // this wave's first duration

  Sweep64 c;
  c.sm = carve64(lds);
  if (tid < kTabN) c.sm.tab[tid] = kTab64[tid];
  __syncthreads();
  c.S = es.S + ob;
  c.row1 = rows ? (fwd ? pb.row_a : pb.row_v) + orow : nullptr;  // alpha / v
  c.row2 = rows ? (fwd ? pb.row_u : pb.row_b) + orow : nullptr;  // u / beta
  c.T = T;
  c.C = C;
  c.K = K;
  c.w = w;
  c.lane = lane;
  c.isig = isig;
  c.rt0 = pb.row_t0;
  c.fwd = fwd;
  c.label = label;
  c.has_dur = s_dur0 <= K;
  // per-lane constants: exp(dur) of this wave's durations in registers
  // (wave 0's duration 1 apart in D1, which every wave holds: the row is
  // formed in all of them); exp(trans) of this wave's 8 input labels
  // (forward: previous label c' -> c; backward: c -> next label c') in LDS
#pragma unroll
  for (int j = 0; j < kA; ++j) {
    const int k = s_dur0 + j;
    c.Dr[j] = (label && k <= K && k > 1) ? exp((double)dur[(size_t)(k - 1) * C + lane]) : 0.0;
  }
  c.D1 = label ? exp((double)dur[lane]) : 0.0;
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    const int cp = kW * w + i;
    c.sm.wtr[(w * kW + i) * kLanes + lane] =
        (label && cp < C)
            ? exp((double)(fwd ? trans[(size_t)cp * C + lane] : trans[(size_t)lane * C + cp]))
            : 0.0;
  }
  // valid ring registers of this wave (wave-uniform)
  const int nval = __builtin_amdgcn_readfirstlane(max(0, min(kA, K - s_dur0 + 1)));
  // stores the ring (head h; wave 0's newest entry e, not yet in its
  // register) whose newest position is tref as a record, with R, o, m: each
  // register to the slot of its entry, so no register is indexed at run time
  auto save_ring = [&](double *__restrict__ dst, int tref, int h, double e, double o, double m) {
    if (label) {
      const int s_first = pslot(tref - isig * (s_dur0 - 1), K);
      double *dl = dst + lane;
#pragma unroll
      for (int p = 0; p < kA; ++p) {
        const int j = (p - h) & (kA - 1);  // the register's entry: duration s_dur0 + j
        if (j < nval) {
          int sl = s_first - isig * j;
          sl += sl < 0 ? K : 0;
          sl -= sl >= K ? K : 0;
          dl[(size_t)sl * C] = (w == 0 && j == 0) ? e : c.r[p];
        }
      }
      if (w == 0) {
        dst[kc + lane] = (double)c.R;
        dst[kc + C + lane] = o;
        dst[kc + 2 * C + lane] = m;
      }
    }
  };

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
          exp_split_t(c.S[(size_t)L * C + (label ? lane : 0)], v, em, c.R, c.sm.tab);
        }
        if (!label) {
          c.R = 0;
          v = 0.0;
        }
#pragma unroll
        for (int j = 0; j < kA; ++j) c.r[j] = (w == 0 && j == 0) ? v : 0.0;
        c.e_first = v;
      } else {
        // neutral start: every entry of the window (positions inside [0, L]) is 1
#pragma unroll
        for (int j = 0; j < kA; ++j) {
          const int q = c.t0 - isig * (s_dur0 - 1 + j);
          c.r[j] = (label && s_dur0 + j <= K && q >= 0 && q <= L) ? 1.0 : 0.0;
        }
        c.e_first = label ? 1.0 : 0.0;
      }
      if (main) {
        save_ring(rec_start, c.t0, 0, c.e_first, exact ? -__builtin_huge_val() : __builtin_nan(""),
                  exact ? 0.0 : __builtin_nan(""));
        if (exact && w == 0 && label && rows)  // u[0] = 0 forward, beta[L] = 0 backward
          c.row2[(size_t)(tstart - c.rt0) * C + lane] = 0.0;
      }
    } else {
      // the chunk's start record (written by the burn-in segment just now, or
      // by an earlier sweep); each wave reads back the slots it wrote itself
      if (wb > 0) {
        __threadfence_block();
        __syncthreads();
      }
#pragma unroll
      for (int j = 0; j < kA; ++j) {
        const int k = s_dur0 + j;
        c.r[j] = (label && k <= K) ? rec_start[(size_t)pslot(c.t0 - isig * (k - 1), K) * C + lane]
                                   : 0.0;
      }
      c.e_first = label ? rec_start[(size_t)pslot(c.t0, K) * C + lane] : 0.0;
      c.R = label ? (int)rec_start[kc + lane] : 0;
      if (replay && rows && w == 0 && label &&
          (fwd ? jc == sh.rj0 : (jc == sh.rj0 + sh.rnb - 1 || p1 == L))) {
        c.row1[(size_t)(tstart - c.rt0) * C + lane] = rec_start[kc + C + lane];
        c.row2[(size_t)(tstart - c.rt0) * C + lane] = rec_start[kc + 2 * C + lane];
      }
    }
    {  // the first block's scores (later blocks: the waves, a block ahead)
      const int np = min(kPf, c.nrun) * kLanes;
      for (int q = tid; q < np; q += kNT) {
        double fx, fy;
        int n;
        const int tq = min(max(c.t0 + isig * (1 + q / kLanes), 0), T);
        split64(c.S[(size_t)tq * C + (q % kLanes < C ? q % kLanes : 0)], fwd, fx, fy, n, c.sm.tab);
        c.sm.pfx[q] = fx;
        c.sm.pfy[q] = fy;
        c.sm.pfn[q] = n;
      }
    }
    {  // the K-sum partials of step 1 and the hand-off entries
      double sa[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < kA; ++j) sa[j & 3] = fma(c.Dr[j], c.r[j], sa[j & 3]);
      c.sm.part[(1 * kW + w) * kLanes + lane] = c.has_dur ? (sa[0] + sa[1]) + (sa[2] + sa[3]) : 0.0;
      c.sm.hand[(1 * kW + w) * kLanes + lane] = c.r[kA - 1];
    }
    vm_drain();
    __syncthreads();
    // ---- the steps, in blocks of kA (the logs of the rows every kW steps,
    // those of the record and log Z values after the loop)
    c.Bm = -(1 << 29);
    c.x_p = c.fy_p = 0.0;
    c.E_p = c.nq_p = c.B_p = 0;
    c.pf_s = 0.0;
    c.r_x = c.r_d = 0.0;
    c.r_t = c.r_E = c.r_B = c.r_mode = 0;
    c.z_end = 0.0;
    c.ended = false;
    for (int base = 0; base < c.nrun && !c.ended; base += kA)
      block64(c, base, std::make_integer_sequence<int, kA>{});
    if (c.ended) {
      flush_row(c);
      if (!replay && tid == 0)
        pb.lz_part[(fwd ? 0 : sh.B) + b] = log_t(c.z_end, c.B_p, c.sm.tab);
    } else {
      // the last step's entry: the ring after the segment, its record
      double e, d;
      int n;
      prev_entry(c, c.nrun & 1, e, n, d);
      if (c.rows && (c.nrun - 1) % kW == w) {
        c.r_t = c.t0 + isig * c.nrun;
        c.r_x = c.x_p;
        c.r_E = c.E_p;
        c.r_d = d;
        c.r_B = c.B_p;
        c.r_mode = 2;
      }
      flush_row(c);
      rebase_ring(c, n);
      const double o = log_t(c.x_p, c.E_p, c.sm.tab), m = log_t(d, c.B_p, c.sm.tab);
      const int h = (kA - c.nrun % kA) % kA;
      if (!main)
        save_ring(rec_start, c.t0 + isig * c.nrun, h, e, o, m);
      else if (!replay)
        save_ring(rec_end, c.t0 + isig * c.nrun, h, e, o, m);
    }
  }
}

size_t sweep64_lds_bytes(int K) {
  (void)K;  // the ring is in registers
  return 3 * kRowBytes + (size_t)2 * kPf * kLanes * 16 + (size_t)2 * kPf * kLanes * 4 +
         (size_t)kTabN * 8 + (size_t)kW * kW * kLanes * 8;
}

bool sweep64_applies(int C, int K) {
  return C > 32 && C <= kLanes && K >= 1 && K <= kW * kA && sweep64_lds_bytes(K) <= kMaxDynLds;
}

hipError_t launch_sweep_64(const ChainShape &sh, const float *trans, const float *dur,
                           const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                           int with_bwd, int iter, hipStream_t st) {
  const size_t lds = sweep64_lds_bytes(sh.K);
  if (!sweep64_applies(sh.C, sh.K) || !lds_fits((const void *)k_sweep64, lds))
    return hipErrorInvalidConfiguration;
  const int grid = iter < 0 ? sh.B * (sh.rnf + sh.rnb) : (with_bwd ? 2 : 1) * sh.B * sh.nchunk;
  hipLaunchKernelGGL(k_sweep64, dim3(grid), dim3(kNT), lds, st, sh, trans, dur, es, lengths, pb,
                     iter);
  return hipGetLastError();
}

}  // namespace semicrf
