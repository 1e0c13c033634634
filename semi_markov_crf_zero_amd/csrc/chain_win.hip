// chain_win.hip -- blocked streaming engine for C <= 32 labels.
//
// Same recurrences, ring contents, checkpoint records and outputs as
// chain.hip (see its header for the equations, the exp-space arithmetic and
// the method citations); this file reorganises the work so that nothing but
// the dependent chain itself runs position by position:
//
//   * blocks of U positions.  The K-sum of step i of a block (position t)
//       sum_{k=1..K} D[k][c] * G[t - sigma*k][c]
//     splits at k = 2U: the "near" terms k < 2U are the 2U-1 newest entries,
//     which the chain wave keeps in a register window that rolls across
//     blocks; the "far" terms k >= 2U read only entries produced before the
//     previous block began.  So while the chain runs block n, the helper
//     waves 1-3 compute the far parts of block n+1 for its U steps at once:
//     thread (g, c) owns the durations k = a0 .. a0+A-1 (a0 >= 2U) of label
//     c, holds their weights exp(dur) in registers for the whole sweep, fills
//     a register window with the entries (consecutive positions, read across
//     the ring's wrap from its mirror copy of the first slots) and
//     accumulates U sums -- U*A fused multiply-adds with full
//     instruction-level parallelism.  Only the ring and small block buffers
//     live in LDS, so two workgroups share a compute unit up to K*C of about
//     8800 (C = 16 with K = 512) and hide each other's step latency.
//     Partials are reduced inside each wave (DPP) and land in the other of
//     two LDS buffers.  One workgroup barrier per block.
//   * the "chain wave" (wave 0, lane c = label c) runs the block's U steps
//     alone, with wave-local synchronisation only: the near part (one fused
//     multiply-add on the dependent chain, the rest summed a step ahead),
//     the product with exp(+-S), the integer maximum of the float64
//     exponents, the C x C contraction (each label's sum shared by two or
//     four lanes, exp(trans) in registers, the e row through LDS), the new
//     entry straight into the ring and its rebase decision; the block's U
//     steps are unrolled.  A rebase (R += n) rescales the register window at once and
//     reaches the far parts -- computed in the reference the labels had when
//     the previous block began -- as an exact ldexp when they are read.
//   * at the block end, if a label rebased, all threads rescale its older
//     ring entries (rare; label by label).
//   * besides the far parts, wave 1 prefetches the split scores of the next
//     block into LDS (loads issued first, stored last) and waves 2-3 turn
//     the previous block's staged values into the per-position log rows: no
//     global-memory access and no logarithm on the chain.
#include <stdio.h>
#include <stdlib.h>

#include "device_math.h"
#include "internal.h"
#include "pitcheck.h"

namespace semicrf {

namespace {

constexpr int kRebaseExp = 512;  // rebase bound, log2 units (see chain.hip)
constexpr int U = kWinU;         // positions per block
constexpr int kNearW = 2 * U - 1;  // near terms k = 1 .. 2U-1 (the chain's register window)

struct WSmem {
  double *ring, *part, *stg, *erow;
  double *efx, *efy;  // split scores of two blocks [2][U][C]
  int *shiftn, *flag, *en;
};

// Contraction width: C padded to the instance bound 8, 16 or 32.
__host__ __device__ __forceinline__ int cpad(int c) { return c <= 8 ? 8 : (c <= 16 ? 16 : 32); }

// Far-part partials are pre-reduced inside each wave: one partial per helper
// wave (all but the chain wave) and label.
__device__ __forceinline__ int part_groups(const ChainShape &sh, int NT) {
  (void)sh;
  return NT / 64 - 1;
}

// Carve-up; the byte count is win_lds_bytes() in internal.h.
__device__ __forceinline__ WSmem wcarve(unsigned char *base, const ChainShape &s, int NT) {
  WSmem m;
  size_t off = 0;
  const int C4 = cpad(s.C);
  m.ring = reinterpret_cast<double *>(base + off); off += (size_t)(s.K + kWinMirror) * s.C * 8;
  m.part = reinterpret_cast<double *>(base + off);
  off += (size_t)2 * U * part_groups(s, NT) * s.C * 8;  // [2][U][G][C]
  m.stg = reinterpret_cast<double *>(base + off); off += (size_t)2 * U * (3 * s.C + 1) * 8;
  off = (off + 15) & ~(size_t)15;
  m.erow = reinterpret_cast<double *>(base + off); off += (size_t)C4 * 8;
  m.shiftn = reinterpret_cast<int *>(base + off); off += (size_t)s.C * 4;
  m.flag = reinterpret_cast<int *>(base + off); off += 2 * 4;
  off = (off + 15) & ~(size_t)15;
  m.efx = reinterpret_cast<double *>(base + off); off += (size_t)2 * U * s.C * 8;
  m.efy = reinterpret_cast<double *>(base + off); off += (size_t)2 * U * s.C * 8;
  m.en = reinterpret_cast<int *>(base + off);
  return m;
}

__device__ __forceinline__ int pos_slot(int pos, int K) {
  int s = pos % K;
  return s < 0 ? s + K : s;
}

// Store ring slot `slot` of label c, and its mirror copy at slot + K for
// the slots below kWinMirror (read by the far loop across the wrap).
__device__ __forceinline__ void ring_put(const WSmem &sm, int K, int C, int slot, int c,
                                         double v) {
  sm.ring[slot * C + c] = v;
  if (slot < kWinMirror) sm.ring[(slot + K) * C + c] = v;
}

// The contraction of a label is split over kSplit lanes of wave 0: lane l
// takes label c = l % CMAX and the previous labels c' of part
// h = (l / CMAX) % kSplit, c' = h*CMAX/kSplit + j; lane_swap_add joins the
// parts (lanes CMAX, 2*CMAX apart).  Fewer multiply-adds, LDS reads and
// weight registers per lane on the dependent chain, for two or three
// cross-lane adds.
template <int CMAX>
constexpr int kSplit = CMAX >= 32 ? 2 : 4;
static_assert(32 * kSplit<32> <= 64 && 16 * kSplit<16> <= 64, "parts fit one wave");

// exp(trans) weights of lane `lane` of wave 0 for the contraction of
// direction fwd (float64, for the same reason): tr[j] = weight of input
// label c' = h*CMAX/kSplit + j for output label c, zero past C.
template <int CMAX>
__device__ __forceinline__ void load_tr_row(const ChainShape &sh, const float *__restrict__ trans,
                                            bool fwd, int lane, double *tr) {
  constexpr int NJ = CMAX / kSplit<CMAX>;
  const int C = sh.C, c = lane % CMAX, h = (lane / CMAX) % kSplit<CMAX>;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int ci = h * NJ + j;
    tr[j] = (c < C && ci < C)
                ? exp((double)(fwd ? trans[(size_t)ci * C + c] : trans[(size_t)c * C + ci]))
                : 0.0;
  }
}

// Sum of a float64 over aligned groups of gw consecutive lanes (gw a power of
// two, 2 <= gw <= 16) by DPP quad permutes and row mirrors (dpp_f64); every
// lane of a group receives the group sum.

__device__ __forceinline__ double group_sum(double v, int gw) {
  v += dpp_f64(v, 0xB1);               // quad_perm [1,0,3,2]: lane ^ 1
  if (gw >= 4) v += dpp_f64(v, 0x4E);  // quad_perm [2,3,0,1]: lane ^ 2
  if (gw >= 8) v += dpp_f64(v, 0x141); // row_half_mirror: the other quad of 8
  if (gw >= 16) v += dpp_f64(v, 0x140);  // row_mirror: the other half of 16
  return v;
}

// Far parts of the K-sums of a block: helper thread (kg, kc) owns the
// durations k = a0 + j, j < nage, of label kc, all k >= 2U (A of them per
// group of wave 1, A2 per group of the row-writing waves 2..).  Labels take cp
// lanes of a wave (C rounded up to a power of two; lanes past C idle), so
// the gw = 64/cp duration groups of one label in a wave are consecutive
// lanes and their partials add up by DPP.
template <int DCH, int CMAX>
struct Win {
  // duration chunks a helper thread holds: A <= DCH * NCH (win_config)
  static constexpr int NCH = DCH == 8 ? kWinFarChunks : 1;
  // the chain wave's weights in the same registers: exp(dur) of the near
  // durations (Dn[k], k = 0 .. 2U-1) and its lane's exp(trans) part
  static constexpr int NCHAIN = kNearW + 1 + CMAX / kSplit<CMAX>;
  static constexpr int NW = DCH * NCH > NCHAIN ? DCH * NCH : NCHAIN;
  int kc, kg, a0, nage, gw;
  bool on;
  // helper waves: exp(dur) of this thread's durations a0 .. a0 + nage - 1, 0
  // past them, in float64 (a rounded weight would perturb the parameters,
  // and the parameter gradients move by that times a sensitivity that grows
  // with the sequence length); held for the whole sweep.  Wave 0 keeps its
  // own weights here instead (the two roles never share a wave, and one
  // array keeps the register count of both within two workgroups per
  // compute unit).
  double wd[NW];

  __device__ __forceinline__ void init(const ChainShape &sh, const float *__restrict__ dur) {
    const int C = sh.C, tid = threadIdx.x, w = tid >> 6;
    int cp = 1;
    while (cp < C) cp *= 2;
    gw = 64 / cp;
    kc = (tid & 63) / gw;
    kg = (w - 1) * gw + (tid & 63) % gw;  // helper waves 1.. only
    on = w >= 1 && kc < C && kg < sh.P;
    // wave 1's groups hold A durations each, those of waves 2.. A2
    const int cap = kg < gw ? sh.A : sh.A2;
    a0 = kNearW + 1 + (kg < gw ? kg * sh.A : gw * sh.A + (kg - gw) * sh.A2);
    int n = on ? sh.K - a0 + 1 : 0;
    n = n < 0 ? 0 : (n > cap ? cap : n);
    nage = n;
    float v[NW];  // all loads in flight before the first exponential
#pragma unroll
    for (int j = 0; j < NW; ++j) v[j] = j < nage ? dur[(size_t)(a0 + j - 1) * C + kc] : 0.0f;
#pragma unroll
    for (int j = 0; j < NW; ++j) wd[j] = j < nage ? exp((double)v[j]) : 0.0;
  }

  // Step i of the block (position t0 + sigma*i) needs, for duration k, the
  // entry at t0 - sigma*(k - i); here k >= 2U > i and k <= K, so k - i lies
  // in [1, K].  Durations go in chunks of DCH (A is a multiple of DCH, so a
  // chunk holds this group's durations or weights past K, which are zero):
  // the chunk's DCH+U-1 entries (consecutive positions, read from a start
  // slot that needs no wrap thanks to the ring's mirror) come from LDS with
  // no branch, then U*DCH fused multiply-adds with compile-time register
  // indices.
  __device__ __forceinline__ void far(const WSmem &sm, const ChainShape &sh, int t0, int sigma,
                                      double (&F)[U]) {
    constexpr int NR = DCH + U - 1;  // entries per chunk
    static_assert(NR - 1 <= kWinMirror, "the mirror covers a chunk");
#pragma unroll
    for (int i = 0; i < U; ++i) F[i] = 0.0;
    if (!on) return;
    const int K = sh.K, C = sh.C;
    const int base = pos_slot(t0, K);
    // byte step to the next older position, held in a vector register: as a
    // uniform value the compiler keeps one multiple of it per read in scalar
    // registers, which spill (a v_readlane per read); here each read's
    // address is one add
    int rstep = -sigma * C * 8;
    __asm__("" : "+v"(rstep));
    // slot of the first chunk's first entry, m = a0 - (U - 1) in [U + 1, K]
    // positions back: base - sigma*m lies in (-K, 2K), so one wrap, no division
    int s0 = base - sigma * (a0 - (U - 1));
    s0 += s0 < 0 ? K : 0;
    s0 -= s0 >= K ? K : 0;
    // forward the slots fall with q, so a chunk whose reads would pass slot 0
    // starts in the mirror copy instead
    if (sigma > 0 && s0 < NR - 1) s0 += K;
    const unsigned c8 = (unsigned)C * 8u;
#pragma unroll
    for (int cb = 0; cb < NCH; ++cb) {
      const int jb = cb * DCH;
      if (jb >= nage) break;
      double wv[NR];
      // wv[q]: entry at m = k - i = m0 + q, m0 = a0 + jb - (U - 1),
      // q = jj - i + U - 1.  The next chunk starts DCH slots further back: one
      // wrap in the direction of travel (jb < nage <= K - a0 + 1, and a
      // forward start in the mirror rows reads copies of slots 0..15)
      if (cb > 0) {
        s0 -= sigma * DCH;
        if (sigma > 0 && s0 < NR - 1) s0 += K;
        if (sigma < 0 && s0 >= K) s0 -= K;
      }
      const char *rp = reinterpret_cast<const char *>(sm.ring) + __umul24((unsigned)s0, c8) +
                       (unsigned)kc * 8u;
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        wv[q] = *reinterpret_cast<const double *>(rp);
        rp += rstep;
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
#pragma unroll
        for (int jj = 0; jj < DCH; ++jj) F[i] = fma(wd[jb + jj], wv[jj - i + U - 1], F[i]);
      }
    }
  }

  // Publish the far partials part[buf][i][w-1][c], summed over the wave's
  // groups of one label (all lanes of the helper waves call).
  __device__ __forceinline__ void publish(const WSmem &sm, const ChainShape &sh, int NT,
                                          double (&F)[U], int buf) {
    const int C = sh.C, G = part_groups(sh, NT);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      double s = F[i];  // 0 on idle lanes
      if (gw <= 16) {
        s = group_sum(s, gw);
      } else {  // C <= 2: groups span rows
        for (int off = 1; off < gw; off <<= 1) s += __shfl_xor(s, off);
      }
      if (lane % gw == 0 && kc < C) sm.part[((buf * U + i) * G + (w - 1)) * C + kc] = s;
    }
  }
};

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
}

// Exp-space contraction: lane c < C holds a[c] = exp(o[c]) / 2^B (at most
// 1, the largest >= 1/2) and receives sum_{c'} a[c'] * tr[c'] in float64.
// The e row is broadcast through LDS, two values per read, all reads issued
// before the first multiply; every lane sums its part of the previous labels
// (load_tr_row) and the parts meet by lane swaps.  All 64 lanes of wave 0
// call.  `meanwhile` runs after the e-row reads are issued and before their
// results are used: independent work placed there hides in the LDS latency
// instead of delaying the step (a wave issues in order).
template <int CMAX, typename F>
__device__ __forceinline__ double chain_contract(const WSmem &sm, const ChainShape &sh, int lane,
                                                 double a, const double *tr,
                                                 F &&meanwhile) {
  constexpr int SP = kSplit<CMAX>, NJ = CMAX / SP;
  static_assert(NJ % 2 == 0, "pairs of previous labels per read");
  if (lane < CMAX) sm.erow[lane] = lane < sh.C ? a : 0.0;
  wave_lds_sync();
  const int h = (lane / CMAX) % SP;
  const double2 *e2 = reinterpret_cast<const double2 *>(sm.erow + h * NJ);
  double2 ev[NJ / 2];
#pragma unroll
  for (int q = 0; q < NJ / 2; ++q) ev[q] = e2[q];
  __builtin_amdgcn_sched_barrier(0);
  meanwhile();
  __builtin_amdgcn_sched_barrier(0);
  double d;
  if constexpr (NJ >= 4) {
    double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
#pragma unroll
    for (int q = 0; q < NJ / 2; q += 2) {
      d0 = fma(ev[q].x, tr[2 * q], d0);
      d1 = fma(ev[q].y, tr[2 * q + 1], d1);
      d2 = fma(ev[q + 1].x, tr[2 * q + 2], d2);
      d3 = fma(ev[q + 1].y, tr[2 * q + 3], d3);
    }
    d = (d0 + d1) + (d2 + d3);
  } else {
    d = fma(ev[0].y, tr[1], ev[0].x * tr[0]);
  }
  d = lane_swap_add<CMAX>(d);
  if constexpr (SP >= 4) d = lane_swap_add<2 * CMAX>(d);
  wave_lds_sync();
  return d;
}

__device__ __forceinline__ void wsave(double *__restrict__ dst, const WSmem &sm,
                                      const ChainShape &sh, bool chain, int lane, int R,
                                      double o, double m, int NT) {
  const int n = sh.K * sh.C;
  for (int i = threadIdx.x; i < n; i += NT) dst[i] = sm.ring[i];
  if (chain) {
    dst[n + lane] = (double)R;
    dst[n + sh.C + lane] = o;
    dst[n + 2 * sh.C + lane] = m;
  }
}

__device__ __forceinline__ void wload(const double *__restrict__ src, const WSmem &sm,
                                      const ChainShape &sh, bool chain, int lane, int &R,
                                      double &o, double &m, int NT) {
  const int n = sh.K * sh.C;
  for (int i0 = threadIdx.x; i0 < n; i0 += 4 * NT) {  // 4 loads in flight per thread
    double v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[min(i0 + u * NT, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * NT < n) sm.ring[i0 + u * NT] = v[u];
  }
  // the mirror of slots [0, kWinMirror) (those below K)
  const int nm = (sh.K < kWinMirror ? sh.K : kWinMirror) * sh.C;
  for (int i = threadIdx.x; i < nm; i += NT) sm.ring[n + i] = src[i];
  if (chain) {
    R = (int)src[n + lane];
    o = src[n + sh.C + lane];
    m = src[n + 2 * sh.C + lane];
  }
}

// Cumulative score of position t for label c (other lanes read label 0);
// t is clamped into [0, T], so every lane loads from a valid address.
__device__ __forceinline__ double es_raw(const Escaled &es, size_t ob, int t, int T, int C, int c) {
  const int tc = t < 0 ? 0 : (t > T ? T : t);
  return es.S[ob + (size_t)tc * C + (c < C ? c : 0)];
}

// Its split in the order the direction uses it: fx multiplies the K-sum
// (exp(S) forward, exp(-S) backward), fy the contraction (the other one), n
// is the exponent (its sign is applied where it is used).
__device__ __forceinline__ void es_split(double s, bool fwd, double &fx, double &fy, int &n) {
  double ep, em;
  exp_split(s, ep, em, n);
  fx = fwd ? ep : em;
  fy = fwd ? em : ep;
}

__device__ __forceinline__ void es_get(const Escaled &es, size_t ob, int t, int T, int C, int c,
                                       bool fwd, double &fx, double &fy, int &n) {
  es_split(es_raw(es, ob, t, T, C, c), fwd, fx, fy, n);
}

// Per-position log rows of a block's staged values: stg = [U][x[C], E[C],
// d[C], B]; step m (position t0 + sigma*m, m < nb) gives row1 = log x + E ln2
// (alpha / v) and row2 = log d + B ln2 (u / beta; not for the step `no2`).
// Threads [first, first + nthr) share the nb * 2C logs.
__device__ __forceinline__ void block_rows(const double *stg, int C, int nb, int t0, int sigma,
                                           double *row1, double *row2, int no2, int first,
                                           int nthr) {
  const int S = 3 * C + 1;
  for (int q = (int)threadIdx.x - first; q < nb * 2 * C; q += nthr) {
    const int m = q / (2 * C), r = q % (2 * C);
    const double *s = stg + m * S;
    const size_t o = (size_t)(t0 + sigma * m) * C;
    if (r < C)
      row1[o + r] = log_plus(s[r], s[C + r]);
    else if (m != no2)
      row2[o + r - C] = log_plus(s[C + r], s[3 * C]);
  }
}

// The same for full blocks of U steps on the row waves, with each thread's
// first item split into (step, entry) once per chunk (RowIdx) instead of by a
// division per block.
struct RowIdx {
  int m0, r0, ms, rs;  // first item's step and entry; the stride's quotient and remainder
  __device__ __forceinline__ void init(int q0, int C, int nthr) {
    const int w = 2 * C;
    m0 = q0 / w;
    r0 = q0 % w;
    ms = nthr / w;
    rs = nthr % w;
  }
};

__device__ __forceinline__ void block_rows_full(const double *stg, int C, int t0, int sigma,
                                                double *row1, double *row2, const RowIdx &ix) {
  const int S = 3 * C, w = 2 * C;
  for (int m = ix.m0, r = ix.r0; m < U;) {
    const double *s = stg + m * (S + 1);
    const size_t o = (size_t)(t0 + sigma * m) * C;
    if (r < C)
      row1[o + r] = log_plus(s[r], s[C + r]);
    else
      row2[o + r - C] = log_plus(s[C + r], s[S]);
    m += ix.ms;
    r += ix.rs;
    if (r >= w) {
      r -= w;
      ++m;
    }
  }
}

// Loader: the split scores of the block of U steps starting at step s0
// (positions first + sigma*(s0 + i)) for every label -- U*C pairs over the
// 64 lanes.
struct BlockLoad {
  static constexpr int NP = (U * 32 + 63) / 64;
  double sv[NP];

  // the scores only; put() splits and stores them a block later
  __device__ __forceinline__ void issue(const Escaled &es, size_t ob, int first, int sigma,
                                        int s0, int T, int C, int lane) {
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int q = lane + 64 * k;  // pair (i, c) = (q / C, q % C)
      const int i = q < U * C ? q / C : 0, c = q < U * C ? q % C : 0;
      sv[k] = es_raw(es, ob, first + sigma * (s0 + i), T, C, c);
    }
  }

  __device__ __forceinline__ void put(const WSmem &sm, int buf, int C, int lane, bool fwd) const {
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int q = lane + 64 * k;
      if (q < U * C) {
        const int o = buf * U * C + q;  // [buf][i][c], q = i*C + c
        double fx, fy;
        int n;
        es_split(sv[k], fwd, fx, fy, n);
        sm.efx[o] = fx;
        sm.efy[o] = fy;
        sm.en[o] = n;
      }
    }
  }
};

}  // namespace

// The chain wave's state carried from block to block: the register window
// of the near terms and the rebase shift its labels took during the block
// before (the far parts being read were computed in the reference they had
// when that block began).
struct ChainState {
  double hist[kNearW];  // hist[m] = entry of the step m+1 steps back (0 outside the window)
  double nr;            // near part of the next step without its newest term
  int shprev;
};

// The chain wave's part of one block (all 64 lanes of wave 0 call; lane c <
// C = label c): nb serial steps, then the shifts the older ring entries of
// each label still need.  The far parts are in part[buf][i][g][c]; the new
// entries go straight into the ring and into the window, so a rebase
// rescales those in place.  Per step only Dn[1] * (previous entry) of the
// near part is on the dependent chain; the rest is summed a step ahead, and
// the next step's LDS inputs are read a step ahead.  Bm, the step scale
// 2^Bm of the contraction inputs, carries over from step to step and is
// recomputed (an exact integer maximum) only when some label's exponent
// leaves [Bm - kScaleSpan, Bm + kScaleSpan]; every value stays exact either
// way.  o / m of step s_rec (the last burn-in step, see k_sweep_w) go to
// o_rec / m_rec, those of the chain's last step to o_end / m_end.
// The U steps are unrolled so the window never moves between registers:
// wv[U - i + m] is the entry m+1 steps before step i, and step i writes its
// entry to wv[U - 1 - i]; the window rolls once per block.
constexpr int kScaleSpan = 256;
template <int CMAX>
__device__ __forceinline__ void chain_block(const ChainShape &sh, const WSmem &sm, int G, int s0,
                                            int nb, int nsteps, int t0, int sigma, int buf,
                                            bool tail, int lane, bool chain,
                                            const double *Dn, const double *tr, int s_rec,
                                            ChainState &cs, int &R, int &Bm, double &o_rec,
                                            double &m_rec, double &o_end, double &m_end,
                                            double &lz) {
  const int C = sh.C, K = sh.K, S = 3 * C + 1;
  const int cl = chain ? lane : 0;  // label whose LDS values this lane reads
  const double *part = sm.part + (size_t)buf * U * G * C;
  auto far_of = [&](int i) {  // the helper waves' partials of step i, in a fixed order
    double f = 0.0;
    for (int g = 0; g < G; ++g) f += part[(i * G + g) * C + cl];
    return f;
  };
  double wv[U + kNearW];
#pragma unroll
  for (int m = 0; m < kNearW; ++m) wv[U + m] = cs.hist[m];
#pragma unroll
  for (int i = 0; i < U; ++i) wv[i] = 0.0;
  int shacc = 0;               // rebase shift of this label since the block began
  int slot = pos_slot(t0, K);  // ring slot of the step's position
  double *stg = sm.stg + buf * U * S;
  // inputs of step 0
  double fxn = sm.efx[buf * U * C + cl], fyn = sm.efy[buf * U * C + cl];
  int nqn = sm.en[buf * U * C + cl];
  double fsn = far_of(0);
  double nr = cs.nr;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    if (i >= nb) break;
    const double fx = fxn, fy = fyn, fs = fsn;
    const int nq = sigma * nqn;
    if (i + 1 < nb) {  // the next step's inputs, read a step ahead
      const int o = (buf * U + i + 1) * C + cl;
      fxn = sm.efx[o];
      fyn = sm.efy[o];
      nqn = sm.en[o];
      fsn = far_of(i + 1);
    }
    // the near part of the next step without its newest term (summed while
    // the contraction's LDS reads are in flight; two chains for latency)
    double nrn = 0.0;
    auto near_next = [&] {
      double n0 = 0.0, n1 = 0.0;
#pragma unroll
      for (int k = 2; k <= kNearW; k += 2) {
        n0 = fma(Dn[k], wv[U - i + k - 2], n0);
        if (k + 1 <= kNearW) n1 = fma(Dn[k + 1], wv[U - i + k - 1], n1);
      }
      nrn = n0 + n1;
      // keep the sum here, inside the LDS latency, rather than sunk to its use
      __asm__ volatile("" : "+v"(nrn));
    };
    const int step = s0 + i;
    const bool last = step == nsteps - 1;
    const bool lz_step = last && tail;
    // exp(o) = x * 2^E, o = alpha (forward) or v (backward)
    const double x =
        chain ? (ldexp(fs, -(cs.shprev + shacc)) + fma(Dn[1], wv[U - i], nr)) * fx : 0.0;
    const int E = R + nq;
    const int ex = (chain && x > 0.0) ? E + exponent_of(x) : kNoExp;
    if (__any(ex - Bm > kScaleSpan) || !__any(ex - Bm >= -kScaleSpan)) Bm = wave_max_i(ex);
    const double a = chain ? ldexp(x, E - Bm) : 0.0;  // exp(o) / 2^Bm
    if (chain) {
      stg[i * S + lane] = x;
      stg[i * S + C + lane] = (double)E;
    }
    if (lz_step) {
      lz = (double)Bm * kLn2 + log(wave_sum(a));
    } else {
      // exp(m) = d * 2^Bm, m = u (forward) or beta (backward).  Every lane
      // runs the rest of the step (lanes past C on harmless values, n = 0,
      // no stores), so the window's registers see no divergent branch.
      const double d = chain_contract<CMAX>(sm, sh, lane, a, tr, near_next);
      // entry exp(m -+ S) / 2^R = y * 2^s
      const double y = d * fy;
      const int s = Bm - nq - R;
      const int ey = exponent_of(y) + s;
      const int n = (chain && (ey > kRebaseExp || ey < -kRebaseExp)) ? ey : 0;
      if (chain) stg[i * S + 2 * C + lane] = d;
      if (__any(n != 0)) {  // rebase: the window and this block's ring entries follow at once
        R += n;
        shacc += n;
#pragma unroll
        for (int m = 0; m < kNearW; ++m) wv[U - i + m] = ldexp(wv[U - i + m], -n);
        nrn = ldexp(nrn, -n);
        if (chain && n != 0) {
          int sl = slot;
#pragma unroll
          for (int m = 0; m < i; ++m) {
            sl -= sigma;
            sl += sl < 0 ? K : 0;
            sl -= sl >= K ? K : 0;
            ring_put(sm, K, C, sl, lane, ldexp(sm.ring[sl * C + lane], -n));
          }
        }
      }
      const double g = ldexp(y, s - n);
      if (chain) ring_put(sm, K, C, slot, lane, g);
      wv[U - 1 - i] = g;
      if (last || step == s_rec) {
        const double o = log(x) + (double)E * kLn2, m = log(d) + (double)Bm * kLn2;
        if (last) {
          o_end = o;
          m_end = m;
        } else {
          o_rec = o;
          m_rec = m;
        }
      }
      if (lane == 0) stg[i * S + 3 * C] = (double)Bm;
    }
    nr = nrn;
    slot += sigma;
    slot += slot < 0 ? K : 0;
    slot -= slot >= K ? K : 0;
  }
  // roll the window by the block (a block of fewer than U steps ends the
  // chunk, so its window is not used again)
#pragma unroll
  for (int m = 0; m < kNearW; ++m) cs.hist[m] = wv[m];
  cs.nr = nr;
  cs.shprev = shacc;
  if (chain) sm.shiftn[lane] = shacc;
  const bool any = __any((chain && shacc != 0) ? 1 : 0);
  if (lane == 0) sm.flag[0] = any ? 1 : 0;
}

// ------------------------------------------------------------------ sweeps
// One workgroup per (direction, sequence b, chunk j), chunk = [p0, p1): the
// forward chain runs t = p0+1 .. p1 from the state at p0, the backward chain
// t = p1-1 .. p0 from the state at p1 (parallel-in-time; pit.hip verifies and
// normalises).  The start state is the chunk's checkpoint record: built at
// iteration 0 (exact at the sequence end the chain starts from, neutral
// elsewhere), re-read afterwards.  The chunk that ends its chain yields log Z
// in its own frame; every other chunk writes its end state.
template <int NT, int CMAX, int DCH, bool REP>
__global__ __launch_bounds__(NT) void k_sweep_w(ChainShape sh, const float *__restrict__ trans,
                                                const float *__restrict__ dur, Escaled es,
                                                const int32_t *__restrict__ lengths, PitBufs pb,
                                                int iter) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int nck = sh.B * sh.nchunk;
  const bool replay = iter == -1;  // a window of chunks swept again from exact records
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
      for (int i = threadIdx.x; i < sh.nchunk; i += NT) pb.nbad[i] = 0;
  }
  const int L = lengths[b];
  const int tid = threadIdx.x, C = sh.C, K = sh.K, T = sh.T;
  const int lane = tid & 63;
  const bool chain = tid < C;  // lanes of wave 0
  // (the iteration flags are loaded with the length: one memory wait)
  const int nbad = REP ? pb.nbad[kPitParallelIters - 1] : iter > 0 ? pb.nbad[iter - 1] : 1,
            redo = !REP && iter > 0 ? pb.redo[idx] : 1;
  if (L < 1 || L > T || jc >= sh.nchunk) return;
  if (jc * sh.delta >= L) return;
  if (nbad == 0 || redo == 0) return;
  const int nvalid = (L + sh.delta - 1) / sh.delta;
  __shared__ PitMaxArg red[NT / 64];  // scratch of the repair's checks
  __shared__ double redd[NT / 64];
  if constexpr (REP) {
    // nothing to repair unless the last parallel check found a chunk of
    // this chain inconsistent
    int marked = 0;
    for (int j = tid; j < nvalid; j += NT) marked |= pb.redo[base + j];
    if (!pit_any<NT>(marked != 0, red)) return;
  }
  const WSmem sm = wcarve(lds, sh, NT);
  Win<DCH, CMAX> win;
  win.init(sh, dur);
  double *const Dn = win.wd;  // near-part weights of the chain lanes (k = 1 .. 2U-1)
  double *const tr = win.wd + kNearW + 1;  // this lane's part of the exp(trans) weights
  if (tid < 64) {
#pragma unroll
    for (int k = 0; k <= kNearW; ++k)
      Dn[k] = (chain && k >= 1 && k <= K) ? exp((double)dur[(size_t)(k - 1) * C + lane]) : 0.0;
    load_tr_row<CMAX>(sh, trans, fwd, lane, tr);
  }
  const size_t ob = (size_t)b * (T + 1) * C;
  const size_t cks = ck_stride(C, K);
  const int sigma = fwd ? 1 : -1;
  const bool rows = pb.row_a != nullptr;
  const int rt0 = pb.row_t0;  // rows are written relative to the window start
  const size_t orow = (size_t)b * pb.row_stride * C;
  double *row1 = rows ? (fwd ? pb.row_a : pb.row_v) + orow : nullptr;  // alpha / v
  double *row2 = rows ? (fwd ? pb.row_u : pb.row_b) + orow : nullptr;  // u / beta

  // one chunk, p0 .. p1, from its start record (or, at iteration 0, from
  // its exact or neutral start after the burn-in)
  auto sweep_chunk = [&](const int jc) __attribute__((always_inline)) {
    const int p0 = jc * sh.delta;
    const int p1 = min(p0 + sh.delta, L);
    double *rec_start = (fwd ? pb.ck_fwd : pb.ck_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
    double *rec_end = (fwd ? pb.end_fwd : pb.end_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
    const int tstart = fwd ? p0 : p1;
    const bool tail = fwd ? (p1 == L) : (p0 == 0);  // this chunk ends the chain
    int R = 0;  // integer log reference of label `lane` (units of ln2)
    // Burn-in: at iteration 0 a chunk without an exact start begins wb
    // positions early (a whole number of blocks) from the neutral state, sweeps
    // them without writing rows, and stores the state it reaches at its true
    // start as its start record.  The recursion forgets where it started, so
    // that record usually already agrees with the predecessor's end and the
    // verification accepts it after one iteration.
    const bool exact = fwd ? (jc == 0) : (p1 == L);
    int wb = 0;
    if (iter == 0 && !exact) {
      wb = min(sh.burn, fwd ? p0 : L - p1);
      wb = wb / U * U;
    }
    const int tbegin = fwd ? p0 - wb : p1 + wb;  // where the sweep starts
    if (iter == 0) {
      for (int i = tid; i < (K + kWinMirror) * C; i += NT) sm.ring[i] = 0.0;
      __syncthreads();
      if (exact) {
        // entry u[0] - S[0] = 0 forward; beta[L] + S[L] = S[L] backward
        if (chain) {
          double v = 1.0;
          if (!fwd) {  // exp(S[L]) = ep * 2^n
            double em;
            exp_split(es.S[ob + (size_t)L * C + lane], v, em, R);
          }
          ring_put(sm, K, C, pos_slot(tstart, K), lane, v);
        }
      } else {
        // neutral start: every entry of the window (positions inside [0, L]) is 1
        for (int i = tid; i < K * C; i += NT) {
          const int dq = i / C, c = i % C;
          const int q = tbegin - sigma * dq;
          if (q >= 0 && q <= L) ring_put(sm, K, C, pos_slot(q, K), c, 1.0);
        }
      }
      __syncthreads();
      // o = NaN marks a neutral start (never accepted by the verification);
      // after a burn-in the record is written when the sweep reaches tstart
      if (wb == 0)
        wsave(rec_start, sm, sh, chain, lane, R,
              exact ? -__builtin_huge_val() : __builtin_nan(""), exact ? 0.0 : __builtin_nan(""), NT);
      if (exact && chain && rows)  // u[0] = 0 forward, beta[L] = 0 backward
        row2[(size_t)(tstart - rt0) * C + lane] = 0.0;
    } else {
      double o0, m0;
      wload(rec_start, sm, sh, chain, lane, R, o0, m0, NT);
      // a replay window's first row (its chunk before is not swept again): the
      // record's exact outputs at the start position
      if (replay && rows && chain &&
          (fwd ? jc == sh.rj0 : (jc == sh.rj0 + sh.rnb - 1 || p1 == L))) {
        row1[(size_t)(tstart - rt0) * C + lane] = o0;
        row2[(size_t)(tstart - rt0) * C + lane] = m0;
      }
    }
    const int first = tbegin + sigma;
    const int nsteps = wb + (p1 - p0);
    {  // the first block's scores (later blocks: the loader wave, a block ahead)
      const int npair = min(U, nsteps) * C;
      for (int q = tid; q < npair; q += NT) {
        double fx, fy;
        int n;
        es_get(es, ob, first + sigma * (q / C), T, C, q % C, fwd, fx, fy, n);
        sm.efx[q] = fx;
        sm.efy[q] = fy;
        sm.en[q] = n;
      }
    }
    vm_drain();
    __syncthreads();

    double o_end = 0.0, m_end = 0.0, lz = 0.0, o_rec = 0.0, m_rec = 0.0;
    int Bm = -(1 << 29);  // step scale of the chain; the first step computes it
    // wave roles: 0 the chain; 1-3 the far parts of the next block, besides
    // which 1 loads the next block's scores and 2-3 write the previous
    // block's rows
    const int w = tid >> 6;
    const int G = part_groups(sh, NT), S = 3 * C + 1;
    ChainState cs;
    if (w == 0) {
      // the window from the start state: entry m+1 steps back is at position
      // tbegin - sigma*m (0 beyond the ring)
  #pragma unroll
      for (int m = 0; m < kNearW; ++m)
        cs.hist[m] = (chain && m < K) ? sm.ring[pos_slot(tbegin - sigma * m, K) * C + lane] : 0.0;
      double nr = 0.0;
  #pragma unroll
      for (int k = 2; k <= kNearW; ++k) nr = fma(Dn[k], cs.hist[k - 1], nr);
      cs.nr = nr;
      cs.shprev = 0;
    } else {
      double F[U];  // far parts of the first block
      win.far(sm, sh, first, sigma, F);
      win.publish(sm, sh, NT, F, 0);
    }
    __syncthreads();
    BlockLoad bl;
    RowIdx rix;  // the row waves' items (threads 128 .. NT-1)
    rix.init(tid - 128, C, NT - 128);
    for (int s0 = 0; s0 < nsteps; s0 += U) {
      const int nb = min(U, nsteps - s0);  // steps in this block
      const int t0 = first + sigma * s0;
      const int buf = (s0 / U) & 1;
      const bool more = s0 + U < nsteps;
      if (wb > 0 && s0 == wb) {  // the burn-in ends: the chunk's start record
        wsave(rec_start, sm, sh, chain, lane, R, o_rec, m_rec, NT);
        __syncthreads();  // read before the chain overwrites ring slots
      }
      if (w == 0) {
        chain_block<CMAX>(sh, sm, G, s0, nb, nsteps, t0, sigma, buf, tail, lane, chain, Dn, tr,
                          wb - 1, cs, R, Bm, o_rec, m_rec, o_end, m_end, lz);
      } else {
        if (w == 1 && more) bl.issue(es, ob, first, sigma, s0 + U, T, C, lane);
        if (w >= 2 && rows && s0 > wb) {
          // the previous block's rows (a full block of U steps, past the burn-in)
          block_rows_full(sm.stg + (buf ^ 1) * U * S, C, t0 - sigma * U - rt0, sigma, row1, row2,
                          rix);
        }
        if (more) {
          // far parts of the next block: entries older than this block only,
          // none of the slots the chain writes meanwhile
          double F[U];
          win.far(sm, sh, t0 + sigma * U, sigma, F);
          win.publish(sm, sh, NT, F, buf ^ 1);
        }
        // the next block's scores land in the other buffer before the barrier
        // that ends this block
        if (w == 1 && more) bl.put(sm, buf ^ 1, C, lane, fwd);
      }
      __syncthreads();
      if (sm.flag[0]) {
        // rare: rescale the older entries of the labels that rebased (every
        // slot but the block's new entries), label by label over all threads
        const int nl = lane < C ? sm.shiftn[lane] : 0;
        unsigned long long rb = __ballot(nl != 0);
        const int slot0 = pos_slot(t0, K);
        while (rb) {
          const int c = __builtin_ctzll(rb);
          rb &= rb - 1;
          const int n = __builtin_amdgcn_readlane(nl, c);
          for (int m = 1 + tid; m <= K - nb; m += NT) {
            int sl = slot0 - sigma * m;
            sl += sl < 0 ? K : 0;
            sl -= sl >= K ? K : 0;
            ring_put(sm, K, C, sl, c, ldexp(sm.ring[sl * C + c], -n));
          }
        }
        __syncthreads();
      }
    }
    if (!replay) {
      if (tail) {
        if (tid == 0) pb.lz_part[(fwd ? 0 : sh.B) + b] = lz;
      } else {
        wsave(rec_end, sm, sh, chain, lane, R, o_end, m_end, NT);
      }
    }
    if (rows) {  // rows of the last block
      const int s0 = (nsteps - 1) / U * U;
      block_rows(sm.stg + ((s0 / U) & 1) * U * (3 * C + 1), C, nsteps - s0,
                 first + sigma * s0 - rt0, sigma, row1, row2, tail ? nsteps - 1 - s0 : -1, 0, NT);
    }
  };
  if constexpr (REP) {
    // the chain's chunks in order, past its exact one: a marked chunk is
    // swept from its replaced start, then its successor is checked against
    // the new end (forced to take it if the successor is marked too: its own
    // end belongs to an older start)
    for (int s = 1; s < nvalid; ++s) {
      const int j = fwd ? s : nvalid - 1 - s;
      __syncthreads();  // the previous chunk's LDS and rows
      if (pb.redo[base + j] == 0) continue;
      sweep_chunk(j);
      if (s + 1 < nvalid) {
        const int jn = fwd ? j + 1 : j - 1;
        __threadfence_block();  // the end record, for every thread of the check
        __syncthreads();
        pit_check<NT>(sh, pb, fwd, b, jn, -1, pb.redo[base + jn] != 0, red, redd);
      }
    }
  } else {
    sweep_chunk(jc);
  }
}

// ------------------------------------------------------------- dispatch
static hipError_t wreport(hipError_t e, const char *what, const ChainShape &sh, size_t lds) {
  if (e != hipSuccess && getenv("SEMICRF_DEBUG"))
    fprintf(stderr, "semicrf: %s (NT=%d C=%d K=%d A=%d lds=%zu) failed: %s\n", what, sh.NT, sh.C,
            sh.K, sh.A, lds, hipGetErrorString(e));
  return e;
}

template <int NT, int CMAX, int DCH>
struct WinKernels {
  static void attrs() {
    static bool done = false;
    if (!done) {
      (void)hipFuncSetAttribute((const void *)k_sweep_w<NT, CMAX, DCH, false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
      (void)hipFuncSetAttribute((const void *)k_sweep_w<NT, CMAX, DCH, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
      (void)hipGetLastError();
      done = true;
    }
  }
  static hipError_t sweep(const ChainShape &sh, const float *trans, const float *dur,
                          const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                          int with_bwd, int iter, hipStream_t st) {
    attrs();
    const size_t lds = win_lds_bytes(sh.C, sh.K, sh.P);
    const bool rep = iter == kPitRepair;
    const void *f = rep ? (const void *)k_sweep_w<NT, CMAX, DCH, true>
                        : (const void *)k_sweep_w<NT, CMAX, DCH, false>;
    if (!lds_fits(f, lds)) return wreport(hipErrorInvalidConfiguration, "k_sweep_w (LDS)", sh, lds);
    const int nd = with_bwd ? 2 : 1;
    if (rep) {
      hipLaunchKernelGGL((k_sweep_w<NT, CMAX, DCH, true>), dim3(nd * sh.B), dim3(NT), lds, st, sh,
                         trans, dur, es, lengths, pb, iter);
    } else {
      const int grid = iter < 0 ? sh.B * (sh.rnf + sh.rnb) : nd * sh.B * sh.nchunk;
      hipLaunchKernelGGL((k_sweep_w<NT, CMAX, DCH, false>), dim3(grid), dim3(NT), lds, st, sh,
                         trans, dur, es, lengths, pb, iter);
    }
    return wreport(hipGetLastError(), "k_sweep_w", sh, lds);
  }
};

// Instances: 256 threads; contraction width CMAX = cpad(C) in {8, 16, 32};
// duration chunk DCH in {2, 4, 8} (the smallest covering A, else 8).
template <int CMAX, typename F>
static hipError_t win_by_dch(const ChainShape &sh, F &&f) {
  if (sh.A <= 2) return f(WinKernels<256, CMAX, 2>());
  if (sh.A <= 4) return f(WinKernels<256, CMAX, 4>());
  return f(WinKernels<256, CMAX, 8>());
}

template <typename F>
static hipError_t win_dispatch(const ChainShape &sh, F &&f) {
  // not a windowed shape: the host configuration never selects these
  if (sh.NT != 256 || sh.C > 32) return hipErrorInvalidValue;
  if (sh.C <= 8) return win_by_dch<8>(sh, f);
  if (sh.C <= 16) return win_by_dch<16>(sh, f);
  return win_by_dch<32>(sh, f);
}

hipError_t launch_sweep_w(const ChainShape &sh, const float *trans, const float *dur,
                          const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                          int with_bwd, int iter, hipStream_t st) {
  return win_dispatch(sh, [&](auto k) {
    return decltype(k)::sweep(sh, trans, dur, es, lengths, pb, with_bwd, iter, st);
  });
}

}  // namespace semicrf
