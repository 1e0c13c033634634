// chain_win.hip -- windowed streaming engine for C <= 32 labels.
//
// Same recurrences, ring contents, checkpoint records and outputs as
// chain.hip (see its header for the equations and the method citations);
// this file only reorganises the work for gfx950 latency:
//
//   * K-sum with register windows.  Thread (g, c) owns the durations
//     k = a0 .. a0+AMAX-1 (a0 = 1 + g*A) of label c.  The ring values it
//     needs slide by one position per step, so it keeps them in registers
//     (W[0 .. AMAX+U-2]) and loads ONE new value from the LDS ring per step;
//     the loop is unrolled U steps so every register index is a compile-time
//     constant, and the window is refilled from the ring once per U steps.
//     LDS traffic per step drops from K*C*8 bytes to about P*C*8*(1+AMAX/U).
//   * one "chain wave" (wave 0, lane c = label c) does the per-position
//     serial part -- the K-sum times exp(+-S), an integer maximum of the
//     float64 exponents, the C x C contraction (exp(trans) staged in LDS), the
//     new ring entry and the rebase decision -- with wave-local
//     synchronisation only: two workgroup barriers per step in total.  No
//     transcendental function sits on this path (see chain.hip: exp(+-S) come
//     split from the score scan, every rescaling is an exact power of two).
//   * the waves specialise (each runs its own copy of the step loop, with
//     the same barriers): wave 1 prefetches the split scores of the next
//     block of U positions into LDS (its loop issues only loads, so nothing
//     waits on them before the block ends), waves 2-3 turn the previous
//     step's staged values into the per-position log rows (their loop issues
//     only stores), and the chain wave reads its scores from LDS -- no
//     global-memory access sits on the per-step critical path.
//   * an exact power-of-two column rebase (rare) runs as its own barrier-
//     separated mini-phase that rescales the register windows and the LDS
//     ring together.
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "device_math.h"
#include "internal.h"

namespace semicrf {

namespace {

constexpr int kRebaseExp = 260;  // rebase bound, log2 units
constexpr int kWinPB = 8;        // largest unroll block (positions); sizes the score buffers

struct WSmem {
  double *ring, *part, *stg, *tr, *erow;
  double *efx, *efy;  // split scores of two blocks [2][kWinPB][C]
  int *shiftn, *flag, *en;
};

__device__ __forceinline__ int round4(int c) { return (c + 3) & ~3; }

// Carve-up; the byte count is win_lds_bytes() in internal.h.
__device__ __forceinline__ WSmem wcarve(unsigned char *base, const ChainShape &s) {
  WSmem m;
  size_t off = 0;
  const int C4 = round4(s.C);
  m.ring = reinterpret_cast<double *>(base + off); off += (size_t)s.K * s.C * 8;
  m.part = reinterpret_cast<double *>(base + off); off += (size_t)s.P * s.C * 8;
  m.stg = reinterpret_cast<double *>(base + off); off += (size_t)2 * (3 * s.C + 1) * 8;
  off = (off + 15) & ~(size_t)15;
  m.tr = reinterpret_cast<double *>(base + off); off += (size_t)C4 * s.C * 8;
  off = (off + 15) & ~(size_t)15;
  m.erow = reinterpret_cast<double *>(base + off); off += (size_t)C4 * 8;
  m.shiftn = reinterpret_cast<int *>(base + off); off += (size_t)s.C * 4;
  m.flag = reinterpret_cast<int *>(base + off); off += 2 * 4;
  off = (off + 15) & ~(size_t)15;
  m.efx = reinterpret_cast<double *>(base + off); off += (size_t)2 * kWinPB * s.C * 8;
  m.efy = reinterpret_cast<double *>(base + off); off += (size_t)2 * kWinPB * s.C * 8;
  m.en = reinterpret_cast<int *>(base + off);
  return m;
}

__device__ __forceinline__ int pos_slot(int pos, int K) {
  int s = pos % K;
  return s < 0 ? s + K : s;
}

// exp(trans) in float64 (a rounded weight would perturb the parameters, and
// the parameter gradients move by that times a sensitivity that grows with
// the sequence length), oriented for the contraction of direction fwd, rows
// padded to a multiple of 4 with zeros: tr[c_in * C + c_out] = weight of
// input label c_in for output label c_out.
__device__ __forceinline__ void stage_trans(const WSmem &sm, const ChainShape &sh,
                                            const float *__restrict__ trans, bool fwd, int NT) {
  const int C = sh.C, C4 = round4(C);
  for (int i = threadIdx.x; i < C4 * C; i += NT) {
    const int ci = i / C, co = i % C;
    double w = 0.0;
    if (ci < C) w = exp((double)(fwd ? trans[(size_t)ci * C + co] : trans[(size_t)co * C + ci]));
    sm.tr[i] = w;
  }
}

// Partials are pre-reduced inside each wave when C divides 64 (lanes of one
// label sit C apart); the chain wave then reads one value per wave.
__device__ __forceinline__ bool wave_reduced(const ChainShape &sh) { return (64 % sh.C) == 0; }

template <int AMAX, int U>
struct Win {
  using DT = typename std::conditional<(AMAX <= 16), double, float>::type;
  DT D[AMAX];
  double W[AMAX + U - 1];
  int kc, kg, a0, nage, yslot;
  bool on;

  __device__ __forceinline__ void init(const ChainShape &sh, const float *__restrict__ dur) {
    const int C = sh.C;
    kc = threadIdx.x % C;
    kg = threadIdx.x / C;
    on = kg < sh.P;
    a0 = 1 + kg * sh.A;
    int n = on ? sh.K - a0 + 1 : 0;
    n = n < 0 ? 0 : (n > sh.A ? sh.A : n);
    nage = n;
#pragma unroll
    for (int j = 0; j < AMAX; ++j)
      D[j] = (j < nage) ? (DT)exp((double)dur[(size_t)(a0 + j - 1) * C + kc]) : (DT)0;
  }

  // Fill W[0 .. AMAX-2] for a block that starts at step t0 (direction sigma)
  // and point yslot at the value the first step of the block loads.
  __device__ __forceinline__ void fill(const WSmem &sm, const ChainShape &sh, int t0, int sigma) {
    if (!on) return;
    const int K = sh.K, C = sh.C;
    int sl = pos_slot(t0 - sigma * (a0 + AMAX - 1), K);
#pragma unroll
    for (int j = 0; j < AMAX - 1; ++j) {
      W[j] = sm.ring[sl * C + kc];
      sl += sigma;
      sl = sl >= K ? sl - K : (sl < 0 ? sl + K : sl);
    }
    yslot = sl;
  }

  // Load the youngest value of step I of the block (I is a constant once the
  // block loop is unrolled) and return the K-sum; with GD also accumulate the
  // segment posteriors gd[j] += q * D[j] * W.
  template <bool GD>
  __device__ __forceinline__ double step(int I, const WSmem &sm, const ChainShape &sh, int sigma,
                                         double (&gd)[AMAX], double q) {
    W[AMAX - 1 + I] = sm.ring[yslot * sh.C + kc];
    yslot += sigma;
    yslot = yslot >= sh.K ? yslot - sh.K : (yslot < 0 ? yslot + sh.K : yslot);
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < AMAX; ++j) {
      const double w = (double)D[j] * W[AMAX - 1 + I - j];
      s += w;
      if (GD) gd[j] += q * w;
    }
    return s;
  }

  // Rebase mini-phase: rescale the register window and the LDS slots of the
  // durations this thread owns (relative to the next step), except the
  // newest entry (position t).
  __device__ __forceinline__ void rebase(const WSmem &sm, const ChainShape &sh, int t, int sigma) {
    if (!on) return;
    const int n = sm.shiftn[kc];
    if (n == 0) return;
#pragma unroll
    for (int j = 0; j < AMAX + U - 1; ++j) W[j] = ldexp(W[j], -n);
    const int tn = t + sigma;
    for (int j = 0; j < nage; ++j) {
      const int k = a0 + j;
      if (k < 2) continue;
      const int sl = pos_slot(tn - sigma * k, sh.K);
      sm.ring[sl * sh.C + kc] = ldexp(sm.ring[sl * sh.C + kc], -n);
    }
  }

  // Publish the K-sum: per thread, or summed over the wave's groups of one
  // label (all lanes of the workgroup call).
  __device__ __forceinline__ void publish(const WSmem &sm, const ChainShape &sh, double s) {
    if (wave_reduced(sh)) {
      for (int off = sh.C; off < 64; off <<= 1) s += __shfl_xor(s, off);
      const int lane = threadIdx.x & 63;
      if (lane < sh.C) sm.part[(threadIdx.x >> 6) * sh.C + lane] = s;
    } else if (on) {
      sm.part[kg * sh.C + kc] = s;
    }
  }
};

// ---------------------------------------------------------------- chain wave
// Lane c < C of wave 0 reads the K-sum of label c.
template <int NT>
__device__ __forceinline__ double chain_sum(const WSmem &sm, const ChainShape &sh, int lane) {
  double sum = 0.0;
  if (wave_reduced(sh)) {
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) sum += sm.part[w * sh.C + lane];
  } else {
#pragma unroll 4
    for (int p = 0; p < sh.P; ++p) sum += sm.part[p * sh.C + lane];
  }
  return sum;
}

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
// 1, the largest >= 1/2) and receives sum_{c'} a[c'] * tr[c'][c] in float64.
// All 64 lanes of wave 0 call.
template <int CMAX>
__device__ __forceinline__ double chain_contract(const WSmem &sm, const ChainShape &sh, int lane,
                                                 double a) {
  const int C = sh.C;
  if (lane < round4(C)) sm.erow[lane] = lane < C ? a : 0.0;
  wave_lds_sync();
  double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
  if (lane < C) {
#pragma unroll
    for (int ci = 0; ci < CMAX; ci += 4) {
      if (ci < C) {
        d0 = fma(sm.erow[ci + 0], sm.tr[(ci + 0) * C + lane], d0);
        d1 = fma(sm.erow[ci + 1], sm.tr[(ci + 1) * C + lane], d1);
        d2 = fma(sm.erow[ci + 2], sm.tr[(ci + 2) * C + lane], d2);
        d3 = fma(sm.erow[ci + 3], sm.tr[(ci + 3) * C + lane], d3);
      }
    }
  }
  wave_lds_sync();
  return (d0 + d1) + (d2 + d3);
}

// New ring entry for position t of label `lane`: y * 2^s relative to the
// label's reference 2^R (y > 0 a float64, s an exact integer).  An entry
// outside [2^-kRebaseExp, 2^kRebaseExp] moves R by its exponent (rebase:
// the column's older entries are rescaled by the same power of two).
__device__ __forceinline__ bool chain_insert(const WSmem &sm, const ChainShape &sh, int lane,
                                             int t, double y, int s, int &R) {
  const int ey = exponent_of(y) + s;
  const int n = (ey > kRebaseExp || ey < -kRebaseExp) ? ey : 0;
  R += n;
  sm.shiftn[lane] = n;
  sm.ring[pos_slot(t, sh.K) * sh.C + lane] = ldexp(y, s - n);
  return n != 0;
}

// Wave-vote the rebase decisions of step t into the flag slot t&1 (lane 0).
__device__ __forceinline__ void chain_flag(const WSmem &sm, int t, bool rb) {
  const bool any = __any(rb ? 1 : 0);
  if ((threadIdx.x & 63) == 0) sm.flag[t & 1] = any ? 1 : 0;
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
  for (int i = threadIdx.x; i < n; i += NT) sm.ring[i] = src[i];
  if (chain) {
    R = (int)src[n + lane];
    o = src[n + sh.C + lane];
    m = src[n + 2 * sh.C + lane];
  }
}

// Split scores of position t for label c (row / chain lanes; other lanes
// read label 0), in the order the direction uses them: fx multiplies the
// K-sum (exp(S) forward, exp(-S) backward), fy the contraction (the other
// one), n is the exponent (its sign is applied where it is used).  t is
// clamped into [0, T], so every lane loads from a valid address and no
// select touches the loaded values: the loads stay in flight until their
// first use several positions later (a prefetch).
__device__ __forceinline__ void es_get(const Escaled &es, size_t ob, int t, int T, int C, int c,
                                       bool fwd, double &fx, double &fy, int &n) {
  const int tc = t < 0 ? 0 : (t > T ? T : t);
  const size_t i = ob + (size_t)tc * C + (c < C ? c : 0);
  fx = (fwd ? es.ep : es.em)[i];
  fy = (fwd ? es.em : es.ep)[i];
  n = es.n[i];
}

// Per-position log rows from a step's staged values (stg: x[C], E[C], d[C],
// B): row1 = log x + E ln2 (alpha / v), row2 = log d + B ln2 (u / beta).
// Threads [first, first + nthr) share the 2C logs.
__device__ __forceinline__ void stage_rows(const double *stg, int C, double *r1, double *r2,
                                           bool with2, int first, int nthr) {
  for (int i = (int)threadIdx.x - first; i < 2 * C; i += nthr) {
    if (i < C)
      r1[i] = log(stg[i]) + stg[C + i] * kLn2;
    else if (with2)
      r2[i - C] = log(stg[C + i]) + stg[3 * C] * kLn2;
  }
}

}  // namespace

// Wave roles of the windowed engine.
enum WinRole { kChainWave = 0, kLoaderWave = 1, kRowWaves = 2 };

// Loader: the split scores of the block of U steps starting at step s0
// (positions first + sigma*(s0 + i), i < U) for every label -- U*C
// (position, label) pairs over the 64 lanes, at most kWinPB*32/64 = 4 each.
template <int U>
struct BlockLoad {
  double fx[(U * 32 + 63) / 64], fy[(U * 32 + 63) / 64];
  int n[(U * 32 + 63) / 64];

  __device__ __forceinline__ void issue(const Escaled &es, size_t ob, int first, int sigma,
                                        int s0, int T, int C, int lane, bool fwd) {
#pragma unroll
    for (int k = 0; k < (U * 32 + 63) / 64; ++k) {
      const int q = lane + 64 * k;  // pair (i, c) = (q / C, q % C)
      const int i = q < U * C ? q / C : 0, c = q < U * C ? q % C : 0;
      es_get(es, ob, first + sigma * (s0 + i), T, C, c, fwd, fx[k], fy[k], n[k]);
    }
  }

  __device__ __forceinline__ void put(const WSmem &sm, int buf, int C, int lane) const {
#pragma unroll
    for (int k = 0; k < (U * 32 + 63) / 64; ++k) {
      const int q = lane + 64 * k;
      if (q < U * C) {
        const int o = buf * kWinPB * C + q;  // [buf][i][c], q = i*C + c
        sm.efx[o] = fx[k];
        sm.efy[o] = fy[k];
        sm.en[o] = n[k];
      }
    }
  }
};

// The step loop of one role (see WinRole).  Per step: K-sum share and
// publish, barrier, role work, barrier (not after the chain's last step),
// and the rare rebase mini-phase with its own barrier.  The chain wave
// leaves log Z (tail chunk) or the end-state o / m in lz / o_end / m_end.
template <int ROLE, int NT, int AMAX, int U, int CMAX>
__device__ __forceinline__ void sweep_w_loop(const ChainShape &sh, const WSmem &sm,
                                             Win<AMAX, U> &win, const Escaled &es, size_t ob,
                                             int first, int nsteps, int sigma, bool fwd,
                                             bool tail, bool rows, double *row1, double *row2,
                                             int lane, bool chain, int &R, double &o_end,
                                             double &m_end, double &lz) {
  const int C = sh.C, T = sh.T;
  double nogd[AMAX];
  BlockLoad<U> bl;
  bool done = false;
  for (int s0 = 0; !done; s0 += U) {
    const int t0 = first + sigma * s0;
    const int buf = (s0 / U) & 1;
    win.fill(sm, sh, t0, sigma);
    if (ROLE == kLoaderWave && s0 + U < nsteps) bl.issue(es, ob, first, sigma, s0 + U, T, C, lane, fwd);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (!done) {
        const int step = s0 + i;
        const int t = t0 + sigma * i;
        // the chain lanes' scores of this step (LDS, staged a block ahead)
        double fx = 0.0, fy = 0.0;
        int nq = 0;
        if (ROLE == kChainWave && chain) {
          const int o = (buf * kWinPB + i) * C + lane;
          fx = sm.efx[o];
          fy = sm.efy[o];
          nq = sigma * sm.en[o];
        }
        const double ks = win.on ? win.template step<false>(i, sm, sh, sigma, nogd, 0.0) : 0.0;
        win.publish(sm, sh, ks);
        __syncthreads();
        const bool last = step == nsteps - 1;
        const bool lz_step = last && tail;
        if (ROLE == kChainWave) {
          // exp(o) = x * 2^E with o = alpha (forward) or v (backward)
          double x = 0.0;
          int E = 0;
          if (chain) {
            x = chain_sum<NT>(sm, sh, lane) * fx;
            E = R + nq;
          }
          const int Bm = wave_max_i((chain && x > 0.0) ? E + exponent_of(x) : kNoExp);
          const double a = chain ? ldexp(x, E - Bm) : 0.0;  // exp(o) / 2^Bm
          double *stg = sm.stg + (step & 1) * (3 * C + 1);
          if (chain) {
            stg[lane] = x;
            stg[C + lane] = (double)E;
          }
          if (lz_step) {
            lz = (double)Bm * kLn2 + log(wave_sum(a));
          } else {
            // exp(m) = d * 2^Bm with m = u (forward) or beta (backward)
            const double d = chain_contract<CMAX>(sm, sh, lane, a);
            bool rb = false;
            if (chain) {
              stg[2 * C + lane] = d;
              // entry exp(m -+ S) / 2^R = d * fy * 2^(Bm -+ n - R)
              rb = chain_insert(sm, sh, lane, t, d * fy, Bm - nq - R, R);
              if (last) {
                o_end = log(x) + (double)E * kLn2;
                m_end = log(d) + (double)Bm * kLn2;
              }
            }
            if (lane == 0) stg[3 * C] = (double)Bm;
            chain_flag(sm, t, rb);
          }
        } else if (ROLE == kLoaderWave) {
          // the next block's scores land in the other buffer before the
          // barrier that ends this block
          if (i == U - 1 && s0 + U < nsteps) bl.put(sm, buf ^ 1, C, lane);
        } else if (rows && step > 0) {
          const size_t tp = (size_t)(t - sigma) * C;
          stage_rows(sm.stg + ((step - 1) & 1) * (3 * C + 1), C, row1 + tp, row2 + tp, true, 128,
                     NT - 128);
        }
        if (!lz_step) {
          __syncthreads();
          if (sm.flag[t & 1]) {
            win.rebase(sm, sh, t, sigma);
            __syncthreads();
          }
        }
        if (last) done = true;
      }
    }
  }
}

// ------------------------------------------------------------------ sweeps
// One workgroup per (direction, sequence b, chunk j), chunk = [p0, p1): the
// forward chain runs t = p0+1 .. p1 from the state at p0, the backward chain
// t = p1-1 .. p0 from the state at p1 (parallel-in-time; pit.hip verifies and
// normalises).  The start state is the chunk's checkpoint record: built at
// iteration 0 (exact at the sequence end the chain starts from, neutral
// elsewhere), re-read afterwards.  The chunk that ends its chain yields log Z
// in its own frame; every other chunk writes its end state.
// Per step: K-sum by every thread (one new ring value each), barrier, the
// chain wave's serial part, barrier; plus the rare rebase mini-phase.
template <int NT, int AMAX, int U, int CMAX>
__global__ __launch_bounds__(NT) void k_sweep_w(ChainShape sh, const float *__restrict__ trans,
                                                const float *__restrict__ dur, Escaled es,
                                                const int32_t *__restrict__ lengths, PitBufs pb,
                                                int iter) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int nck = sh.B * sh.nchunk;
  const bool fwd = (int)blockIdx.x < nck;
  const int rem = fwd ? blockIdx.x : blockIdx.x - nck;
  const int b = rem / sh.nchunk, jc = rem % sh.nchunk;
  const int L = lengths[b];
  const int tid = threadIdx.x, C = sh.C, K = sh.K, T = sh.T;
  const int lane = tid & 63;
  const bool chain = tid < C;  // lanes of wave 0
  const bool wave0 = tid < 64;
  if (L < 1 || L > T) return;
  const int p0 = jc * sh.delta;
  if (p0 >= L) return;
  const int p1 = min(p0 + sh.delta, L);
  const size_t idx = (fwd ? 0 : (size_t)nck) + (size_t)b * sh.nchunk + jc;
  if (iter > 0 && (pb.nbad[iter - 1] == 0 || pb.redo[idx] == 0)) return;
  const WSmem sm = wcarve(lds, sh);
  Win<AMAX, U> win;
  win.init(sh, dur);
  stage_trans(sm, sh, trans, fwd, NT);
  const size_t ob = (size_t)b * (T + 1) * C;
  const size_t cks = ck_stride(C, K);
  double *rec_start = (fwd ? pb.ck_fwd : pb.ck_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  double *rec_end = (fwd ? pb.end_fwd : pb.end_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  const int sigma = fwd ? 1 : -1;
  const int tstart = fwd ? p0 : p1;
  const bool tail = fwd ? (p1 == L) : (p0 == 0);  // this chunk ends the chain
  const bool rows = pb.row_a != nullptr;
  double *row1 = (fwd ? pb.row_a : pb.row_v) + ob;  // alpha / v
  double *row2 = (fwd ? pb.row_u : pb.row_b) + ob;  // u / beta

  int R = 0;  // integer log reference of label `lane` (units of ln2)
  if (iter == 0) {
    for (int i = tid; i < K * C; i += NT) sm.ring[i] = 0.0;
    __syncthreads();
    const bool exact = fwd ? (jc == 0) : (p1 == L);
    if (exact) {
      // entry u[0] - S[0] = 0 forward; beta[L] + S[L] = S[L] backward
      if (chain) {
        double v = 1.0;
        if (!fwd) {
          const size_t i = ob + (size_t)L * C + lane;
          v = es.ep[i];
          R = es.n[i];
        }
        sm.ring[pos_slot(tstart, K) * C + lane] = v;
      }
    } else {
      // neutral start: every entry of the window (positions inside [0, L]) is 1
      for (int i = tid; i < K * C; i += NT) {
        const int dq = i / C, c = i % C;
        const int q = tstart - sigma * dq;
        if (q >= 0 && q <= L) sm.ring[pos_slot(q, K) * C + c] = 1.0;
      }
    }
    __syncthreads();
    // o = NaN marks a neutral start (never accepted by the verification)
    wsave(rec_start, sm, sh, chain, lane, R,
          exact ? -__builtin_huge_val() : __builtin_nan(""), exact ? 0.0 : __builtin_nan(""), NT);
    if (exact && chain && rows)  // u[0] = 0 forward, beta[L] = 0 backward
      row2[(size_t)tstart * C + lane] = 0.0;
  } else {
    double o0, m0;
    wload(rec_start, sm, sh, chain, lane, R, o0, m0, NT);
  }
  __syncthreads();

  const int first = fwd ? p0 + 1 : p1 - 1;
  const int nsteps = p1 - p0;
  double o_end = 0.0, m_end = 0.0, lz = 0.0;
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
  const int w = tid >> 6;
  if (w == 0)
    sweep_w_loop<kChainWave, NT, AMAX, U, CMAX>(sh, sm, win, es, ob, first, nsteps, sigma, fwd,
                                                tail, rows, row1, row2, lane, chain, R, o_end,
                                                m_end, lz);
  else if (w == 1)
    sweep_w_loop<kLoaderWave, NT, AMAX, U, CMAX>(sh, sm, win, es, ob, first, nsteps, sigma, fwd,
                                                 tail, rows, row1, row2, lane, chain, R, o_end,
                                                 m_end, lz);
  else
    sweep_w_loop<kRowWaves, NT, AMAX, U, CMAX>(sh, sm, win, es, ob, first, nsteps, sigma, fwd,
                                               tail, rows, row1, row2, lane, chain, R, o_end,
                                               m_end, lz);
  if (tail) {
    if (tid == 0) pb.lz_part[(fwd ? 0 : sh.B) + b] = lz;
  } else {
    wsave(rec_end, sm, sh, chain, lane, R, o_end, m_end, NT);
  }
  if (rows) {  // rows of the last step (t = p1 forward, p0 backward)
    __syncthreads();
    const size_t tp = (size_t)(fwd ? p1 : p0) * C;
    stage_rows(sm.stg + ((nsteps - 1) & 1) * (3 * C + 1), C, row1 + tp, row2 + tp, !tail, 0, NT);
  }
}

// ------------------------------------------------------------- dispatch
static hipError_t wreport(hipError_t e, const char *what, const ChainShape &sh, size_t lds) {
  if (e != hipSuccess && getenv("SEMICRF_DEBUG"))
    fprintf(stderr, "semicrf: %s (NT=%d C=%d K=%d A=%d lds=%zu) failed: %s\n", what, sh.NT, sh.C,
            sh.K, sh.A, lds, hipGetErrorString(e));
  return e;
}

template <int NT, int AMAX, int U, int UC, int CMAX>
struct WinKernels {
  static void attrs() {
    static bool done = false;
    if (!done) {
      (void)hipFuncSetAttribute((const void *)k_sweep_w<NT, AMAX, U, CMAX>,
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
    if (!lds_fits((const void *)k_sweep_w<NT, AMAX, U, CMAX>, lds))
      return wreport(hipErrorInvalidConfiguration, "k_sweep_w (LDS)", sh, lds);
    hipLaunchKernelGGL((k_sweep_w<NT, AMAX, U, CMAX>), dim3((with_bwd ? 2 : 1) * sh.B * sh.nchunk),
                       dim3(NT), lds, st, sh, trans, dur, es, lengths, pb, iter);
    return wreport(hipGetLastError(), "k_sweep_w", sh, lds);
  }
};

// Instances: 256 threads; durations per thread AMAX in {8, 16, 32}; unroll
// block U (also the score-prefetch block; UC is unused), smaller for the
// 32-duration windows (register budget); contraction bound CMAX in {8, 32}.
template <int NT, int AMAX, int U, int UC>
struct WinByC {
  template <typename F>
  static hipError_t run(int C, F &&f) {
    if (C <= 8) return f(WinKernels<NT, AMAX, U, UC, 8>());
    return f(WinKernels<NT, AMAX, U, UC, 32>());
  }
};

template <typename F>
static hipError_t win_dispatch(const ChainShape &sh, F &&f) {
  // not a windowed shape: the host configuration never selects these
  if (sh.NT != 256 || sh.A > 32 || sh.C > 32) return hipErrorInvalidValue;
  if (sh.A <= 8) return WinByC<256, 8, 8, 8>::run(sh.C, f);
  if (sh.A <= 16) return WinByC<256, 16, 8, 8>::run(sh.C, f);
  return WinByC<256, 32, 4, 4>::run(sh.C, f);
}

hipError_t launch_sweep_w(const ChainShape &sh, const float *trans, const float *dur,
                          const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                          int with_bwd, int iter, hipStream_t st) {
  return win_dispatch(sh, [&](auto k) {
    return decltype(k)::sweep(sh, trans, dur, es, lengths, pb, with_bwd, iter, st);
  });
}

}  // namespace semicrf
