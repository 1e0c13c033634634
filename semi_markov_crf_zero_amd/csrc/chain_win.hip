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
//     serial part -- log of the K-sum, max, exp, the C x C contraction
//     (exp(trans) staged in LDS), the new ring entry and the rebase decision
//     -- with wave-local synchronisation only: two workgroup barriers per
//     step in total.
//   * S rows (and, in the backward marginal pass, the alpha/u rows of the
//     chunk) are prefetched U steps ahead into per-lane register queues, so
//     no global-memory latency sits on the per-step critical path.
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

constexpr double kRebaseNatsW = 180.0;  // ~2^260

struct WSmem {
  double *ring, *part, *qrow, *tr, *erow;
  int *shiftn, *flag;
};

__device__ __forceinline__ int round4(int c) { return (c + 3) & ~3; }

// Carve-up; the byte count is win_lds_bytes() in internal.h.
__device__ __forceinline__ WSmem wcarve(unsigned char *base, const ChainShape &s) {
  WSmem m;
  size_t off = 0;
  const int C4 = round4(s.C);
  m.ring = reinterpret_cast<double *>(base + off); off += (size_t)s.K * s.C * 8;
  m.part = reinterpret_cast<double *>(base + off); off += (size_t)s.P * s.C * 8;
  m.qrow = reinterpret_cast<double *>(base + off); off += (size_t)s.C * 8;
  off = (off + 15) & ~(size_t)15;
  m.tr = reinterpret_cast<double *>(base + off); off += (size_t)C4 * s.C * 8;
  off = (off + 15) & ~(size_t)15;
  m.erow = reinterpret_cast<double *>(base + off); off += (size_t)C4 * 8;
  m.shiftn = reinterpret_cast<int *>(base + off); off += (size_t)s.C * 4;
  m.flag = reinterpret_cast<int *>(base + off);
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

// Row rotation by DPP; lanes whose source would be invalid keep their own
// value (update_dpp with old = src), so no register is ever left undefined.
__device__ __forceinline__ float dpp_ror(float v, int ctrl_sel) {
  const int iv = __builtin_bit_cast(int, v);
  int r;
  switch (ctrl_sel) {
    case 8: r = __builtin_amdgcn_update_dpp(iv, iv, 0x128, 0xf, 0xf, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(iv, iv, 0x124, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(iv, iv, 0x122, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(iv, iv, 0x121, 0xf, 0xf, false); break;
  }
  return __builtin_bit_cast(float, r);
}

// Wave-wide max of a float (all 64 lanes call): row rotations by DPP, then
// the four row maxima through scalar reads.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_ror(v, 8));
  v = fmaxf(v, dpp_ror(v, 4));
  v = fmaxf(v, dpp_ror(v, 2));
  v = fmaxf(v, dpp_ror(v, 1));
  const int iv = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
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

// Max-shifted exp-space contraction of the row o (lane c holds o[c]):
// returns M + log(sum_{c'} exp(o[c'] - M) * tr[c'][c]); e = exp(o - M) and M
// are returned too.  The shift M only needs to be near the maximum (it
// cancels), so it is a float32 wave reduction; e, the sum and the log are
// float64-accurate because their rounding would accumulate along the chain.
// All 64 lanes of wave 0 call.
template <int CMAX>
__device__ __forceinline__ double chain_contract(const WSmem &sm, const ChainShape &sh, int lane,
                                                 double o, double &e_out, double &M_out) {
  const int C = sh.C;
  const bool act = lane < C;
  const float M = wave_max(act ? (float)o : -__builtin_huge_valf());
  const double Md = (double)M;
  const double e = act ? exp(o - Md) : 0.0;
  if (lane < round4(C)) sm.erow[lane] = e;
  wave_lds_sync();
  double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
  if (act) {
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
  e_out = e;
  M_out = Md;
  return Md + log((d0 + d1) + (d2 + d3));
}

// New ring entry for position t of label `lane`, given as d = entry minus
// the label's log reference R*ln2 (R an exact integer), and the rebase
// decision.
__device__ __forceinline__ bool chain_insert(const WSmem &sm, const ChainShape &sh, int lane,
                                             int t, double d, int &R) {
  int n = 0;
  if (fabs(d) > kRebaseNatsW) {
    n = (int)rint(d * kLog2e);
    R += n;
    d -= (double)n * kLn2;
  }
  sm.shiftn[lane] = n;
  sm.ring[pos_slot(t, sh.K) * sh.C + lane] = exp(d);
  return n != 0;
}

// The chain wave's per-step base: label 0's integer reference.  Each step
// runs relative to base*ln2 so that only small numbers enter the recursion
// (absolute log values reach ~5e6 at a million positions).
__device__ __forceinline__ int chain_base(int R) { return __builtin_amdgcn_readlane(R, 0); }

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

__device__ __forceinline__ double ld_or(const double *p, bool ok) { return ok ? *p : 0.0; }

}  // namespace

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
                                                const float *__restrict__ dur,
                                                const double *__restrict__ S,
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
  const double *Sb = S + (size_t)b * (T + 1) * C;
  const size_t cks = ck_stride(C, K);
  double *rec_start = (fwd ? pb.ck_fwd : pb.ck_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  double *rec_end = (fwd ? pb.end_fwd : pb.end_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  const int sigma = fwd ? 1 : -1;
  const double sg = (double)sigma;
  const int tstart = fwd ? p0 : p1;
  const bool tail = fwd ? (p1 == L) : (p0 == 0);  // this chunk ends the chain

  int R = 0;  // integer log reference of label `lane` (units of ln2)
  if (iter == 0) {
    for (int i = tid; i < K * C; i += NT) sm.ring[i] = 0.0;
    __syncthreads();
    const bool exact = fwd ? (jc == 0) : (p1 == L);
    if (exact) {
      if (chain) {
        double d = 0.0;  // entry minus R*ln2: u[0] - S[0] = 0 forward, beta[L] + S[L] backward
        if (!fwd) {
          const double sl = Sb[(size_t)L * C + lane];
          R = (int)rint(sl * kLog2e);
          d = sl - (double)R * kLn2;
        }
        sm.ring[pos_slot(tstart, K) * C + lane] = exp(d);
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
    if (exact && chain && pb.row_a)  // u[0] = 0 forward, beta[L] = 0 backward
      (fwd ? pb.row_u : pb.row_b)[((size_t)b * (T + 1) + tstart) * C + lane] = 0.0;
  } else {
    double o0, m0;
    wload(rec_start, sm, sh, chain, lane, R, o0, m0, NT);
  }
  __syncthreads();

  const int first = fwd ? p0 + 1 : p1 - 1;
  const int nsteps = p1 - p0;
  double Sq[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int t = first + sigma * i;
    Sq[i] = chain ? ld_or(Sb + (size_t)t * C + lane, t >= 0 && t <= T) : 0.0;
  }
  double nogd[AMAX];
  bool done = false;
  for (int s0 = 0; !done; s0 += U) {
    const int t0 = first + sigma * s0;
    win.fill(sm, sh, t0, sigma);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (!done) {
        const int step = s0 + i;
        const int t = t0 + sigma * i;
        const double ks = win.on ? win.template step<false>(i, sm, sh, sigma, nogd, 0.0) : 0.0;
        win.publish(sm, sh, ks);
        __syncthreads();
        const bool last = step == nsteps - 1;
        const bool lz_step = last && tail;
        double o = 0.0, m = 0.0;  // relative to bl
        double bl = 0.0;
        if (wave0) {
          const double st = Sq[i];
          const int base = chain_base(R);
          bl = (double)base * kLn2;
          o = chain ? sg * st + (double)(R - base) * kLn2 + log(chain_sum<NT>(sm, sh, lane)) : 0.0;
          if (lz_step) {
            const float M = wave_max(chain ? (float)o : -__builtin_huge_valf());
            const double ex = chain ? exp(o - (double)M) : 0.0;
            const double lz = bl + ((double)M + log(wave_sum(ex)));
            if (tid == 0) pb.lz_part[(fwd ? 0 : sh.B) + b] = lz;
          } else {
            double e, M;
            m = chain_contract<CMAX>(sm, sh, lane, o, e, M);
            bool rb = false;
            if (chain)
              rb = chain_insert(sm, sh, lane, t, (m - sg * st) + (double)(base - R) * kLn2, R);
            chain_flag(sm, t, rb);
          }
          if (chain && pb.row_a) {  // per-position rows, in this chunk's frame
            const size_t ri = ((size_t)b * (T + 1) + t) * C + lane;
            (fwd ? pb.row_a : pb.row_v)[ri] = bl + o;
            if (!lz_step) (fwd ? pb.row_u : pb.row_b)[ri] = bl + m;
          }
          if (chain) {  // prefetch S for the same block offset of the next block
            const int tp = t + sigma * U;
            Sq[i] = ld_or(Sb + (size_t)tp * C + lane, tp >= 0 && tp <= T);
          }
        }
        if (!lz_step) {
          __syncthreads();
          if (sm.flag[t & 1]) {
            win.rebase(sm, sh, t, sigma);
            __syncthreads();
          }
        }
        if (last) {
          done = true;
          if (!lz_step) wsave(rec_end, sm, sh, chain, lane, R, bl + o, bl + m, NT);
        }
      }
    }
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
                          const double *S, const int32_t *lengths, const PitBufs &pb,
                          int with_bwd, int iter, hipStream_t st) {
    attrs();
    const size_t lds = win_lds_bytes(sh.C, sh.K, sh.P);
    hipLaunchKernelGGL((k_sweep_w<NT, AMAX, U, CMAX>), dim3((with_bwd ? 2 : 1) * sh.B * sh.nchunk),
                       dim3(NT), lds, st, sh, trans, dur, S, lengths, pb, iter);
    return wreport(hipGetLastError(), "k_sweep_w", sh, lds);
  }
};

// Instances: 256 threads; durations per thread AMAX in {8, 16, 32}; unroll /
// prefetch depth U (sweep) and UC (marginal pass), smaller for the
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
                          const double *S, const int32_t *lengths, const PitBufs &pb,
                          int with_bwd, int iter, hipStream_t st) {
  return win_dispatch(sh, [&](auto k) {
    return decltype(k)::sweep(sh, trans, dur, S, lengths, pb, with_bwd, iter, st);
  });
}

}  // namespace semicrf
