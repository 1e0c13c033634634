// chain.hip -- streaming semi-CRF forward-backward on gfx950.
//
// Method ("Streaming Structured Inference with Flash-SemiCRF"; abstract and
// technical summary at gist.science, sections 2.A-2.C):
//   * segment scores are read on the fly from the cumulative scores S
//     (scan.hip); no edge tensor exists anywhere;
//   * the forward and backward messages stream through a ring buffer of the
//     K most recent rows (section 2.B);
//   * the forward state is stored every `delta` ~ sqrt(T*K) positions
//     together with its running log normaliser, and the backward pass
//     recomputes the forward messages between those checkpoints (2.C).
//
// Recurrences (0-based, per sequence of length L; sigma = +1 forward, -1
// backward; "entry" is what a position contributes to the ring):
//   forward   o[t,c] = alpha[t,c] = S[t,c] + LSE_{k<=min(K,t)} (dur[k-1,c] + g[t-k,c])
//             m[t,c] = u[t,c]     = LSE_{c'} (alpha[t,c'] + trans[c',c]);  u[0,.] = 0
//             entry  g[t,c]       = u[t,c] - S[t,c]
//   backward  o[t,c] = v[t,c]     = -S[t,c] + LSE_{k<=min(K,L-t)} (dur[k-1,c] + h[t+k,c])
//             m[t,c] = beta[t,c]  = LSE_{c'} (trans[c,c'] + v[t,c']);    beta[L,.] = 0
//             entry  h[t,c]       = beta[t,c] + S[t,c]
// This is the plain semi-CRF dynamic programme (score of a segment [s,s+k)
// with label c = S[s+k,c] - S[s,c] + dur[k-1,c]) written in the ring's
// variables.
//
// MI355X design:
//   * exp-space ring in LDS: ring[slot][c] = exp(entry - R[c]*ln2) in
//     float64, R[c] a per-label integer log reference.  The K-way
//     log-sum-exp becomes a K-term float64 dot product with
//     D[k][c] = exp(dur[k-1][c]) (no transcendental per segment cell).
//     Whenever a new entry leaves [2^-260, 2^260] relative to its reference,
//     the label's column is rescaled by an exact power of two (v_ldexp_f64)
//     and R[c] moves by that exponent.  The recurrence guarantees
//     g[t] >= g[t-k] + trans[c,c] + dur[k-1,c] (and the mirror for h), so
//     older ring entries never exceed the newest by more than a
//     parameter-bounded factor, and the rescale keeps every entry in float64
//     range.
//   * the log values themselves grow linearly along the sequence (~5e6 at a
//     million positions, where a float64 holds only ~1e-9 absolute).  Each
//     step therefore runs relative to base*ln2, base = label 0's integer
//     reference: only small numbers and small integer differences R - base
//     enter the recursion, so no rounding of a large number accumulates.
//     Absolute alpha/u/beta (formed once, for the posterior exponents) and
//     log Z carry a single rounding each.
//   * the transition contraction is an exp-space matrix-vector product with
//     exp(trans) held in registers (fp32), max-shifted per row.
//   * one workgroup per chain; the forward and the backward chain of every
//     sequence run concurrently (they are independent).  The marginal pass is
//     chunk-parallel: one workgroup per (sequence, checkpoint interval)
//     recomputes alpha from the forward checkpoint and beta from the backward
//     checkpoint and accumulates the posteriors.
//   * parameter-gradient partials are per chunk and reduced in a fixed order
//     in float64 (deterministic; no floating-point atomics).
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "device_math.h"
#include "internal.h"

namespace semicrf {

constexpr double kRebaseNats = 180.0;  // ~2^260

struct Smem {
  double *ring, *part, *orow, *refs, *scal, *erow, *dotp;
  int *shiftn;
};

__device__ __forceinline__ Smem carve(unsigned char *base, const ChainShape &s) {
  Smem m;
  size_t off = 0;
  m.ring = reinterpret_cast<double *>(base + off); off += (size_t)s.K * s.C * 8;
  m.part = reinterpret_cast<double *>(base + off); off += (size_t)s.P * s.C * 8;
  m.orow = reinterpret_cast<double *>(base + off); off += (size_t)s.C * 8;
  m.refs = reinterpret_cast<double *>(base + off); off += (size_t)s.C * 8;
  m.scal = reinterpret_cast<double *>(base + off); off += 8 * 8;
  m.erow = reinterpret_cast<double *>(base + off); off += (size_t)s.C * 8;
  m.dotp = reinterpret_cast<double *>(base + off); off += (size_t)s.QT * s.C * 8;
  m.shiftn = reinterpret_cast<int *>(base + off);
  return m;
}

// Per-thread constants of one chain direction.  The contraction weights are
// float64 for slices of up to 16 previous labels (every C <= 64): a rounded
// exp(trans) is a fixed perturbation of the parameters, and the parameter
// gradients -- sums over the whole sequence -- move by it times their own
// sensitivity, which grows with the sequence length.  Wider slices (C > 90
// at 512 threads, C > 128 at 1024) keep float32 weights for registers.
template <int AMAX, int TRMAX, typename DT>
struct Regs {
  using WT = typename std::conditional<(TRMAX <= 16), double, float>::type;
  DT D[AMAX];    // exp(dur[k-1][c]) for the thread's durations
  WT Tr[TRMAX];  // exp(trans) slice for the contraction role
  int kc, kp, age0, nage;
  int cc, cq, cp0, ncp;
};

template <int AMAX, int TRMAX, typename DT>
__device__ __forceinline__ void init_regs(Regs<AMAX, TRMAX, DT> &r, const ChainShape &sh,
                                          const float *__restrict__ dur) {
  const int tid = threadIdx.x, C = sh.C;
  r.kc = tid % C;
  r.kp = tid / C;
  r.age0 = r.kp * sh.A + 1;
  int n = (r.kp < sh.P) ? sh.K - r.age0 + 1 : 0;
  n = n < 0 ? 0 : (n > sh.A ? sh.A : n);
  r.nage = n;
#pragma unroll
  for (int j = 0; j < AMAX; ++j)
    r.D[j] = (j < r.nage) ? (DT)exp((double)dur[(size_t)(r.age0 + j - 1) * C + r.kc]) : (DT)0;
  r.cc = tid % C;
  r.cq = tid / C;
  r.cp0 = r.cq * sh.CS;
  int m = (r.cq < sh.QT) ? C - r.cp0 : 0;
  r.ncp = m < 0 ? 0 : (m > sh.CS ? sh.CS : m);
}

// Contraction weights for direction `fwd`: forward sums over the previous
// label c' (rows of trans), backward over the next label (columns).
template <int AMAX, int TRMAX, typename DT>
__device__ __forceinline__ void load_trans(Regs<AMAX, TRMAX, DT> &r, const ChainShape &sh,
                                           const float *__restrict__ trans, bool fwd) {
  const int C = sh.C;
#pragma unroll
  for (int j = 0; j < TRMAX; ++j) {
    double w = 0.0;
    if (j < r.ncp) {
      const int cp = r.cp0 + j;
      w = exp((double)(fwd ? trans[(size_t)cp * C + r.cc] : trans[(size_t)r.cc * C + cp]));
    }
    r.Tr[j] = (typename Regs<AMAX, TRMAX, DT>::WT)w;
  }
}

__device__ __forceinline__ int slot_of(int tm, int k, int K, bool fwd) {
  int s = fwd ? tm - k : tm + k;
  s += (s < 0) ? K : 0;
  s -= (s >= K) ? K : 0;
  return s;
}

// K-sum over the thread's durations: sum_k D[k] * ring[slot(t,k)].  With
// WITH_GD (backward marginal pass) also accumulates the segment posteriors
// gd[j] += q * D[k] * ring[slot].
template <bool WITH_GD, int AMAX, int TRMAX, typename DT, typename GT>
__device__ __forceinline__ double ksum(const Regs<AMAX, TRMAX, DT> &r, const Smem &sm,
                                       const ChainShape &sh, int t, bool fwd, GT (&gd)[AMAX],
                                       double q) {
  double s = 0.0;
  const int K = sh.K, C = sh.C;
  const int tm = t % K;
#pragma unroll
  for (int j = 0; j < AMAX; ++j) {
    if (j < r.nage) {
      const int sl = slot_of(tm, r.age0 + j, K, fwd);
      const double w = (double)r.D[j] * sm.ring[sl * C + r.kc];
      s += w;
      if (WITH_GD) gd[j] += (GT)(q * w);
    }
  }
  return s;
}

// Max over the C row values (row threads hold `v`).  All threads call.
__device__ __forceinline__ double row_max(double v, bool is_row, const ChainShape &sh,
                                          const Smem &sm) {
  double x = is_row ? v : -__builtin_huge_val();
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmax(x, __shfl_xor(x, off));
  if (sh.C <= 64) return x;  // all row threads are in wave 0
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0 && w < sh.Q) sm.scal[w] = x;
  __syncthreads();
  double m = sm.scal[0];
  for (int i = 1; i < sh.Q; ++i) m = fmax(m, sm.scal[i]);
  return m;
}

// Contraction: row thread c receives M + log(sum_{c'} e[c'] * W[c'][c]),
// summed in float64 (any per-step rounding here would accumulate along the
// chain).  Slice partials meet in LDS and the row thread adds them in a
// fixed order.  Requires sm.erow written and a barrier before the call.
// All threads call.
template <int AMAX, int TRMAX, typename DT>
__device__ __forceinline__ double contract(const Regs<AMAX, TRMAX, DT> &r, const Smem &sm,
                                           const ChainShape &sh, double M) {
  using WT = typename Regs<AMAX, TRMAX, DT>::WT;
  double dp = 0.0;
#pragma unroll
  for (int j = 0; j < TRMAX; ++j) {
    if (j < r.ncp) {
      WT w = r.Tr[j];
      if (!std::is_same<WT, double>::value) {
        // keep a float32 weight live as float32: converting all TRMAX
        // weights once, outside the time loop, would double their registers
        asm volatile("" : "+v"(w));
      }
      dp = fma(sm.erow[r.cp0 + j], (double)w, dp);
    }
  }
  if (sh.QT > 1) {
    if (r.cq < sh.QT) sm.dotp[r.cq * sh.C + r.cc] = dp;
    __syncthreads();
    if ((int)threadIdx.x < sh.C) {
      dp = 0.0;
      for (int q = 0; q < sh.QT; ++q) dp += sm.dotp[q * sh.C + threadIdx.x];
    }
  }
  return M + log(dp);
}

// Row thread c inserts the entry for position t, given as d = entry minus
// its log reference R*ln2 (R an exact integer), and decides an exact
// power-of-two rebase of its column.  Returns true if the column must be
// rescaled by 2^-n (n in sm.shiftn[c]).
__device__ __forceinline__ bool insert_entry(const Smem &sm, const ChainShape &sh, int t,
                                             double d, int &R) {
  const int c = threadIdx.x;
  int n = 0;
  if (fabs(d) > kRebaseNats) {
    n = (int)rint(d * kLog2e);
    R += n;
    d -= (double)n * kLn2;
  }
  sm.shiftn[c] = n;
  sm.refs[c] = (double)R;
  sm.ring[(t % sh.K) * sh.C + c] = exp(d);
  return n != 0;
}

// Apply pending column rescales: every ring slot except the newest (position
// t) is multiplied by 2^-shiftn[c].  Slots are owned through the durations
// of the next step, so each is touched by exactly one thread.
template <int AMAX, int TRMAX, typename DT>
__device__ __forceinline__ void apply_rebase(const Regs<AMAX, TRMAX, DT> &r, const Smem &sm,
                                             const ChainShape &sh, int t, bool fwd) {
  if (r.nage > 0) {
    const int n = sm.shiftn[r.kc];
    if (n != 0) {
      const int tn = fwd ? t + 1 : t - 1;
      const int tm = tn % sh.K;
      for (int j = 0; j < r.nage; ++j) {
        const int k = r.age0 + j;
        if (k < 2) continue;
        const int sl = slot_of(tm, k, sh.K, fwd);
        sm.ring[sl * sh.C + r.kc] = ldexp(sm.ring[sl * sh.C + r.kc], -n);
      }
    }
  }
  __syncthreads();
}


__device__ __forceinline__ void save_ckpt(double *__restrict__ dst, const Smem &sm,
                                          const ChainShape &sh, int R, double o, double m) {
  const int n = sh.K * sh.C;
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = sm.ring[i];
  if ((int)threadIdx.x < sh.C) {
    dst[n + threadIdx.x] = (double)R;
    dst[n + sh.C + threadIdx.x] = o;
    dst[n + 2 * sh.C + threadIdx.x] = m;
  }
}

__device__ __forceinline__ void load_ckpt(const double *__restrict__ src, const Smem &sm,
                                          const ChainShape &sh, int &R, double &o, double &m) {
  const int n = sh.K * sh.C;
  for (int i = threadIdx.x; i < n; i += blockDim.x) sm.ring[i] = src[i];
  if ((int)threadIdx.x < sh.C) {
    R = (int)src[n + threadIdx.x];
    o = src[n + sh.C + threadIdx.x];
    m = src[n + 2 * sh.C + threadIdx.x];
    sm.refs[threadIdx.x] = (double)R;
  }
  __syncthreads();
}

// Sum over labels of exp(o - M) for the log normaliser at a sequence end.
__device__ __forceinline__ double row_lse(double o, bool is_row, const ChainShape &sh,
                                          const Smem &sm) {
  const double M = row_max(o, is_row, sh, sm);
  if (is_row) sm.orow[threadIdx.x] = exp(o - M);
  __syncthreads();
  double s = 0.0;
  for (int c = 0; c < sh.C; ++c) s += sm.orow[c];
  return M + log(s);
}

// ---------------------------------------------------------------- sweeps
// One workgroup per (direction, sequence b, chunk j), chunk = [p0, p1): the
// forward chain runs t = p0+1 .. p1 from the state at p0, the backward chain
// t = p1-1 .. p0 from the state at p1 (parallel-in-time; pit.hip verifies and
// normalises).  The start state is the chunk's checkpoint record: built at
// iteration 0 (exact at the sequence end the chain starts from, neutral
// elsewhere), re-read afterwards.  The chunk that ends its chain yields log Z
// in its own frame; every other chunk writes its end state.
template <int NT, int AMAX, int TRMAX, typename DT>
__global__ __launch_bounds__(NT) void k_sweep(ChainShape sh, const float *__restrict__ trans,
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
  const int tid = threadIdx.x, C = sh.C, K = sh.K;
  const bool is_row = tid < C;
  if (L < 1 || L > sh.T) return;
  const int p0 = jc * sh.delta;
  if (p0 >= L) return;
  const int p1 = min(p0 + sh.delta, L);
  const size_t idx = (fwd ? 0 : (size_t)nck) + (size_t)b * sh.nchunk + jc;
  if (iter > 0 && (pb.nbad[iter - 1] == 0 || pb.redo[idx] == 0)) return;
  Smem sm = carve(lds, sh);
  Regs<AMAX, TRMAX, DT> r;
  init_regs(r, sh, dur);
  load_trans(r, sh, trans, fwd);
  const double *Sb = S + (size_t)b * (sh.T + 1) * C;
  const size_t cks = ck_stride(C, K);
  double *rec_start = (fwd ? pb.ck_fwd : pb.ck_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  double *rec_end = (fwd ? pb.end_fwd : pb.end_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  const double sigma = fwd ? 1.0 : -1.0;
  const int isig = fwd ? 1 : -1;
  const int tstart = fwd ? p0 : p1;
  const bool tail = fwd ? (p1 == L) : (p0 == 0);  // this chunk ends the chain

  int R = 0;
  double o = 0.0, m = 0.0;
  if (iter == 0) {
    for (int i = tid; i < K * C; i += NT) sm.ring[i] = 0.0;
    __syncthreads();
    const bool exact = fwd ? (jc == 0) : (p1 == L);
    if (exact) {
      // forward position 0 (u = 0), backward position L (beta = 0)
      if (is_row) {
        double d = 0.0;  // entry minus R*ln2
        if (!fwd) {
          const double sl = Sb[(size_t)L * C + tid];
          R = (int)rint(sl * kLog2e);
          d = sl - (double)R * kLn2;
        }
        sm.ring[(tstart % K) * C + tid] = exp(d);
      }
    } else {
      // neutral start: every entry of the window (positions inside [0, L]) is 1
      for (int i = tid; i < K * C; i += NT) {
        const int dq = i / C, c = i % C;
        const int q = tstart - isig * dq;
        if (q >= 0 && q <= L) sm.ring[(q % K) * C + c] = 1.0;
      }
    }
    if (is_row) sm.refs[tid] = (double)R;
    __syncthreads();
    // o = NaN marks a neutral start (never accepted by the verification)
    save_ckpt(rec_start, sm, sh, R, exact ? -__builtin_huge_val() : __builtin_nan(""),
              exact ? 0.0 : __builtin_nan(""));
    if (exact && is_row && pb.row_a)  // u[0] = 0 forward, beta[L] = 0 backward
      (fwd ? pb.row_u : pb.row_b)[((size_t)b * (sh.T + 1) + tstart) * C + tid] = 0.0;
    __syncthreads();
  } else {
    load_ckpt(rec_start, sm, sh, R, o, m);
  }

  const int nsteps = p1 - p0;  // forward t = p0+1..p1, backward t = p1-1..p0
  for (int step = 1; step <= nsteps; ++step) {
    const int t = fwd ? p0 + step : p1 - step;
    double nogd[AMAX];
    const double s = r.kp < sh.P ? ksum<false>(r, sm, sh, t, fwd, nogd, 0.0) : 0.0;
    if (r.kp < sh.P) sm.part[r.kp * C + r.kc] = s;
    __syncthreads();
    // the step runs relative to base*ln2, base = label 0's integer reference
    const int base = (int)sm.refs[0];
    const double bl = (double)base * kLn2;
    o = 0.0;  // alpha (forward) or v (backward) minus bl
    if (is_row) {
      double sum = 0.0;
      for (int p = 0; p < sh.P; ++p) sum += sm.part[p * C + tid];
      o = sigma * Sb[(size_t)t * C + tid] + (double)(R - base) * kLn2 + log(sum);
    }
    const bool last = step == nsteps;
    if (is_row && pb.row_a)  // per-position rows, in this chunk's frame
      (fwd ? pb.row_a : pb.row_v)[((size_t)b * (sh.T + 1) + t) * C + tid] = bl + o;
    if (last && tail) {
      const double lz = bl + row_lse(o, is_row, sh, sm);
      if (tid == 0) pb.lz_part[(fwd ? 0 : sh.B) + b] = lz;
      break;
    }
    const double M = row_max(o, is_row, sh, sm);
    if (is_row) sm.erow[tid] = exp(o - M);
    __syncthreads();
    m = contract(r, sm, sh, M);  // u (forward) or beta (backward) minus bl
    if (is_row && pb.row_a)
      (fwd ? pb.row_u : pb.row_b)[((size_t)b * (sh.T + 1) + t) * C + tid] = bl + m;
    bool need = false;
    if (is_row)
      need = insert_entry(sm, sh, t,
                          (m - sigma * Sb[(size_t)t * C + tid]) + (double)(base - R) * kLn2, R);
    if (__syncthreads_or(need)) apply_rebase(r, sm, sh, t, fwd);
    if (last) save_ckpt(rec_end, sm, sh, R, bl + o, bl + m);
  }
}

// ------------------------------------------------------------- dispatch
// With SEMICRF_DEBUG set, name a failed launch and its configuration.
static hipError_t report(hipError_t e, const char *what, const ChainShape &sh, size_t lds) {
  if (e != hipSuccess && getenv("SEMICRF_DEBUG"))
    fprintf(stderr, "semicrf: %s (NT=%d C=%d K=%d lds=%zu) failed: %s\n", what, sh.NT, sh.C, sh.K,
            lds, hipGetErrorString(e));
  return e;
}

template <int NT, int AMAX, int TRMAX, typename DT, typename GT>
struct ChainKernels {
  // Raise the dynamic-LDS limit once per instance (the ring can exceed 64 KB);
  // clear the error state so a refusal cannot masquerade as a launch error.
  static void set_attrs() {
    static bool done = false;
    if (!done) {
      (void)hipFuncSetAttribute((const void *)k_sweep<NT, AMAX, TRMAX, DT>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
      (void)hipGetLastError();
      done = true;
    }
  }
  static hipError_t sweep(const ChainShape &sh, const float *trans, const float *dur,
                          const double *S, const int32_t *lengths, const PitBufs &pb,
                          int with_bwd, int iter, hipStream_t st) {
    const size_t lds = chain_lds_bytes(sh.C, sh.K, sh.P, sh.QT);
    set_attrs();
    hipLaunchKernelGGL((k_sweep<NT, AMAX, TRMAX, DT>), dim3((with_bwd ? 2 : 1) * sh.B * sh.nchunk),
                       dim3(NT), lds, st, sh, trans, dur, S, lengths, pb, iter);
    return report(hipGetLastError(), "k_sweep", sh, lds);
  }
};

// Instances: threads NT x slice width TRMAX (>= sh.CS, the contraction
// slice; float64 weights up to 16).
#define SEMICRF_CHAIN_DISPATCH(SH, CALL)                                                   \
  do {                                                                                     \
    const int cs_ = (SH).CS;                                                               \
    const int trmax_ = cs_ <= 8 ? 8 : (cs_ <= 16 ? 16 : (cs_ <= 32 ? 32 : 64));           \
    if ((SH).NT == 256) {                                                                  \
      if (trmax_ == 8) return ChainKernels<256, 32, 8, double, double>::CALL;              \
      if (trmax_ == 16) return ChainKernels<256, 32, 16, double, double>::CALL;            \
      if (trmax_ == 32) return ChainKernels<256, 32, 32, double, double>::CALL;            \
      return ChainKernels<256, 32, 64, double, double>::CALL;                              \
    } else if ((SH).NT == 512) {                                                           \
      if (trmax_ == 8) return ChainKernels<512, 32, 8, double, double>::CALL;              \
      if (trmax_ == 16) return ChainKernels<512, 32, 16, double, double>::CALL;            \
      if (trmax_ == 32) return ChainKernels<512, 32, 32, double, double>::CALL;            \
      return ChainKernels<512, 32, 64, double, double>::CALL;                              \
    } else {                                                                               \
      if (trmax_ == 8) return ChainKernels<1024, 16, 8, float, float>::CALL;               \
      if (trmax_ == 16) return ChainKernels<1024, 16, 16, float, float>::CALL;             \
      if (trmax_ == 32) return ChainKernels<1024, 16, 32, float, float>::CALL;             \
      return ChainKernels<1024, 16, 64, float, float>::CALL;                               \
    }                                                                                      \
  } while (0)

hipError_t launch_sweep(const ChainShape &sh, const float *trans, const float *dur,
                        const double *S, const int32_t *lengths, const PitBufs &pb,
                        int with_bwd, int iter, hipStream_t st) {
  if (sh.win) return launch_sweep_w(sh, trans, dur, S, lengths, pb, with_bwd, iter, st);
  SEMICRF_CHAIN_DISPATCH(sh, sweep(sh, trans, dur, S, lengths, pb, with_bwd, iter, st));
}

}  // namespace semicrf
