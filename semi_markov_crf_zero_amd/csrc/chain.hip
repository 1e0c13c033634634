// chain.hip -- streaming semi-CRF forward-backward on gfx950.
//
// Method ("Streaming Structured Inference with Flash-SemiCRF"; abstract and
// technical summary at gist.science, sections 2.A-2.C):
//   * segment scores are read on the fly from the cumulative scores S
//     (scan.hip); no edge tensor exists anywhere;
//   * the forward and backward messages stream through a ring buffer of the
//     K most recent rows (section 2.B);
//   * the state (ring and integer log references) is stored every `delta`
//     positions (the pages' interval ~ sqrt(T*K), section 2.C).  Every
//     interval is swept concurrently from its record (pit.hip); by default
//     the sweeps also keep the per-position rows for the posterior pass,
//     and in the low-memory mode the posterior pass recomputes them between
//     the checkpoints instead, window by window, from the records (api.hip).
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
//   * the whole step stays in exp space, so no transcendental function sits
//     on the serial path at all.  The loader waves split exp(+-S[t,c]) (from S)
//     as a float64 mantissa in [2^-1/2, 2^1/2] times 2^(+-n[t,c]); with the
//     K-sum ks[c] (relative to 2^R[c])
//       exp(o[t,c]) = x[c] * 2^E[c],  x = ks * exp(+-S) mantissa, E = R +- n
//     (an exact integer E); the step's scale 2^B is the largest float64
//     exponent of these (an integer maximum over the labels), the
//     contraction input a[c] = x[c] * 2^(E[c] - B) <= 1 is an exact ldexp,
//       exp(m[t,c]) = d[c] * 2^B,  d = sum_{c'} a[c'] * exp(trans)
//     and the new entry is d * exp(-+S) mantissa * 2^(B -+ n - R), again an
//     exact power-of-two scaling.  Every operation on the path is a float64
//     multiply-add or an exact scaling, so the recursion carries no error
//     beyond float64 rounding of products and sums, whatever the length.
//   * whenever a new entry leaves [2^-260, 2^260] relative to its reference,
//     the label's column is rescaled by an exact power of two (v_ldexp_f64)
//     and R[c] moves by that exponent.  The recurrence guarantees
//     g[t] >= g[t-k] + trans[c,c] + dur[k-1,c] (and the mirror for h), so
//     older ring entries never exceed the newest by more than a
//     parameter-bounded factor, and the rescale keeps every entry in float64
//     range.
//   * the waves specialise, each running its own copy of the step loop with
//     the same barriers: the row waves do the recursion; loader waves
//     prefetch the split scores of the next block of positions into LDS
//     (their loop issues only loads, consumed a block later); writer waves
//     take the per-position log rows (alpha, u / v, beta: log x + E ln2 and
//     log d + B ln2, a single rounding each) one step behind from values
//     staged in LDS (their loop issues only stores).  So neither a
//     global-memory access nor a logarithm sits on the serial path.
//   * the transition contraction is an exp-space matrix-vector product with
//     exp(trans) held in registers, split over the thread rows.
//   * one workgroup per (direction, sequence, checkpoint interval); the
//     intervals are swept concurrently and stitched by pit.hip.
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "device_math.h"
#include "internal.h"

namespace semicrf {

constexpr int kRebaseExp = 512;  // rebase bound, log2 units (see insert_entry)
constexpr int kScaleSpan = 256;  // step-scale span, log2 units (see sweep_loop)
constexpr int kErowPad = 64;     // zero tail of the e row: the widest slice reads past C

struct Smem {
  double *ring, *part, *erow, *scal, *dotp, *stg;
  double *efx, *efy;  // split scores of two prefetch blocks [2][pf][C]
  int *en, *shiftn;
};

__device__ __forceinline__ Smem carve(unsigned char *base, const ChainShape &s) {
  Smem m;
  size_t off = 0;
  m.ring = reinterpret_cast<double *>(base + off); off += (size_t)s.K * s.C * 8;
  m.part = reinterpret_cast<double *>(base + off); off += (size_t)s.P * s.C * 8;
  off = (off + 15) & ~(size_t)15;  // the e row is read as 16-byte pairs
  m.erow = reinterpret_cast<double *>(base + off); off += (size_t)(s.C + kErowPad) * 8;
  m.scal = reinterpret_cast<double *>(base + off); off += 8 * 8;
  m.dotp = reinterpret_cast<double *>(base + off); off += (size_t)s.QT * s.C * 8;
  m.stg = reinterpret_cast<double *>(base + off); off += (size_t)2 * (3 * s.C + 1) * 8;
  m.efx = reinterpret_cast<double *>(base + off); off += (size_t)2 * s.pf * s.C * 8;
  m.efy = reinterpret_cast<double *>(base + off); off += (size_t)2 * s.pf * s.C * 8;
  m.en = reinterpret_cast<int *>(base + off); off += (size_t)2 * s.pf * s.C * 4;
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
  // The 1024-thread instances (float32 weights) read their exp(trans) slice
  // from the workspace every step: holding it would take 64 of their 128
  // registers and spill the loop to scratch.
  static constexpr bool kGlobalW = std::is_same<DT, float>::value;
  DT D[AMAX];                    // exp(dur[k-1][c]) for the thread's durations
  WT Tr[kGlobalW ? 1 : TRMAX];   // exp(trans) slice for the contraction role
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
  if (Regs<AMAX, TRMAX, DT>::kGlobalW) return;
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

// K-sum over the thread's durations: sum_k D[k] * ring[slot(t,k)], its
// first term (duration age0) returned apart in `first`.  With WITH_GD
// (backward marginal pass) also accumulates the segment posteriors
// gd[j] += q * D[k] * ring[slot].
template <bool WITH_GD, int AMAX, int TRMAX, typename DT, typename GT>
__device__ __forceinline__ double ksum(const Regs<AMAX, TRMAX, DT> &r, const Smem &sm,
                                       const ChainShape &sh, int t, bool fwd, GT (&gd)[AMAX],
                                       double q, double &first) {
  // The ring offset of duration age0 + j moves by one row per duration
  // (wrapping once), so no multiply per term; past the thread's durations
  // the weight is 0 and the offset merely stays inside the ring.  Reads go
  // in batches of 8 into separate registers, so they pipeline, and four
  // running sums keep the additions off one chain.
  const int K = sh.K, C = sh.C, KC = K * C;
  int off = slot_of(t % K, min(r.age0, K), K, fwd) * C + r.kc;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int jb = 0; jb < AMAX; jb += 8) {
    double v[8];
    if (fwd) {  // older positions at lower slots: one wrap check per term
#pragma unroll
      for (int u = 0; u < 8 && jb + u < AMAX; ++u) {
        v[u] = sm.ring[off];
        off -= C;
        off += off < 0 ? KC : 0;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8 && jb + u < AMAX; ++u) {
        v[u] = sm.ring[off];
        off += C;
        off -= off >= KC ? KC : 0;
      }
    }
#pragma unroll
    for (int u = 0; u < 8 && jb + u < AMAX; ++u) {
      const double w = (double)r.D[jb + u] * v[u];
      if (jb + u == 0)
        first = w;
      else
        s[u & 3] += w;
      if (WITH_GD) gd[jb + u] += (GT)(q * w);
    }
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// Sum of n values at stride `stride` (in a fixed order): reads in batches of
// 8 into separate registers so they pipeline.
__device__ __forceinline__ double sum_strided(const double *p, int n, int stride) {
  double s0 = 0.0, s1 = 0.0;
  int q = 0;
  for (; q + 8 <= n; q += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(q + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      s0 += v[u];
      s1 += v[u + 1];
    }
  }
  for (; q < n; ++q) s0 += p[q * stride];
  return s0 + s1;
}

// Maximum over the row threads of an int (others pass kNoExp).  All threads
// call; the result is meaningful on the row waves.
__device__ __forceinline__ int rows_max_i(int v, const ChainShape &sh, const Smem &sm) {
  const int w = threadIdx.x >> 6;
  const int x = w < sh.Q ? wave_max_i(v) : kNoExp;
  if (sh.Q == 1) return x;  // all row threads are in wave 0
  int *si = reinterpret_cast<int *>(sm.scal);
  if ((threadIdx.x & 63) == 0 && w < sh.Q) si[w] = x;
  __syncthreads();
  int m = si[0];
  for (int i = 1; i < sh.Q; ++i) m = max(m, si[i]);
  return m;
}

// Contraction: row thread c receives sum_{c'} e[c'] * W[c'][c] in float64
// (any per-step rounding here would accumulate along the chain).  Slice
// partials meet in LDS and the row thread adds them in a fixed order.
// Requires sm.erow written and a barrier before the call.  All threads call.
template <int AMAX, int TRMAX, typename DT>
__device__ __forceinline__ double contract(const Regs<AMAX, TRMAX, DT> &r, const Smem &sm,
                                           const ChainShape &sh, const float *__restrict__ trw) {
  using WT = typename Regs<AMAX, TRMAX, DT>::WT;
  // weights streamed from the workspace ([c_in][c_out] for this direction);
  // the base is made opaque here so the loads stay in the step loop instead
  // of being hoisted into 64 long-lived registers
  const float *base = trw;
  if (Regs<AMAX, TRMAX, DT>::kGlobalW) asm volatile("" : "+s"(base));
  const float *wp = base + (size_t)r.cq * kTrwRows * sh.C + r.cc;
  // the slice's e values two at a time (the e row starts on 16 bytes and
  // cp0 is a multiple of the even slice width, so the pairs are aligned),
  // in batches of 8 with a scheduling
  // barrier between them: hoisting every load of a wide slice would need
  // two registers per weight on top of the weights themselves.  Weights past
  // the slice are 0 (in registers and in the padded table alike) and the e
  // row has a zero tail, so no bound is checked.
  const double2 *e2 = reinterpret_cast<const double2 *>(sm.erow + r.cp0);
  double d0 = 0.0, d1 = 0.0;
  if (r.ncp > 0) {
#pragma unroll
    for (int j = 0; j < TRMAX; j += 8) {
      double2 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = e2[j / 2 + q];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        WT w0, w1;
        if (Regs<AMAX, TRMAX, DT>::kGlobalW) {
          w0 = (WT)wp[(size_t)(j + 2 * q) * sh.C];
          w1 = (WT)wp[(size_t)(j + 2 * q + 1) * sh.C];
        } else {
          w0 = r.Tr[(j + 2 * q) % (Regs<AMAX, TRMAX, DT>::kGlobalW ? 1 : TRMAX)];
          w1 = r.Tr[(j + 2 * q + 1) % (Regs<AMAX, TRMAX, DT>::kGlobalW ? 1 : TRMAX)];
        }
        if (!std::is_same<WT, double>::value && !Regs<AMAX, TRMAX, DT>::kGlobalW) {
          // keep a float32 weight live as float32: converting all TRMAX
          // weights once, outside the time loop, would double their registers
          asm volatile("" : "+v"(w0), "+v"(w1));
        }
        d0 = fma(v[q].x, (double)w0, d0);
        d1 = fma(v[q].y, (double)w1, d1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  double dp = d0 + d1;
  if (sh.QT > 1) {
    if (r.cq < sh.QT) sm.dotp[r.cq * sh.C + r.cc] = dp;
    __syncthreads();
    if ((int)threadIdx.x < sh.C) dp = sum_strided(sm.dotp + threadIdx.x, sh.QT, sh.C);
  }
  return dp;
}

// Row thread c inserts the entry for position t, y * 2^s relative to its
// reference 2^R (y > 0, s an exact integer), and decides an exact
// power-of-two rebase of its column: an entry outside
// [2^-kRebaseExp, 2^kRebaseExp] moves R by its exponent.  Returns that
// shift n (0: none); the column's older slots must be rescaled by 2^-n (n
// also in sm.shiftn[c]).  The bound
// leaves headroom for the K-sum, at most 2^kRebaseExp * K * max exp(dur),
// below float64's 2^1023 for K <= 16384 and dur below ~270 nats; older
// entries that fall below the float64 range are smaller than the newest by
// more than 2^kRebaseExp and weigh nothing.
__device__ __forceinline__ int insert_entry(const Smem &sm, const ChainShape &sh, int t,
                                            double y, int s, int &R) {
  const int c = threadIdx.x;
  const int ey = exponent_of(y) + s;
  const int n = (ey > kRebaseExp || ey < -kRebaseExp) ? ey : 0;
  R += n;
  sm.shiftn[c] = n;
  sm.ring[(t % sh.K) * sh.C + c] = ldexp(y, s - n);
  return n;
}

// Rebase votes of two consecutive steps (by step parity), in the scalar area.
__device__ __forceinline__ int *vote_of(const Smem &sm) {
  return reinterpret_cast<int *>(sm.scal) + 8;
}

// Apply pending column rescales: every ring slot except the newest (position
// t) is multiplied by 2^-shiftn[c].  Slots are owned through the durations
// of the next step, so each is touched by exactly one thread; no barrier
// here (the caller orders the rescale against the slots' other readers).
template <int AMAX, int TRMAX, typename DT>
__device__ __forceinline__ void apply_rebase(const Regs<AMAX, TRMAX, DT> &r, const Smem &sm,
                                             const ChainShape &sh, int t, bool fwd) {
  // the thread's own slots only (another thread owns every other slot, so
  // nothing past them is written); reads in batches of 8 without a branch so
  // they pipeline, stores predicated
  const int n = r.nage > 0 ? sm.shiftn[r.kc] : 0;
  if (n != 0) {
    const int K = sh.K, C = sh.C, KC = K * C;
    const int dC = fwd ? -C : C;
    const int tn = fwd ? t + 1 : t - 1;
    int off = slot_of(tn % K, min(r.age0, K), K, fwd) * C + r.kc;
#pragma unroll
    for (int jb = 0; jb < AMAX; jb += 8) {
      double v[8];
      int o[8];
#pragma unroll
      for (int u = 0; u < 8 && jb + u < AMAX; ++u) {
        o[u] = off;
        v[u] = sm.ring[off];
        off += dC;
        off += off < 0 ? KC : 0;
        off -= off >= KC ? KC : 0;
      }
#pragma unroll
      for (int u = 0; u < 8 && jb + u < AMAX; ++u) {
        const int j = jb + u;
        // duration 1 is the entry just inserted in the new reference
        if (j < r.nage && r.age0 + j >= 2) sm.ring[o[u]] = ldexp(v[u], -n);
      }
    }
  }
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
  }
  __syncthreads();
}

// Cumulative score of position t for label c (row / chain lanes; other
// lanes read label 0).  t is clamped into [0, T], so every lane loads from a
// valid address and no select touches the loaded value: the load stays in
// flight until its first use (a prefetch).
__device__ __forceinline__ double es_raw(const Escaled &es, size_t ob, int t, int T, int C, int c) {
  const int tc = t < 0 ? 0 : (t > T ? T : t);
  return es.S[ob + (size_t)tc * C + (c < C ? c : 0)];
}

// The split of a score in the order the direction uses it: fx multiplies
// the K-sum (exp(S) forward, exp(-S) backward), fy the contraction (the
// other one), n is the exponent (its sign is applied where it is used).
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

// Log rows from a step's staged values (stg: x[C], E[C], d[C], B), rows
// [lo, hi) of the 2C (alpha / v first, then u / beta), shared by threads
// [first, first + nthr).
__device__ __forceinline__ void stage_rows(const double *stg, int C, double *r1, double *r2,
                                           int lo, int hi, int first, int nthr) {
  for (int i = lo + (int)threadIdx.x - first; i < hi; i += nthr) {
    if (i < C)
      r1[i] = log(stg[i]) + stg[C + i] * kLn2;
    else
      r2[i - C] = log(stg[C + i]) + stg[3 * C] * kLn2;
  }
}

// ---------------------------------------------------------------- sweeps
// One workgroup per (direction, sequence b, chunk j), chunk = [p0, p1): the
// forward chain runs t = p0+1 .. p1 from the state at p0, the backward chain
// t = p1-1 .. p0 from the state at p1 (parallel-in-time; pit.hip verifies and
// normalises).  The start state is the chunk's checkpoint record: built at
// iteration 0 (exact at the sequence end the chain starts from, neutral
// elsewhere), re-read afterwards.  The chunk that ends its chain yields log Z
// in its own frame; every other chunk writes its end state.
// Wave roles of the LDS-ring engine: row waves (w < Q), loader waves
// (Q <= w < Q + nload), writer waves (the rest).
enum ChainRole { kRowRole = 0, kLoadRole = 1, kWriteRole = 2 };

// Loader: the split scores of the prefetch block starting at step s (steps
// s .. s+pf-1, positions tstart + isig*step) for every label, pf*C pairs
// over the loader lanes, at most kMaxPairs each.  issue() only loads the
// scores; put() -- a block later -- splits and stores them.
struct PfLoad {
  double sv[kMaxPairs];

  __device__ __forceinline__ void issue(const Escaled &es, size_t ob, const ChainShape &sh,
                                        int tstart, int isig, int s, int lid) {
#pragma unroll
    for (int k = 0; k < kMaxPairs; ++k) {
      const int q = lid + 64 * sh.nload * k;  // pair (i, c) = (q / C, q % C)
      const bool in = q < sh.pf * sh.C;
      const int i = in ? q / sh.C : 0, c = in ? q % sh.C : 0;
      sv[k] = es_raw(es, ob, tstart + isig * (s + i), sh.T, sh.C, c);
    }
  }

  __device__ __forceinline__ void put(const Smem &sm, const ChainShape &sh, int buf, int lid,
                                      bool fwd) const {
#pragma unroll
    for (int k = 0; k < kMaxPairs; ++k) {
      const int q = lid + 64 * sh.nload * k;
      if (q < sh.pf * sh.C) {
        const int o = buf * sh.pf * sh.C + q;  // [buf][i][c], q = i*C + c
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

// The step loop of one role.  Per step: K-sum share, barrier (then the
// previous step's rebases reach the ring), row phase (label maximum, with a
// barrier when the rows span several waves), barrier, contraction (a
// barrier when it is split), insertion with the rebase vote; a step that
// stores a record adds a barrier and applies its own rebase at once.  The
// row threads leave log Z (tail chunk) or the end-state o / m in lz /
// o_end / m_end.
// Steps 1..nsteps run at positions tb + sigma*step; the first wb of them are
// a burn-in (no rows), after which the state is the chunk's start record.
template <int ROLE, int NT, int AMAX, int TRMAX, typename DT>
__device__ __forceinline__ void sweep_loop(const ChainShape &sh, const Smem &sm,
                                           const Regs<AMAX, TRMAX, DT> &r, const Escaled &es,
                                           size_t ob, int tb, int nsteps, int wb,
                                           double *rec_start, bool fwd, bool tail, bool rows,
                                           double *row1, double *row2, int rt0, const float *trw,
                                           int &R, double &o_end, double &m_end, double &lz) {
  const int tid = threadIdx.x, C = sh.C;
  const bool is_row = tid < C;
  const int isig = fwd ? 1 : -1;
  const int pf = sh.pf;
  const int lid = tid - 64 * sh.Q;  // loader lane
  const int wfirst = 64 * (sh.Q + sh.nload), wn = NT - wfirst;  // writer threads
  const int tstart = tb;
  double o_rec = 0.0, m_rec = 0.0;
  int Bm = -(1 << 29);  // step scale of the rows; the first step computes it
  // A rebase decided at one step reaches the ring's older slots during the
  // next one, after its first barrier (uniform `lazy`, the vote of the step
  // before); that step's K-sum still reads them in the old reference, so
  // the row thread scales all but the newest term by 2^-npend, its label's
  // shift.  The steps that store a record apply their rebases at once.
  int npend = 0;
  bool lazy = false;
  PfLoad ld;
  for (int step = 1; step <= nsteps; ++step) {
    const int t = tb + isig * step;
    const int i = pf > 0 ? (step - 1) % pf : 0;  // position in the prefetch block
    const int buf = pf > 0 ? ((step - 1) / pf) & 1 : 0;
    double fx = 0.0, fy = 0.0;
    int nq = 0;
    if (ROLE == kRowRole && is_row && pf == 0) {  // (prefetched scores: after the first barrier)
      int n;
      es_get(es, ob, t, sh.T, C, tid, fwd, fx, fy, n);
      nq = isig * n;
    }
    const bool next_blk = pf > 0 && step - 1 - i + pf < nsteps;  // a block follows this one
    if (ROLE == kLoadRole && i == 0 && next_blk)
      ld.issue(es, ob, sh, tstart, isig, step + pf, lid);
    double nogd[AMAX];
    double first = 0.0;  // the thread's first term (the row threads': duration 1, the newest entry)
    const double s = r.kp < sh.P ? ksum<false>(r, sm, sh, t, fwd, nogd, 0.0, first) : 0.0;
    if (r.kp < sh.P) sm.part[r.kp * C + r.kc] = r.kp == 0 ? s : s + first;
    __syncthreads();
    // the previous step's rebases (every thread rescales the slots it has
    // just read; the next readers are past the barriers below)
    if (lazy && vote_of(sm)[(step - 1) & 1]) apply_rebase(r, sm, sh, t - isig, fwd);
    if (ROLE == kRowRole && is_row && pf > 0) {
      const int o = (buf * pf + i) * C + tid;
      fx = sm.efx[o];
      fy = sm.efy[o];
      nq = isig * sm.en[o];
    }
    const bool last = step == nsteps;
    const bool lz_step = last && tail;
    const double *sprev = sm.stg + ((step - 1) & 1) * (3 * C + 1);
    const size_t tprev = (size_t)(t - isig - rt0) * C;  // rows are window-relative
    // exp(o) = x * 2^E, o = alpha (forward) or v (backward)
    double x = 0.0;
    int E = 0;
    if (ROLE == kRowRole && is_row) {
      x = (ldexp(sum_strided(sm.part + tid, sh.P, C), -npend) + first) * fx;
      E = R + nq;
    }
    const bool prev_rows = rows && step - 1 > wb;  // the previous step is past the burn-in
    if (ROLE == kWriteRole && prev_rows)
      stage_rows(sprev, C, row1 + tprev, row2 + tprev, 0, C, wfirst, wn);
    // the step scale: with the rows in one wave it carries over from step to
    // step and is recomputed (an exact integer maximum) only when some
    // label's exponent leaves [Bm - kScaleSpan, Bm + kScaleSpan], as in
    // chain_win.hip; every value stays exact either way
    const int ex = (is_row && x > 0.0) ? E + exponent_of(x) : kNoExp;
    if (sh.Q == 1) {
      if (__any(ex - Bm > kScaleSpan) || !__any(ex - Bm >= -kScaleSpan)) Bm = wave_max_i(ex);
    } else {
      Bm = rows_max_i(ex, sh, sm);
    }
    double *stg = sm.stg + (step & 1) * (3 * C + 1);
    if (ROLE == kRowRole && is_row) {
      stg[tid] = x;
      stg[C + tid] = (double)E;
      sm.erow[tid] = ldexp(x, E - Bm);  // exp(o) / 2^Bm
    }
    __syncthreads();
    if (lz_step) {
      if (ROLE == kRowRole && tid == 0) {
        double z = 0.0;
        for (int c = 0; c < C; ++c) z += sm.erow[c];
        lz = (double)Bm * kLn2 + log(z);
      }
      if (ROLE == kWriteRole && prev_rows)
        stage_rows(sprev, C, row1 + tprev, row2 + tprev, C, 2 * C, wfirst, wn);
      break;  // the chain's last step (uniform)
    }
    const double d = contract(r, sm, sh, trw);  // exp(m) / 2^Bm, m = u or beta
    if (ROLE == kWriteRole && prev_rows)
      stage_rows(sprev, C, row1 + tprev, row2 + tprev, C, 2 * C, wfirst, wn);
    int *vote = vote_of(sm);  // rebase votes of two steps
    if (ROLE == kRowRole && is_row) {
      if (tid == 0) vote[(step + 1) & 1] = 0;  // every thread has read it (last step)
      stg[2 * C + tid] = d;
      if (tid == 0) stg[3 * C] = (double)Bm;
      // entry exp(m -+ S) / 2^R = d * fy * 2^(Bm -+ n - R)
      npend = insert_entry(sm, sh, t, d * fy, Bm - nq - R, R);
      if (npend != 0) vote[step & 1] = 1;
      if (last || step == wb) {
        const double o = log(x) + (double)E * kLn2, m = log(d) + (double)Bm * kLn2;
        if (last) {
          o_end = o;
          m_end = m;
        } else {
          o_rec = o;
          m_rec = m;
        }
      }
    }
    // the next block's scores land in the other buffer before the next
    // step's first barrier, after which the row threads read them
    if (ROLE == kLoadRole && i == pf - 1 && next_blk) ld.put(sm, sh, buf ^ 1, lid, fwd);
    if (last || step == wb) {  // a record follows: the ring made whole now
      __syncthreads();
      if (vote[step & 1]) {
        apply_rebase(r, sm, sh, t, fwd);
        __syncthreads();
      }
      npend = 0;
      lazy = false;
      if (step == wb) save_ckpt(rec_start, sm, sh, R, o_rec, m_rec);  // the burn-in ends
    } else {
      lazy = true;
    }
  }
}

template <int NT, int AMAX, int TRMAX, typename DT>
__global__ __launch_bounds__(NT) void k_sweep(ChainShape sh, const float *__restrict__ trans,
                                              const float *__restrict__ dur, Escaled es,
                                              const int32_t *__restrict__ lengths, PitBufs pb,
                                              int iter) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int nck = sh.B * sh.nchunk;
  const bool replay = iter < 0;  // a window of chunks swept again from exact records
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
      for (int i = threadIdx.x; i < sh.nchunk; i += NT) pb.nbad[i] = 0;
  }
  const int L = lengths[b];
  const int tid = threadIdx.x, C = sh.C, K = sh.K;
  const bool is_row = tid < C;
  if (L < 1 || L > sh.T || jc >= sh.nchunk) return;
  const int p0 = jc * sh.delta;
  if (p0 >= L) return;
  const int p1 = min(p0 + sh.delta, L);
  if (iter > 0 && (pb.nbad[iter - 1] == 0 || pb.redo[idx] == 0)) return;
  const int rt0 = pb.row_t0;
  Smem sm = carve(lds, sh);
  for (int i = tid; i < kErowPad; i += NT) sm.erow[sh.C + i] = 0.0;
  Regs<AMAX, TRMAX, DT> r;
  init_regs(r, sh, dur);
  load_trans(r, sh, trans, fwd);
  const float *trw = pb.trw ? pb.trw + (fwd ? 0 : trw_floats(sh.C, sh.QT) / 2) : nullptr;
  const size_t ob = (size_t)b * (sh.T + 1) * C;
  const size_t cks = ck_stride(C, K);
  double *rec_start = (fwd ? pb.ck_fwd : pb.ck_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  double *rec_end = (fwd ? pb.end_fwd : pb.end_bwd) + ((size_t)b * sh.nchunk + jc) * cks;
  const int isig = fwd ? 1 : -1;
  const int tstart = fwd ? p0 : p1;
  const bool tail = fwd ? (p1 == L) : (p0 == 0);  // this chunk ends the chain
  const bool rows = pb.row_a != nullptr;
  const size_t orow = (size_t)b * pb.row_stride * C;
  double *row1 = rows ? (fwd ? pb.row_a : pb.row_v) + orow : nullptr;  // alpha / v
  double *row2 = rows ? (fwd ? pb.row_u : pb.row_b) + orow : nullptr;  // u / beta

  int R = 0;
  // burn-in of a chunk without an exact start at iteration 0 (see chain_win.hip)
  const bool exact = fwd ? (jc == 0) : (p1 == L);
  const int wb = (iter == 0 && !exact) ? min(sh.burn, fwd ? p0 : L - p1) : 0;
  const int tb = fwd ? p0 - wb : p1 + wb;  // where the sweep starts
  if (iter == 0) {
    for (int i = tid; i < K * C; i += NT) sm.ring[i] = 0.0;
    __syncthreads();
    if (exact) {
      // entry u[0] - S[0] = 0 forward; beta[L] + S[L] = S[L] backward
      if (is_row) {
        double v = 1.0;
        if (!fwd) {  // exp(S[L]) = ep * 2^n
          double em;
          exp_split(es.S[ob + (size_t)L * C + tid], v, em, R);
        }
        sm.ring[(tstart % K) * C + tid] = v;
      }
    } else {
      // neutral start: every entry of the window (positions inside [0, L]) is 1
      for (int i = tid; i < K * C; i += NT) {
        const int dq = i / C, c = i % C;
        const int q = tb - isig * dq;
        if (q >= 0 && q <= L) sm.ring[(q % K) * C + c] = 1.0;
      }
    }
    __syncthreads();
    // o = NaN marks a neutral start (never accepted by the verification);
    // after a burn-in the record is written when the sweep reaches tstart
    if (wb == 0)
      save_ckpt(rec_start, sm, sh, R, exact ? -__builtin_huge_val() : __builtin_nan(""),
                exact ? 0.0 : __builtin_nan(""));
    if (exact && is_row && rows)  // u[0] = 0 forward, beta[L] = 0 backward
      row2[(size_t)(tstart - rt0) * C + tid] = 0.0;
    __syncthreads();
  } else {
    double o0, m0;
    load_ckpt(rec_start, sm, sh, R, o0, m0);
    // a replay window's first row (its chunk before is not swept again): the
    // record's exact outputs at the start position
    if (replay && rows && is_row &&
        (fwd ? jc == sh.rj0 : (jc == sh.rj0 + sh.rnb - 1 || p1 == L))) {
      row1[(size_t)(tstart - rt0) * C + tid] = o0;
      row2[(size_t)(tstart - rt0) * C + tid] = m0;
    }
  }
  const int nsteps = wb + (p1 - p0);
  if (sh.pf > 0) {  // the first block's scores (later blocks: the loader waves)
    const int npair = min(sh.pf, nsteps) * C;
    for (int q = tid; q < npair; q += NT) {
      double fx, fy;
      int n;
      es_get(es, ob, tb + isig * (1 + q / C), sh.T, C, q % C, fwd, fx, fy, n);
      sm.efx[q] = fx;
      sm.efy[q] = fy;
      sm.en[q] = n;
    }
  }
  if (tid == 0) {  // rebase votes of the first two steps
    reinterpret_cast<int *>(sm.scal)[8] = 0;
    reinterpret_cast<int *>(sm.scal)[9] = 0;
  }
  vm_drain();
  __syncthreads();

  double o_end = 0.0, m_end = 0.0, lz = 0.0;
  const int w = tid >> 6;
  if (w < sh.Q)
    sweep_loop<kRowRole, NT>(sh, sm, r, es, ob, tb, nsteps, wb, rec_start, fwd, tail, rows,
                             row1, row2, rt0, trw, R, o_end, m_end, lz);
  else if (w < sh.Q + sh.nload)
    sweep_loop<kLoadRole, NT>(sh, sm, r, es, ob, tb, nsteps, wb, rec_start, fwd, tail, rows,
                              row1, row2, rt0, trw, R, o_end, m_end, lz);
  else
    sweep_loop<kWriteRole, NT>(sh, sm, r, es, ob, tb, nsteps, wb, rec_start, fwd, tail, rows,
                               row1, row2, rt0, trw, R, o_end, m_end, lz);
  if (!replay) {
    if (tail) {
      if (tid == 0) pb.lz_part[(fwd ? 0 : sh.B) + b] = lz;
    } else {
      save_ckpt(rec_end, sm, sh, R, o_end, m_end);
    }
  }
  if (rows) {  // rows of the last step (t = p1 forward, p0 backward)
    __syncthreads();
    const size_t tl = (size_t)((fwd ? p1 : p0) - rt0) * C;
    stage_rows(sm.stg + (nsteps & 1) * (3 * C + 1), C, row1 + tl, row2 + tl, 0,
               tail ? C : 2 * C, 0, NT);
  }
}

// exp(trans) in float32 for the instances that stream their weights, one
// block of kTrwRows rows per contraction slice q (previous labels
// c_in = q*CS + j, row j < CS; rows past the slice or past C are 0):
// trw[0][q][j][c_out] = exp(trans[c_in][c_out]) (forward contraction) and
// trw[1][q][j][c_out] = exp(trans[c_out][c_in]) (backward).
__global__ void k_trw(int C, int CS, int QT, const float *__restrict__ trans,
                      float *__restrict__ trw) {
  const int per = kTrwRows * C, n = QT * per;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < 2 * n; i += gridDim.x * blockDim.x) {
    const int d = i / n, e = i % n, q = e / per, j = (e % per) / C, co = e % C;
    const int ci = q * CS + j;
    float w = 0.0f;
    if (j < CS && ci < C)
      w = (float)exp((double)(d == 0 ? trans[(size_t)ci * C + co] : trans[(size_t)co * C + ci]));
    trw[i] = w;
  }
}

hipError_t launch_trw(int C, int CS, int QT, const float *trans, float *trw, hipStream_t st) {
  const size_t n = trw_floats(C, QT);
  int grid = (int)((n + 255) / 256);
  grid = grid > 1024 ? 1024 : grid;
  hipLaunchKernelGGL(k_trw, dim3(grid), dim3(256), 0, st, C, CS, QT, trans, trw);
  return hipGetLastError();
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
                          const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                          int with_bwd, int iter, hipStream_t st) {
    const size_t lds = chain_lds_bytes(sh.C, sh.K, sh.P, sh.QT, sh.pf);
    set_attrs();
    if (!lds_fits((const void *)k_sweep<NT, AMAX, TRMAX, DT>, lds))
      return report(hipErrorInvalidConfiguration, "k_sweep (LDS)", sh, lds);
    const int grid = iter < 0 ? sh.B * (sh.rnf + sh.rnb) : (with_bwd ? 2 : 1) * sh.B * sh.nchunk;
    hipLaunchKernelGGL((k_sweep<NT, AMAX, TRMAX, DT>), dim3(grid), dim3(NT), lds, st, sh, trans,
                       dur, es, lengths, pb, iter);
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
                        const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                        int with_bwd, int iter, hipStream_t st) {
  if (sh.win) return launch_sweep_w(sh, trans, dur, es, lengths, pb, with_bwd, iter, st);
  if (sh.e64) return launch_sweep_64(sh, trans, dur, es, lengths, pb, with_bwd, iter, st);
  if (sh.e256) return launch_sweep_256(sh, trans, dur, es, lengths, pb, with_bwd, iter, st);
  SEMICRF_CHAIN_DISPATCH(sh, sweep(sh, trans, dur, es, lengths, pb, with_bwd, iter, st));
}

}  // namespace semicrf
