// vpit.hip -- parallel-in-time Viterbi decoding on gfx950.
//
// The pages give no decoder; this is the (max,+) form of the forward
// recurrence over the segment scores that the cumulative scores S give on
// the fly ("Streaming Structured Inference with Flash-SemiCRF", abstract;
// technical summary, section 2.A):
//   ahat[t,c] = S[t,c] + max_{k <= min(K,t)} (dur[k-1,c] + ghat[t-k,c])   argmax k
//   uhat[t,c] = max_{c'} (ahat[t,c'] + trans[c',c]),  uhat[0,.] = 0        argmax c'
//   ghat[t,c] = uhat[t,c] - S[t,c];  best = max_c ahat[L,c]
// with the tie rule of viterbi.hip (a candidate within 1e-11 (|max| + 1) of
// the maximum ties; smallest k, then smallest c', then smallest final c).
//
// Parallel in time.  The state at a position is the ring of the K newest
// ghat rows.  Max-plus is shift-equivariant: start the recursion from a
// state that differs from the true one by a constant and every later value
// differs by that constant, every decision is the same.  And it forgets its
// start: after enough positions the optimal paths from all start entries
// run through common nodes, and the state differs from the true one by a
// constant, whatever the start.  So the positions are cut into chunks that
// run concurrently, one workgroup each:
//   1. relative sweep: chunk j starts `burn` positions early from a neutral
//      state (every start entry 0; a chunk whose burn-in reaches position 0
//      starts from the true state there), records its state at its first
//      position p0 (R_j) and at its end p1 (E_j);
//   2. verification: chunk j is consistent when R_j - E_{j-1} is one
//      constant over the ring (up to rounding); the constant is recorded.
//      Otherwise E_{j-1} becomes R_j and the chunk is swept again; a second
//      parallel pass, then one workgroup per sequence repairs what is left
//      in order, so the result never depends on how fast the starts forget;
//   3. the prefix sums of the constants give each chunk's frame offset, and
//      an absolute sweep from R_j minus that offset -- the true state up to
//      rounding, so the tie tolerance sees the true magnitudes -- takes and
//      stores the decisions.
// One sweep step: every label group takes the maximum over its durations
// and the smallest tied k by DPP within the group, writes ahat to LDS; one
// LDS-only barrier; every group takes the maximum over previous labels and
// the smallest tied c' the same way and writes ghat into its own ring row.
// Scores S arrive in blocks of U positions staged through LDS (loads issued
// a block ahead, so the barriers never wait for them), and the decisions
// leave in blocks of U from registers.
//
// Backtrack, parallel too: a gather pass turns the decisions into one
// predecessor word per (t, c); each sub-chunk of dbt >= K positions walks
// back from a guessed entry node and marks the nodes it visits; then the
// walk from the true entry (the exit of the successor sub-chunk's walk) is
// followed until it meets a marked node -- from there on the two walks
// coincide -- and a serial repair covers the rare sub-chunk whose walks do
// not meet.  Segment counts, their prefix sums, and a parallel write give
// the segments in start order.
#include "device_math.h"
#include "internal.h"

namespace semicrf {

namespace {

constexpr double kVitTol = 0x1p-40;  // deviation from one constant offset, relative to the values
constexpr int kVHelp = 256;          // threads of the helper kernels
constexpr int kNoArg = 0x7fffffff;

// sub-chunk fields
//   N: nodes of the guessed walk; Ex: its exit node (the first node at or
//   before lo); En: entry node of the true path; H: true-path nodes before it
//   meets the guessed walk; Mi: index in the guessed walk where it meets (N
//   if never); Tx: exit node of the true path; Off: index of its first
//   segment in the output (segments of later sub-chunks come after)
enum { kSubN = 0, kSubExT, kSubExC, kSubEnT, kSubEnC, kSubH, kSubMi, kSubTxT, kSubTxC, kSubOff };
static_assert(kSubOff < kVSubFields, "sub-chunk record too small");

__device__ __forceinline__ size_t rec_base(const VShape &vs, int b, int j) {
  return ((size_t)b * vs.nchunk + j) * (size_t)vs.K * vs.C;
}

// Per-thread constants of a sweep workgroup.
template <int AMAX, int CAMAX>
struct VRegs {
  float dr[AMAX];   // dur[k-1][c] for k = g + 1 + NG*a
  float tr[CAMAX];  // trans[c'][c] for c' = g + NG*i
  int c, g;
  bool on;
};

template <int AMAX, int CAMAX>
__device__ __forceinline__ void vregs_init(VRegs<AMAX, CAMAX> &r, const VShape &vs,
                                           const float *__restrict__ trans,
                                           const float *__restrict__ dur) {
  const int tid = threadIdx.x, C = vs.C, K = vs.K, NG = vs.NG;
  r.c = tid / NG;
  r.g = tid % NG;
  r.on = r.c < C;
#pragma unroll
  for (int a = 0; a < AMAX; ++a) {
    const int k = r.g + 1 + NG * a;
    r.dr[a] = (r.on && a < vs.A && k <= K) ? dur[(size_t)(k - 1) * C + r.c] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < CAMAX; ++i) {
    const int cp = r.g + NG * i;
    r.tr[i] = (r.on && i < vs.CA && cp < C) ? trans[(size_t)cp * C + r.c] : 0.0f;
  }
}

// A float32 constant converted to float64 where it is used.  In the wide
// instances the opaque copy keeps the conversion inside the step loop, where
// hoisting it would hold two registers per constant for the whole loop.
template <bool OPAQUE>
__device__ __forceinline__ double wide(float v) {
  if (OPAQUE) asm volatile("" : "+v"(v));
  return (double)v;
}

// LDS of a sweep workgroup.
struct VSmem {
  double *ring;  // [C][K] ghat by position mod K
  double *arow;  // [2][C] ahat of the current position (double buffered)
  double *sst;   // [2][U][C] staged scores
  int *flag;     // [NT / 64] verification votes
};

__device__ __forceinline__ VSmem vsmem(const VShape &vs, unsigned char *lds) {
  VSmem sm;
  sm.ring = reinterpret_cast<double *>(lds);
  sm.arow = sm.ring + (size_t)vs.C * vs.K;
  sm.sst = sm.arow + 2 * vs.C;
  sm.flag = reinterpret_cast<int *>(sm.sst + (size_t)2 * vs.U * vs.C);
  return sm;
}

// Modes of a sweep.
enum { kRel = 0, kRedo = 1, kAbs = 2 };

// Sweep chunk j of sequence b (all NT threads).  kRel: from a neutral (or,
// if the burn-in reaches 0, the true) state `burn` positions before p0,
// recording R_j at p0 and E_j at p1; kRedo: from R_j at p0, recording E_j;
// kAbs: from R_j minus the chunk's frame offset, storing the decisions of
// (p0, p1] and, for the last chunk, the best final label.
// NGT: the label-group width as a compile-time constant (0: vs.NG), so the
// wide instances address their previous labels by immediate offsets.
template <int NT, int AMAX, int CAMAX, int NGT>
__device__ __forceinline__ void vsweep(const VShape &vs, const VRegs<AMAX, CAMAX> &r,
                                       const VSmem &sm, int mode, int b, int j, int L,
                                       const double *__restrict__ S, const VBufs &vb) {
  constexpr bool kWide = CAMAX > 4;
  const int C = vs.C, K = vs.K, NG = NGT ? NGT : vs.NG, U = vs.U, T = vs.T;
  const int tid = threadIdx.x;
  const int p0 = j * vs.delta, p1 = min(p0 + vs.delta, L);
  const int q = mode == kRel ? p0 - min(vs.burn, p0) : p0;  // the sweep takes positions (q, p1]
  const size_t rb = rec_base(vs, b, j);
  const double off = mode == kAbs ? vb.delta[(size_t)b * vs.nchunk + j] : 0.0;
  for (int i = tid; i < C * K; i += NT) {
    double v = 0.0;
    if (mode != kRel) v = vb.rec_r[rb + i] - off;
    sm.ring[i] = v;
  }
  if (mode == kRel && q == p0)
    for (int i = tid; i < C * K; i += NT) vb.rec_r[rb + i] = 0.0;
  const double *Sb = S + (size_t)b * (T + 1) * C;
  const int nst = U * C;  // staged values per block
  for (int i = tid; i < nst; i += NT) {
    const int row = min(q + 1 + i / C, T);
    sm.sst[i] = Sb[(size_t)row * C + i % C];
  }
  __syncthreads();

  const int c = r.on ? r.c : 0, g = r.g;
  const double ninf = -__builtin_huge_val();
  // decisions of (t, c) at bpc[t - bp_t0] (kAbs only)
  uint32_t *bpc = vb.bp + ((size_t)b * C + c) * vs.bp_stride;
  const int bt0 = vs.bp_t0;
  int kslot = (((q - g) % K) + K) % K;  // slot of position t - 1 - g at t = q + 1
  int tslot = (q + 1) % K;              // slot of position t
  double sreg = 0.0;  // this thread's staged score of the next block (U*C <= NT)
  uint32_t dec = 0;
  const int nsteps = p1 - q;

  // (always inlined: an outlined step would keep the register arrays in memory)
  auto step = [&](int s) __attribute__((always_inline)) {
    const int t = q + 1 + s;
    const int w = s & (U - 1), blk = s / U;
    if (w == 0 && tid < nst) {  // scores of the next block, needed U steps from now
      const int row = min(q + 1 + (blk + 1) * U + tid / C, T);
      sreg = Sb[(size_t)row * C + tid % C];
    }
    // durations: max over k and the smallest tied k.  Every candidate is
    // read without a branch (the slot clamped into the ring; invalid ones
    // masked afterwards), in batches of 8, so the reads pipeline.
    const int kmax = min(K, t);
    const double *rc = sm.ring + c * K;
    // (the wide instances, short of registers, keep one guarded read per
    // candidate and read again for the smallest tied k)
    constexpr bool kFlat = CAMAX <= 4;
    double cand[kFlat ? AMAX : 1];
    double m = ninf;
    if constexpr (kFlat) {
#pragma unroll
    for (int ab = 0; ab < AMAX; ab += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8 && ab + u < AMAX; ++u) {
        int sl = kslot - NG * (ab + u);
        sl += sl < 0 ? K : 0;
        sl = sl < 0 ? 0 : sl;
        v[u] = rc[sl];
      }
#pragma unroll
      for (int u = 0; u < 8 && ab + u < AMAX; ++u) {
        const int a = ab + u, k = g + 1 + NG * a;
        const bool ok = r.on && a < vs.A && k <= kmax;
        cand[a] = ok ? wide<kWide>(r.dr[a]) + v[u] : ninf;
      }
    }
#pragma unroll
    for (int a = 0; a < AMAX; ++a) m = fmax(m, cand[a]);
    } else {
#pragma unroll
      for (int a = 0; a < AMAX; ++a) {
        const int k = g + 1 + NG * a;
        if (r.on && a < vs.A && k <= kmax) {
          int sl = kslot - NG * a;
          sl += sl < 0 ? K : 0;
          m = fmax(m, wide<kWide>(r.dr[a]) + rc[sl]);
        }
      }
    }
    const double M = group_max(m, NG);
    const double st = sm.sst[((blk & 1) * U + w) * C + c];
    const double ah = st + M;
    const double thr = M - viterbi_tie_eps(ah);
    int kb = kNoArg;
    if constexpr (kFlat) {
#pragma unroll
      for (int a = AMAX - 1; a >= 0; --a)
        if (cand[a] >= thr) kb = g + 1 + NG * a;  // invalid candidates are -inf
    } else {
      if (AMAX > 4) asm volatile("" ::: "memory");  // read again rather than hold
#pragma unroll
      for (int a = AMAX - 1; a >= 0; --a) {
        const int k = g + 1 + NG * a;
        if (r.on && a < vs.A && k <= kmax) {
          int sl = kslot - NG * a;
          sl += sl < 0 ? K : 0;
          if (wide<kWide>(r.dr[a]) + rc[sl] >= thr) kb = k;
        }
      }
    }
    kb = group_min_i(kb, NG);
    if (r.on && g == 0) sm.arow[(t & 1) * C + c] = ah;
    // stage the next block (its buffer was last read a block ago)
    if (w == U - 1 && s + 1 < nsteps && tid < nst) sm.sst[((blk + 1) & 1) * nst + tid] = sreg;
    lds_barrier();
    // previous labels: max over c' and the smallest tied c'
    int cb = 0xffff;
    if (t < L) {
      const double *ar = sm.arow + (t & 1) * C;
      double m2 = ninf;
#pragma unroll
      for (int i = 0; i < CAMAX; ++i) {
        const int cp = g + NG * i;
        const bool ok = r.on && i < vs.CA && cp < C;
        if constexpr (CAMAX <= 4) {
          const double v = ar[ok ? cp : 0] + wide<kWide>(r.tr[i]);  // read without a branch
          m2 = fmax(m2, ok ? v : ninf);
        } else if (ok) {
          m2 = fmax(m2, ar[cp] + wide<kWide>(r.tr[i]));
        }
        // batches of 8 loads: hoisting all of them would take two registers each
        if (CAMAX > 8 && (i & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      }
      const double M2 = group_max(m2, NG);
      if (CAMAX > 4) asm volatile("" ::: "memory");
      const double thr2 = M2 - viterbi_tie_eps(M2);
      int cl = kNoArg;
#pragma unroll
      for (int i = CAMAX - 1; i >= 0; --i) {
        const int cp = g + NG * i;
        const bool ok = r.on && i < vs.CA && cp < C;
        if constexpr (CAMAX <= 4) {
          const double v = ar[ok ? cp : 0] + wide<kWide>(r.tr[i]);
          if (ok && v >= thr2) cl = cp;
        } else if (ok && ar[cp] + wide<kWide>(r.tr[i]) >= thr2) {
          cl = cp;
        }
        if (CAMAX > 8 && (i & 7) == 0) __builtin_amdgcn_sched_barrier(0);
      }
      cb = group_min_i(cl, NG) & 0xffff;
      if (r.on && g == 0) sm.ring[c * K + tslot] = M2 - st;
    }
    if (mode == kAbs) {
      if (g == w) dec = (uint32_t)(kb & 0xffff) | ((uint32_t)cb << 16);
      if (w == U - 1 || s + 1 == nsteps) {
        if (r.on && g <= w) bpc[t - w + g - bt0] = dec;
      }
    }
    kslot = kslot + 1 == K ? 0 : kslot + 1;
    tslot = tslot + 1 == K ? 0 : tslot + 1;
  };

  int s = 0;
  if (mode == kRel && q < p0) {
    for (; s < p0 - q; ++s) step(s);
    lds_barrier();
    for (int i = tid; i < C * K; i += NT) vb.rec_r[rb + i] = sm.ring[i];
  }
  for (; s < nsteps; ++s) step(s);
  lds_barrier();
  if (mode != kAbs) {
    for (int i = tid; i < C * K; i += NT) vb.rec_e[rb + i] = sm.ring[i];
  } else if (p1 == L && tid < 64) {
    // best final label: maximum of ahat[L, .], smallest tied label
    const double *ar = sm.arow + (L & 1) * C;
    double m = ninf;
    for (int cc = tid; cc < C; cc += 64) m = fmax(m, ar[cc]);
    const double M = group_max(m, 64);
    const double thr = M - viterbi_tie_eps(M);
    int cl = kNoArg;
    for (int cc = tid; cc < C; cc += 64)
      if (cl == kNoArg && ar[cc] >= thr) cl = cc;
    cl = group_min_i(cl, 64);
    if (tid == 0) {
      vb.vbest[b] = M;
      vb.vcbest[b] = cl == kNoArg ? 0 : cl;
    }
  }
  __syncthreads();  // the LDS is reused by the caller
}

// Consistency of chunk j (>= 1) with chunk j-1 (all threads of the block):
// R_j - E_{j-1} must be one constant over the ring entries of positions
// (p0 - K, p0] that exist.  Records the constant, or makes E_{j-1} the start
// of chunk j and marks it for another sweep.  Returns true if consistent.
// With `force` the test is skipped and E_{j-1} becomes the start: for a
// chunk already marked, whose E_j does not follow from R_j yet.
__device__ bool vverify(const VShape &vs, int b, int j, const VBufs &vb, int *flag, int iter,
                        bool force = false) {
  const int C = vs.C, K = vs.K, tid = threadIdx.x, nt = blockDim.x;
  const int p0 = j * vs.delta;
  double *R = vb.rec_r + rec_base(vs, b, j);
  const double *E = vb.rec_e + rec_base(vs, b, j - 1);
  const int s0 = p0 % K;
  const double r0 = R[s0], e0 = E[s0];  // label 0, position p0
  const double d = r0 - e0;
  const double mag0 = fabs(r0) + fabs(e0) + 1.0;
  int bad = 0;
  for (int i = tid; i < C * K; i += nt) {
    const int sl = i % K;
    const int pos = p0 - ((p0 - sl) % K + K) % K;
    if (pos < 0) continue;
    const double rv = R[i], ev = E[i];
    const double dev = fabs((rv - ev) - d);
    if (!(dev <= kVitTol * (fabs(rv) + fabs(ev) + mag0))) bad = 1;
  }
  bad = __any(bad);
  if ((tid & 63) == 0) flag[tid >> 6] = bad;
  __syncthreads();
  bad = force ? 1 : 0;
  for (int w = 0; w < nt / 64; ++w) bad |= flag[w];
  const size_t idx = (size_t)b * vs.nchunk + j;
  __syncthreads();  // every read of R precedes the copy below
  if (!bad) {
    if (tid == 0) {
      vb.corr[idx] = d;
      vb.redo[idx] = 0;
    }
  } else {
    for (int i = tid; i < C * K; i += nt) R[i] = E[i];
    if (tid == 0) {
      vb.corr[idx] = 0.0;
      vb.redo[idx] = 1;
      if (iter >= 0) atomicAdd(&vb.nbad[iter], 1);
    }
  }
  __syncthreads();
  return !bad;
}

template <int NT, int AMAX, int CAMAX, int NGT>
__global__ __launch_bounds__(NT) void k_vsweep(VShape vs, int mode, int iter,
                                               const float *__restrict__ trans,
                                               const float *__restrict__ dur,
                                               const double *__restrict__ S,
                                               const int32_t *__restrict__ lengths, VBufs vb) {
  extern __shared__ __align__(16) unsigned char lds[];
  // kAbs: the chunks aj0 .. aj0+anj-1 (all of them, or one low-memory window)
  const int nj = mode == kAbs ? vs.anj : vs.nchunk, j0 = mode == kAbs ? vs.aj0 : 0;
  const int b = blockIdx.x / nj, j = j0 + blockIdx.x % nj;
  const int L = lengths[b];
  if (L < 1 || L > vs.T) {
    if (mode == kAbs && j == 0 && threadIdx.x == 0) {
      vb.vbest[b] = __builtin_nan("");
      vb.vcbest[b] = -1;
    }
    return;
  }
  if (j * vs.delta >= L) return;
  if (mode == kRedo) {
    if (vb.nbad[iter - 1] == 0 || !vb.redo[(size_t)b * vs.nchunk + j]) return;
  }
  VRegs<AMAX, CAMAX> r;
  vregs_init(r, vs, trans, dur);
  vsweep<NT, AMAX, CAMAX, NGT>(vs, r, vsmem(vs, lds), mode, b, j, L, S, vb);
}

// Serial repair, one workgroup per sequence: chunks still marked after the
// parallel passes are swept in order, each followed by the check of its
// successor, so every chunk ends consistent with its predecessor.  A
// successor that is itself still marked was given a new start by the last
// parallel check but not swept from it, so its end state belongs to an
// older start: it is not checked against its predecessor (a passing check
// would keep that stale end) but takes the predecessor's new end as its
// start and is swept in turn.
template <int NT, int AMAX, int CAMAX, int NGT>
__global__ __launch_bounds__(NT) void k_vrepair(VShape vs, const float *__restrict__ trans,
                                                const float *__restrict__ dur,
                                                const double *__restrict__ S,
                                                const int32_t *__restrict__ lengths, VBufs vb) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int b = blockIdx.x;
  const int L = lengths[b];
  if (L < 1 || L > vs.T || vb.nbad[kVitIters - 1] == 0) return;
  const int nvalid = (L + vs.delta - 1) / vs.delta;
  VRegs<AMAX, CAMAX> r;
  vregs_init(r, vs, trans, dur);
  const VSmem sm = vsmem(vs, lds);
  for (int j = 1; j < nvalid; ++j) {
    __syncthreads();
    if (!vb.redo[(size_t)b * vs.nchunk + j]) continue;
    vsweep<NT, AMAX, CAMAX, NGT>(vs, r, sm, kRedo, b, j, L, S, vb);
    if (j + 1 < nvalid)
      vverify(vs, b, j + 1, vb, sm.flag, -1, vb.redo[(size_t)b * vs.nchunk + j + 1] != 0);
  }
}

__global__ __launch_bounds__(kVHelp) void k_vinit(VShape vs, VBufs vb) {
  const int n = vs.B * vs.nchunk;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    vb.redo[i] = 0;
    vb.corr[i] = 0.0;
  }
  if (blockIdx.x == 0 && threadIdx.x < kVitIters) vb.nbad[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kVHelp) void k_vverify(VShape vs, const int32_t *__restrict__ lengths,
                                                    VBufs vb, int iter) {
  __shared__ int flag[kVHelp / 64];
  const int b = blockIdx.x / vs.nchunk, j = blockIdx.x % vs.nchunk;
  const int L = lengths[b];
  if (L < 1 || L > vs.T || j == 0 || j * vs.delta >= L) return;
  if (iter > 0 && vb.nbad[iter - 1] == 0) return;
  vverify(vs, b, j, vb, flag, iter);
}

// Frame offsets: prefix sums of the recorded constants along each sequence.
__global__ __launch_bounds__(64) void k_vfix(VShape vs, const int32_t *__restrict__ lengths,
                                             VBufs vb) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= vs.B) return;
  const int L = lengths[b];
  if (L < 1 || L > vs.T) return;
  const int nvalid = (L + vs.delta - 1) / vs.delta;
  const size_t base = (size_t)b * vs.nchunk;
  double acc = 0.0;
  vb.delta[base] = 0.0;
  for (int j = 1; j < nvalid; ++j) {
    acc += vb.corr[base + j];
    vb.delta[base + j] = acc;
  }
}

// ------------------------------------------------------------ backtrack

// pred[t, c] = k | (label of the segment before) << 16 for the segment of
// label c ending at t, from the decisions (0xffff: no segment before), for
// t in (wp0, wp1] (its start t - k > wp0 - K lies inside the decisions).
__global__ __launch_bounds__(kVHelp) void k_vpred(VShape vs, const int32_t *__restrict__ lengths,
                                                  VBufs vb) {
  const int C = vs.C, nw = vs.wp1 - vs.wp0;
  const size_t n = (size_t)vs.B * C * nw;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const int t = vs.wp0 + 1 + (int)(i % nw);
    const size_t bc = i / nw;
    const int b = (int)(bc / C);
    const int L = lengths[b];
    if (L < 1 || L > vs.T || t > L) continue;
    const size_t o = bc * vs.bp_stride + (t - vs.bp_t0);
    int k = (int)(vb.bp[o] & 0xffffu);
    if (k < 1 || k > t) k = t;  // only reachable with non-finite scores
    const int s = t - k;
    uint32_t prev = 0xffffu;
    if (s > 0) {
      prev = vb.bp[o - k] >> 16;
      if (prev >= (uint32_t)C) prev = 0;  // only reachable with non-finite scores
    }
    vb.pred[o] = (uint32_t)k | (prev << 16);
  }
}

__device__ __forceinline__ int32_t *sub_of(const VShape &vs, const VBufs &vb, int b, int j) {
  return vb.sub + ((size_t)b * vs.wsub + j) * kVSubFields;
}

// The entry node of the range's last sub-chunk: the path's end (L, best
// final label) when it lies in the range, else the exit of the walk through
// the range after it (low-memory windows).
__device__ __forceinline__ void range_entry(const VShape &vs, const VBufs &vb, int b, int L,
                                            int &t, int &c) {
  if (L <= vs.wp1) {
    t = L;
    c = vb.vcbest[b];
    if (c < 0 || c >= vs.C) c = 0;  // only reachable with non-finite scores
  } else {
    t = vb.node[3 * (size_t)b];
    c = vb.node[3 * (size_t)b + 1];
  }
}

// One thread per (sequence, sub-chunk): walk back from a guessed entry node
// (the true one for the last sub-chunk) while inside (lo, hi], recording
// the nodes and marking them.
__global__ __launch_bounds__(kVHelp) void k_vwalk(VShape vs, const int32_t *__restrict__ lengths,
                                                  VBufs vb) {
  const int id = blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= vs.B * vs.wsub) return;
  const int b = id / vs.wsub, j = id % vs.wsub;
  const int L = lengths[b];
  if (L < 1 || L > vs.T) return;
  const int lo = vs.wp0 + j * vs.dbt, top = min(vs.wp1, L);
  if (lo >= top) return;
  const int hi = min(lo + vs.dbt, top), C = vs.C, T1 = vs.bp_stride, t0 = vs.bp_t0;
  int32_t *mk = vb.mark + (size_t)b * T1;  // position t at mk[t - t0]
  for (int t = lo + 1; t <= hi; ++t) mk[t - t0] = -1;
  int t = hi, c = 0;
  if (hi == top) range_entry(vs, vb, b, L, t, c);
  const uint32_t *pr = vb.pred + (size_t)b * C * T1;
  int32_t *lt = vb.lst_t + (size_t)b * vs.lst_stride + (lo - vs.wp0);
  int32_t *lc = vb.lst_c + (size_t)b * vs.lst_stride + (lo - vs.wp0);
  int n = 0;
  while (t > lo) {
    const uint32_t w = pr[(size_t)c * T1 + (t - t0)];
    lt[n] = t;
    lc[n] = c;
    mk[t - t0] = n * 512 + c;
    ++n;
    t -= (int)(w & 0xffffu);
    c = (int)(w >> 16);
  }
  int32_t *f = sub_of(vs, vb, b, j);
  f[kSubN] = n;
  f[kSubExT] = t;
  f[kSubExC] = c;
}

// From the entry (t, c), follow the predecessors inside (lo, hi] until a
// node of the sub-chunk's guessed walk; record the head length, the merge
// index and the exit of the true path.
__device__ void vmerge_one(const VShape &vs, const VBufs &vb, int b, int j, int t, int c) {
  const int lo = vs.wp0 + j * vs.dbt, C = vs.C, T1 = vs.bp_stride, t0 = vs.bp_t0;
  const int32_t *mk = vb.mark + (size_t)b * T1;
  const uint32_t *pr = vb.pred + (size_t)b * C * T1;
  int32_t *f = sub_of(vs, vb, b, j);
  f[kSubEnT] = t;
  f[kSubEnC] = c;
  int h = 0, mi = -1;
  while (t > lo) {
    const int m = mk[t - t0];
    if (m >= 0 && (m & 511) == c) {
      mi = m >> 9;
      break;
    }
    const uint32_t w = pr[(size_t)c * T1 + (t - t0)];
    ++h;
    t -= (int)(w & 0xffffu);
    c = (int)(w >> 16);
  }
  if (mi >= 0) {
    f[kSubMi] = mi;
    f[kSubTxT] = f[kSubExT];
    f[kSubTxC] = f[kSubExC];
  } else {
    f[kSubMi] = f[kSubN];
    f[kSubTxT] = t;
    f[kSubTxC] = c;
  }
  f[kSubH] = h;
}

__global__ __launch_bounds__(kVHelp) void k_vmerge(VShape vs, const int32_t *__restrict__ lengths,
                                                   VBufs vb) {
  const int id = blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= vs.B * vs.wsub) return;
  const int b = id / vs.wsub, j = id % vs.wsub;
  const int L = lengths[b];
  if (L < 1 || L > vs.T) return;
  const int lo = vs.wp0 + j * vs.dbt, top = min(vs.wp1, L);
  if (lo >= top) return;
  const int hi = min(lo + vs.dbt, top);
  int t, c;
  if (hi == top) {
    range_entry(vs, vb, b, L, t, c);
  } else {
    const int32_t *fn = sub_of(vs, vb, b, j + 1);
    t = fn[kSubExT];
    c = fn[kSubExC];
  }
  vmerge_one(vs, vb, b, j, t, c);
}

// One workgroup per sequence: while some sub-chunk was entered from a node
// other than its successor's true exit, redo the highest such one and walk
// down while the mismatch carries; then count and place the segments.
__global__ __launch_bounds__(kVHelp) void k_vfinish(VShape vs, const int32_t *__restrict__ lengths,
                                                    VBufs vb, float *__restrict__ best_out,
                                                    int32_t *__restrict__ num_segs) {
  __shared__ int red[kVHelp];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = lengths[b];
  const bool win = vs.lm_w > 0;  // one window of a low-memory decode
  if (L < 1 || L > vs.T) {
    if (tid == 0 && !win) {
      num_segs[b] = 0;
      best_out[b] = __builtin_nanf("");
    }
    return;
  }
  if (L <= vs.wp0) return;  // the path ends before this window
  const int nv = (min(vs.wp1, L) - vs.wp0 + vs.dbt - 1) / vs.dbt;
  auto mismatch = [&](int j) {
    const int32_t *f = sub_of(vs, vb, b, j), *fn = sub_of(vs, vb, b, j + 1);
    return f[kSubEnT] != fn[kSubTxT] || f[kSubEnC] != fn[kSubTxC];
  };
  for (;;) {
    int hi = -1;
    for (int j = tid; j + 1 < nv; j += kVHelp)
      if (mismatch(j)) hi = j;
    red[tid] = hi;
    __syncthreads();
    if (tid == 0) {
      int m = -1;
      for (int q = 0; q < kVHelp; ++q) m = max(m, red[q]);
      for (int j = m; j >= 0 && mismatch(j); --j) {
        const int32_t *fn = sub_of(vs, vb, b, j + 1);
        vmerge_one(vs, vb, b, j, fn[kSubTxT], fn[kSubTxC]);
      }
      red[0] = m;
    }
    __syncthreads();
    const int m = red[0];
    __syncthreads();
    if (m < 0) break;
  }
  // counts and their exclusive prefix sums, in order of the sub-chunks
  const int per = (nv + kVHelp - 1) / kVHelp;
  const int j0 = tid * per, j1 = min(j0 + per, nv);
  int own = 0;
  for (int j = j0; j < j1; ++j) {
    const int32_t *f = sub_of(vs, vb, b, j);
    own += f[kSubH] + f[kSubN] - f[kSubMi];
  }
  red[tid] = own;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int q = 0; q < kVHelp; ++q) {
      const int v = red[q];
      red[q] = run;
      run += v;
    }
    if (win) {
      // the window's segments go to row slots [T - after - run, T - after)
      // (after: the segments of the windows behind it); the exit of the
      // first sub-chunk's true path is the next window's entry
      int32_t *nd = vb.node + 3 * (size_t)b;
      const int after = nd[2], base = vs.T - after - run;
      for (int q = 0; q < kVHelp; ++q) red[q] += base;
      const int32_t *f0 = sub_of(vs, vb, b, 0);
      nd[0] = f0[kSubTxT];
      nd[1] = f0[kSubTxC];
      nd[2] = after + run;
    } else {
      num_segs[b] = run;
      best_out[b] = (float)vb.vbest[b];
    }
  }
  __syncthreads();
  int run = red[tid];
  for (int j = j0; j < j1; ++j) {
    int32_t *f = sub_of(vs, vb, b, j);
    f[kSubOff] = run;
    run += f[kSubH] + f[kSubN] - f[kSubMi];
  }
}

// One thread per (sequence, sub-chunk): write its segments of the true
// path (head nodes, then the guessed walk from the merge index) in start order.
__global__ __launch_bounds__(kVHelp) void k_vwrite(VShape vs, const int32_t *__restrict__ lengths,
                                                   VBufs vb, int32_t *__restrict__ seg_start,
                                                   int32_t *__restrict__ seg_len,
                                                   int32_t *__restrict__ seg_label) {
  const int id = blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= vs.B * vs.wsub) return;
  const int b = id / vs.wsub, j = id % vs.wsub;
  const int L = lengths[b];
  if (L < 1 || L > vs.T) return;
  const int lo = vs.wp0 + j * vs.dbt;
  if (lo >= min(vs.wp1, L)) return;
  const int C = vs.C, T1 = vs.bp_stride, t0 = vs.bp_t0;
  const int32_t *f = sub_of(vs, vb, b, j);
  const int h = f[kSubH], n = f[kSubN], mi = f[kSubMi];
  const int cnt = h + n - mi, off = f[kSubOff];
  const uint32_t *pr = vb.pred + (size_t)b * C * T1;
  int32_t *ss = seg_start + (size_t)b * vs.T, *sl = seg_len + (size_t)b * vs.T,
          *sc = seg_label + (size_t)b * vs.T;
  int t = f[kSubEnT], c = f[kSubEnC];
  for (int w = 0; w < h; ++w) {
    const uint32_t p = pr[(size_t)c * T1 + (t - t0)];
    const int k = (int)(p & 0xffffu), o = off + cnt - 1 - w;
    ss[o] = t - k;
    sl[o] = k;
    sc[o] = c;
    t -= k;
    c = (int)(p >> 16);
  }
  const int32_t *lt = vb.lst_t + (size_t)b * vs.lst_stride + (lo - vs.wp0);
  const int32_t *lc = vb.lst_c + (size_t)b * vs.lst_stride + (lo - vs.wp0);
  for (int i = mi; i < n; ++i) {
    const int tt = lt[i], cc = lc[i];
    const int k = (int)(pr[(size_t)cc * T1 + (tt - t0)] & 0xffffu);
    const int o = off + cnt - 1 - (h + i - mi);
    ss[o] = tt - k;
    sl[o] = k;
    sc[o] = cc;
  }
}

__global__ __launch_bounds__(kVHelp) void k_vpad(int B, int T, const int32_t *__restrict__ num_segs,
                                                 int32_t *__restrict__ seg_start,
                                                 int32_t *__restrict__ seg_len,
                                                 int32_t *__restrict__ seg_label) {
  const size_t n = (size_t)B * T;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const int b = (int)(i / T), p = (int)(i % T);
    if (p >= num_segs[b]) {
      seg_start[i] = -1;
      seg_len[i] = -1;
      seg_label[i] = -1;
    }
  }
}

// ------------------------------------------------- low-memory backtrack

// node[b] = {t, c, n}: the entry node of the next window's walk (the
// segment of label c that ends at t; t = -1 before the path's last window)
// and the number of segments found so far.
__global__ __launch_bounds__(64) void k_vlm_init(VShape vs, VBufs vb) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= vs.B) return;
  vb.node[3 * (size_t)b] = -1;
  vb.node[3 * (size_t)b + 1] = 0;
  vb.node[3 * (size_t)b + 2] = 0;
}

// One workgroup per sequence: its n segments sit at row slots [T - n, T) in
// start order; move them to [0, n), blocks in increasing order, each block
// read before any of it is written (a destination block never reaches a
// later block's source: T - n >= 0); then the count and the best score.
__global__ __launch_bounds__(kVHelp) void k_vlm_finish(VShape vs,
                                                       const int32_t *__restrict__ lengths,
                                                       VBufs vb, float *__restrict__ best_out,
                                                       int32_t *seg_start, int32_t *seg_len,
                                                       int32_t *seg_label,
                                                       int32_t *__restrict__ num_segs) {
  const int b = blockIdx.x, T = vs.T;
  const int L = lengths[b];
  const bool ok = L >= 1 && L <= T;
  const int n = ok ? vb.node[3 * (size_t)b + 2] : 0;
  const size_t base = (size_t)b * T;
  for (int i0 = 0; i0 < n; i0 += kVHelp) {
    const int i = i0 + threadIdx.x;
    int32_t st = 0, ln = 0, lb = 0;
    if (i < n) {
      st = seg_start[base + T - n + i];
      ln = seg_len[base + T - n + i];
      lb = seg_label[base + T - n + i];
    }
    __syncthreads();
    if (i < n) {
      seg_start[base + i] = st;
      seg_len[base + i] = ln;
      seg_label[base + i] = lb;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    num_segs[b] = n;
    best_out[b] = ok ? (float)vb.vbest[b] : __builtin_nanf("");
  }
}

int grid_for(size_t n);
hipError_t vit_backtrack(const VShape &vs, const int32_t *lengths, const VBufs &vb,
                         float *best_out, int32_t *seg_start, int32_t *seg_len,
                         int32_t *seg_label, int32_t *num_segs, hipStream_t st, bool pad);

template <int NT, int AMAX, int CAMAX, int NGT>
hipError_t vsweep_abs(const VShape &vs, const float *trans, const float *dur, const double *S,
                      const int32_t *lengths, const VBufs &vb, hipStream_t st) {
  const size_t lds = vit_lds_bytes(vs.C, vs.K, vs.U);
  hipLaunchKernelGGL((k_vsweep<NT, AMAX, CAMAX, NGT>), dim3(vs.B * vs.anj), dim3(NT), lds, st, vs,
                     (int)kAbs, 0, trans, dur, S, lengths, vb);
  return hipGetLastError();
}

// The parallel-in-time passes: relative sweeps, verification, repair and
// frame offsets; then (abs) the absolute sweep of vs.aj0 .. that stores the
// decisions.
template <int NT, int AMAX, int CAMAX, int NGT>
hipError_t vsweeps(const VShape &vs, const float *trans, const float *dur, const double *S,
                   const int32_t *lengths, const VBufs &vb, bool abs, hipStream_t st) {
  const size_t lds = vit_lds_bytes(vs.C, vs.K, vs.U);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void *)k_vsweep<NT, AMAX, CAMAX, NGT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    (void)hipFuncSetAttribute((const void *)k_vrepair<NT, AMAX, CAMAX, NGT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    (void)hipGetLastError();
    attr = true;
  }
  if (!lds_fits((const void *)k_vsweep<NT, AMAX, CAMAX, NGT>, lds) ||
      !lds_fits((const void *)k_vrepair<NT, AMAX, CAMAX, NGT>, lds))
    return hipErrorInvalidConfiguration;
  const int nck = vs.B * vs.nchunk;
  hipLaunchKernelGGL(k_vinit, dim3((nck + kVHelp - 1) / kVHelp), dim3(kVHelp), 0, st, vs, vb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int it = 0; it < kVitIters; ++it) {
    hipLaunchKernelGGL((k_vsweep<NT, AMAX, CAMAX, NGT>), dim3(nck), dim3(NT), lds, st, vs,
                       it == 0 ? (int)kRel : (int)kRedo, it, trans, dur, S, lengths, vb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_vverify, dim3(nck), dim3(kVHelp), 0, st, vs, lengths, vb, it);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_vrepair<NT, AMAX, CAMAX, NGT>), dim3(vs.B), dim3(NT), lds, st, vs, trans, dur,
                     S, lengths, vb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_vfix, dim3((vs.B + 63) / 64), dim3(64), 0, st, vs, lengths, vb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return abs ? vsweep_abs<NT, AMAX, CAMAX, NGT>(vs, trans, dur, S, lengths, vb, st) : hipSuccess;
}

// Low-memory decoding (working memory sublinear in T beyond the cumulative
// scores; the pages' recompute-between-checkpoints, technical summary 2.C,
// in the max semiring): the parallel passes keep only the chunk start
// states; then, window by window from the end of the sequences, the
// absolute sweep recomputes the decisions of the window's chunks -- and of
// the chunk before, whose last K positions hold the previous labels of the
// segments that start in the window -- into buffers of one window, and the
// parallel backtrack (sub-chunk walks, merge, count, write) runs on the
// window, entered where the window after it left the path.  Segments are
// found window by window from the end and written from the end of the
// output rows (k_vfinish places them); k_vlm_finish moves them to the front.
// The decisions are the whole-sequence sweep's (same start states, same
// arithmetic), so the segmentation is the same.
template <int NT, int AMAX, int CAMAX, int NGT>
hipError_t vit_lowmem(const VShape &vs, const float *trans, const float *dur, const double *S,
                      const int32_t *lengths, const VBufs &vb, float *best_out,
                      int32_t *seg_start, int32_t *seg_len, int32_t *seg_label,
                      int32_t *num_segs, hipStream_t st) {
  hipError_t e = vsweeps<NT, AMAX, CAMAX, NGT>(vs, trans, dur, S, lengths, vb, false, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_vlm_init, dim3((vs.B + 63) / 64), dim3(64), 0, st, vs, vb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int W = vs.lm_w, nwin = (vs.nchunk + W - 1) / W;
  for (int w = nwin - 1; w >= 0; --w) {
    const int j0 = w * W, j1 = min(j0 + W, vs.nchunk);
    VShape ws = vs;
    ws.aj0 = j0 > 0 ? j0 - 1 : 0;
    ws.anj = j1 - ws.aj0;
    ws.bp_t0 = ws.aj0 * vs.delta;
    ws.wp0 = j0 * vs.delta;
    ws.wp1 = min(j1 * vs.delta, vs.T);
    ws.bp_stride = ws.wp1 - ws.bp_t0 + 1;
    ws.wsub = (ws.wp1 - ws.wp0 + vs.dbt - 1) / vs.dbt;
    ws.lst_stride = W * vs.delta;
    e = vsweep_abs<NT, AMAX, CAMAX, NGT>(ws, trans, dur, S, lengths, vb, st);
    if (e != hipSuccess) return e;
    e = vit_backtrack(ws, lengths, vb, best_out, seg_start, seg_len, seg_label, num_segs, st,
                      false);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_vlm_finish, dim3(vs.B), dim3(kVHelp), 0, st, vs, lengths, vb, best_out,
                     seg_start, seg_len, seg_label, num_segs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_vpad, dim3(grid_for((size_t)vs.B * vs.T)), dim3(kVHelp), 0, st, vs.B,
                     vs.T, num_segs, seg_start, seg_len, seg_label);
  return hipGetLastError();
}

// The whole decoder for one kernel instance.
template <int NT, int AMAX, int CAMAX, int NGT>
hipError_t vit_run(const VShape &vs, const float *trans, const float *dur, const double *S,
                   const int32_t *lengths, const VBufs &vb, float *best_out, int32_t *seg_start,
                   int32_t *seg_len, int32_t *seg_label, int32_t *num_segs, hipStream_t st) {
  if (vs.lm_w > 0)
    return vit_lowmem<NT, AMAX, CAMAX, NGT>(vs, trans, dur, S, lengths, vb, best_out, seg_start,
                                            seg_len, seg_label, num_segs, st);
  hipError_t e = vsweeps<NT, AMAX, CAMAX, NGT>(vs, trans, dur, S, lengths, vb, true, st);
  if (e != hipSuccess) return e;
  return vit_backtrack(vs, lengths, vb, best_out, seg_start, seg_len, seg_label, num_segs, st,
                       true);
}

int grid_for(size_t n) {
  size_t g = (n + kVHelp - 1) / kVHelp;
  return (int)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

}  // namespace

// Shape of the parallel-in-time decoder, false if it does not apply (the
// serial decoder of viterbi.hip takes those shapes).
bool vit_config(int B, int T, int C, int K, VShape &vs) {
  if (B < 1 || T < 1 || C < 1 || C > kMaxC || K < 1 || K > 65535) return false;
  vs = VShape{};
  vs.B = B;
  vs.T = T;
  vs.C = C;
  vs.K = K;
  int ng = 64;
  while (ng > 4 && ng * C > 1024) ng >>= 1;
  if (ng * C > 1024) return false;
  // narrower groups (fewer threads, fewer waves at every barrier) while a
  // lane then still holds at most 16 durations and 4 previous labels
  while (ng * C > 256 && ng > 4 && (K + ng / 2 - 1) / (ng / 2) <= 16 && C <= 4 * (ng / 2)) ng >>= 1;
  vs.NG = ng;
  vs.NT = ng * C <= 256 ? 256 : (ng * C <= 512 && C <= 4 * ng ? 512 : 1024);
  vs.A = (K + ng - 1) / ng;
  vs.CA = (C + ng - 1) / ng;
  if (vs.A > 16 || vs.CA > 64) return false;
  int u = ng < 16 ? ng : 16;
  while (u > 2 && vit_lds_bytes(C, K, u) > kMaxDynLds) u >>= 1;
  if (vit_lds_bytes(C, K, u) > kMaxDynLds) return false;
  vs.U = u;  // u <= ng and ng * C <= NT: one staged score per thread and block
  // enough chunks for about one workgroup per compute unit, each at least 2K
  // positions (and 64) long; burn-in max(2K, chunk / 4)
  const int want = (256 + B - 1) / B;
  long long d = ((long long)T + want - 1) / want;
  const long long lo = 2LL * K > 64 ? 2LL * K : 64;
  if (d < lo) d = lo;
  if (d > T) d = T;
  vs.delta = (int)d;
  vs.nchunk = (T + vs.delta - 1) / vs.delta;
  vs.burn = 2 * K > vs.delta / 4 ? 2 * K : vs.delta / 4;
  vs.dbt = K > 128 ? K : 128;
  vs.nsub = (T + vs.dbt - 1) / vs.dbt;
  vs.aj0 = 0;
  vs.anj = vs.nchunk;
  vs.bp_t0 = 0;
  vs.bp_stride = T + 1;
  vs.lm_w = 0;
  vs.wp0 = 0;
  vs.wp1 = T;
  vs.wsub = vs.nsub;
  vs.lst_stride = T;
  return true;
}

hipError_t launch_vit_pit(const VShape &vs, const float *trans, const float *dur,
                          const double *S, const int32_t *lengths, const VBufs &vb,
                          float *best_out, int32_t *seg_start, int32_t *seg_len,
                          int32_t *seg_label, int32_t *num_segs, hipStream_t st) {
  // instances: durations per lane (<= 4, <= 16) x previous labels per lane
  // (<= 4 at any group width; <= 16 at width 8, C <= 128; <= 64 at width 4)
  const bool a4 = vs.A <= 4;
#define SEMICRF_VIT_RUN(...) \
  vit_run<__VA_ARGS__>(vs, trans, dur, S, lengths, vb, best_out, seg_start, seg_len, seg_label, \
                       num_segs, st)
  if (vs.NT == 256)  // C <= 4: one previous label per lane
    return a4 ? SEMICRF_VIT_RUN(256, 4, 4, 0) : SEMICRF_VIT_RUN(256, 16, 4, 0);
  if (vs.NT == 512)  // at most 4 previous labels per lane
    return a4 ? SEMICRF_VIT_RUN(512, 4, 4, 0) : SEMICRF_VIT_RUN(512, 16, 4, 0);
  if (vs.CA <= 4) return a4 ? SEMICRF_VIT_RUN(1024, 4, 4, 0) : SEMICRF_VIT_RUN(1024, 16, 4, 0);
  if (vs.NG == 8) return a4 ? SEMICRF_VIT_RUN(1024, 4, 16, 8) : SEMICRF_VIT_RUN(1024, 16, 16, 8);
  return a4 ? SEMICRF_VIT_RUN(1024, 4, 64, 4) : SEMICRF_VIT_RUN(1024, 16, 64, 4);
#undef SEMICRF_VIT_RUN
}

namespace {

// The parallel backtrack over the decisions of positions (wp0, wp1]: the
// whole sequence, or one low-memory window (then no padding: the segments
// are moved into place at the end).
hipError_t vit_backtrack(const VShape &vs, const int32_t *lengths, const VBufs &vb,
                         float *best_out, int32_t *seg_start, int32_t *seg_len,
                         int32_t *seg_label, int32_t *num_segs, hipStream_t st, bool pad) {
  hipError_t e;
  const size_t npred = (size_t)vs.B * vs.C * (vs.wp1 - vs.wp0);
  hipLaunchKernelGGL(k_vpred, dim3(grid_for(npred)), dim3(kVHelp), 0, st, vs, lengths, vb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nsub = vs.B * vs.wsub;
  const int gs = (nsub + kVHelp - 1) / kVHelp;
  hipLaunchKernelGGL(k_vwalk, dim3(gs), dim3(kVHelp), 0, st, vs, lengths, vb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_vmerge, dim3(gs), dim3(kVHelp), 0, st, vs, lengths, vb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_vfinish, dim3(vs.B), dim3(kVHelp), 0, st, vs, lengths, vb, best_out,
                     num_segs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_vwrite, dim3(gs), dim3(kVHelp), 0, st, vs, lengths, vb, seg_start,
                     seg_len, seg_label);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!pad) return hipSuccess;
  hipLaunchKernelGGL(k_vpad, dim3(grid_for((size_t)vs.B * vs.T)), dim3(kVHelp), 0, st, vs.B,
                     vs.T, num_segs, seg_start, seg_len, seg_label);
  return hipGetLastError();
}

}  // namespace

}  // namespace semicrf
