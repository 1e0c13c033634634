// viterbi.hip -- max-semiring semi-CRF decoding on gfx950.
//
// The pages give no decoder.  This is the (max,+) version of the forward
// recurrence of chain.hip over the same segment scores (read on the fly from
// the cumulative scores S, "Streaming Structured Inference with
// Flash-SemiCRF", abstract; technical summary 2.A):
//   ahat[t,c] = S[t,c] + max_{k<=min(K,t)} (dur[k-1,c] + ghat[t-k,c])   argmax k
//   uhat[t,c] = max_{c'} (ahat[t,c'] + trans[c',c]),  uhat[0,.] = 0    argmax c'
//   ghat[t,c] = uhat[t,c] - S[t,c]
//   best      = max_c ahat[L,c]
// Ties are structural: segmentations that differ only in the order of the
// segment lengths inside a run of one label score exactly the same, and
// floating point sees them as equal only up to rounding.  A candidate ties
// with the maximum when it lies within eps = 1e-11 (|max| + 1) of it; among
// tied candidates the smallest k wins, then the smallest c', and at the end
// the smallest final label c.  The stored value is the maximum itself.
// Log-space float64 throughout (max-plus needs no exponentials); the ring of
// the K most recent ghat rows lives in LDS, backpointers (k, c') are packed
// as two 16-bit fields per (t, c) in the workspace, and a second kernel
// walks them back (O(number of segments)).
#include "device_math.h"
#include "internal.h"

namespace semicrf {

__device__ __forceinline__ double tie_eps(double best) { return viterbi_tie_eps(best); }

template <int NT, int AMAX, int TRMAX>
__global__ __launch_bounds__(NT) void k_viterbi(ChainShape sh, const float *__restrict__ trans,
                                                const float *__restrict__ dur,
                                                const double *__restrict__ S,
                                                const int32_t *__restrict__ lengths,
                                                uint32_t *__restrict__ bp,
                                                double *__restrict__ vbest,
                                                int32_t *__restrict__ vcbest) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, C = sh.C, K = sh.K;
  const int L = lengths[b];
  if (L < 1 || L > sh.T) {
    if (tid == 0) {
      vbest[b] = __builtin_nan("");
      vcbest[b] = -1;
    }
    return;
  }
  size_t off = 0;
  double *ring = reinterpret_cast<double *>(lds + off); off += (size_t)K * C * 8;
  double *pmax = reinterpret_cast<double *>(lds + off); off += (size_t)sh.P * C * 8;
  int *parg = reinterpret_cast<int *>(lds + off); off += (size_t)sh.P * C * 4;
  double *arow = reinterpret_cast<double *>(lds + off); off += (size_t)C * 8;
  double *qmax = reinterpret_cast<double *>(lds + off); off += (size_t)sh.Q * C * 8;
  int *qarg = reinterpret_cast<int *>(lds + off); off += (size_t)sh.Q * C * 4;

  // duration role
  const int kc = tid % C, kp = tid / C;
  const int age0 = kp * sh.A + 1;
  int nage = (kp < sh.P) ? K - age0 + 1 : 0;
  nage = nage < 0 ? 0 : (nage > sh.A ? sh.A : nage);
  double dv[AMAX];
#pragma unroll
  for (int j = 0; j < AMAX; ++j) dv[j] = (j < nage) ? (double)dur[(size_t)(age0 + j - 1) * C + kc] : 0.0;
  // contraction role: trans[c'][cc] for c' in [64 cq, 64 cq + 64)
  const int cc = tid % C, cq = tid / C;
  const int cp0 = cq * 64;
  int ncp = (cq < sh.Q) ? C - cp0 : 0;
  ncp = ncp < 0 ? 0 : (ncp > 64 ? 64 : ncp);
  float tw[TRMAX];
#pragma unroll
  for (int j = 0; j < TRMAX; ++j) tw[j] = (j < ncp) ? trans[(size_t)(cp0 + j) * C + cc] : 0.f;

  const double *Sb = S + (size_t)b * (sh.T + 1) * C;
  uint32_t *bpb = bp + (size_t)b * (sh.T + 1) * C;
  const double ninf = -__builtin_huge_val();
  for (int i = tid; i < K * C; i += NT) ring[i] = ninf;
  __syncthreads();
  if (tid < C) ring[tid] = 0.0;  // position 0: uhat = 0, S = 0
  __syncthreads();

  for (int t = 1; t <= L; ++t) {
    const int tm = t % K;
    // duration decision, pass 1: maximum of dur[k-1,c] + ghat[t-k,c]
    if (kp < sh.P) {
      double best = ninf;
#pragma unroll
      for (int j = 0; j < AMAX; ++j) {
        if (j < nage) {
          int sl = tm - (age0 + j);
          sl += (sl < 0) ? K : 0;
          best = fmax(best, dv[j] + ring[sl * C + kc]);
        }
      }
      pmax[kp * C + kc] = best;
    }
    __syncthreads();
    if (tid < C) {
      double best = ninf;
      for (int p = 0; p < sh.P; ++p) best = fmax(best, pmax[p * C + tid]);
      qmax[tid] = best;  // broadcast slot (Q*C >= C)
    }
    __syncthreads();
    // pass 2: smallest k inside the tie set of the maximum
    if (kp < sh.P) {
      const double best = qmax[kc];
      const double eps = tie_eps(best + Sb[(size_t)t * C + kc]);
      int arg = 0;
#pragma unroll
      for (int j = 0; j < AMAX; ++j) {
        if (j < nage && arg == 0) {
          int sl = tm - (age0 + j);
          sl += (sl < 0) ? K : 0;
          if (dv[j] + ring[sl * C + kc] >= best - eps) arg = age0 + j;
        }
      }
      parg[kp * C + kc] = arg;
    }
    __syncthreads();
    if (tid < C) {
      int arg = 0;
      for (int p = 0; p < sh.P && arg == 0; ++p) arg = parg[p * C + tid];
      arow[tid] = qmax[tid] + Sb[(size_t)t * C + tid];
      bpb[(size_t)t * C + tid] = (uint32_t)arg;
    }
    __syncthreads();
    if (t == L) break;
    // label decision: uhat[t,c] = max_{c'} (ahat[t,c'] + trans[c',c])
    double best = ninf;
    if (cq < sh.Q) {
#pragma unroll
      for (int j = 0; j < TRMAX; ++j)
        if (j < ncp) best = fmax(best, arow[cp0 + j] + (double)tw[j]);
    }
    if (sh.Q > 1) {
      if (cq < sh.Q) qmax[cq * C + cc] = best;
      __syncthreads();
      best = ninf;
      if (cq < sh.Q)
        for (int q = 0; q < sh.Q; ++q) best = fmax(best, qmax[q * C + cc]);
    }
    int arg = -1;
    if (cq < sh.Q) {
      const double eps = tie_eps(best);
#pragma unroll
      for (int j = 0; j < TRMAX; ++j)
        if (j < ncp && arg < 0 && arow[cp0 + j] + (double)tw[j] >= best - eps) arg = cp0 + j;
    }
    if (sh.Q > 1) {
      if (cq < sh.Q) qarg[cq * C + cc] = arg;
      __syncthreads();
      if (tid < C) {
        arg = -1;
        for (int q = 0; q < sh.Q && arg < 0; ++q) arg = qarg[q * C + tid];
      }
    }
    if (tid < C) {
      bpb[(size_t)t * C + tid] |= ((uint32_t)arg) << 16;
      ring[tm * C + tid] = best - Sb[(size_t)t * C + tid];
    }
    __syncthreads();
  }
  if (tid == 0) {
    double best = ninf;
    for (int c = 0; c < C; ++c) best = fmax(best, arow[c]);
    int cb = 0;
    const double eps = tie_eps(best);
    for (int c = C - 1; c >= 0; --c)
      if (arow[c] >= best - eps) cb = c;
    vbest[b] = best;
    vcbest[b] = cb;
  }
}

// One workgroup per sequence: thread 0 walks the backpointers twice (count,
// then write in start order); all threads pad the remaining slots with -1.
__global__ __launch_bounds__(256) void k_backtrack(ChainShape sh,
                                                   const int32_t *__restrict__ lengths,
                                                   const uint32_t *__restrict__ bp,
                                                   const double *__restrict__ vbest,
                                                   const int32_t *__restrict__ vcbest,
                                                   float *__restrict__ best_out,
                                                   int32_t *__restrict__ seg_start,
                                                   int32_t *__restrict__ seg_len,
                                                   int32_t *__restrict__ seg_label,
                                                   int32_t *__restrict__ num_segs) {
  __shared__ int nseg_sh;
  const int b = blockIdx.x, C = sh.C, T = sh.T;
  const int L = lengths[b];
  const bool ok = L >= 1 && L <= T;
  const uint32_t *bpb = bp + (size_t)b * (T + 1) * C;
  int32_t *ss = seg_start + (size_t)b * T;
  int32_t *sl = seg_len + (size_t)b * T;
  int32_t *sc = seg_label + (size_t)b * T;
  if (threadIdx.x == 0) {
    int n = 0;
    if (ok) {
      int t = L, c = vcbest[b];
      while (t > 0) {
        int k = (int)(bpb[(size_t)t * C + c] & 0xffffu);
        if (k < 1 || k > t) k = t;  // only reachable with non-finite scores
        const int s = t - k;
        if (s > 0) c = (int)(bpb[(size_t)s * C + c] >> 16);
        if (c >= C) c = 0;  // only reachable with non-finite scores
        t = s;
        ++n;
      }
      t = L;
      c = vcbest[b];
      int i = n;
      while (t > 0) {
        int k = (int)(bpb[(size_t)t * C + c] & 0xffffu);
        if (k < 1 || k > t) k = t;
        const int s = t - k;
        --i;
        ss[i] = s;
        sl[i] = k;
        sc[i] = c;
        if (s > 0) c = (int)(bpb[(size_t)s * C + c] >> 16);
        if (c >= C) c = 0;  // only reachable with non-finite scores
        t = s;
      }
    }
    nseg_sh = n;
    num_segs[b] = n;
    best_out[b] = ok ? (float)vbest[b] : __builtin_nanf("");
  }
  __syncthreads();
  for (int i = nseg_sh + (int)threadIdx.x; i < T; i += blockDim.x) {
    ss[i] = -1;
    sl[i] = -1;
    sc[i] = -1;
  }
}

template <int NT, int AMAX, int TRMAX>
static hipError_t viterbi_impl(const ChainShape &sh, const float *trans, const float *dur,
                               const double *S, const int32_t *lengths, uint32_t *bp,
                               double *vbest, int32_t *vcbest, hipStream_t st) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void *)k_viterbi<NT, AMAX, TRMAX>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    (void)hipGetLastError();
    attr = true;
  }
  const size_t lds = viterbi_lds_bytes(sh.C, sh.K, sh.P, sh.Q);
  if (!lds_fits((const void *)k_viterbi<NT, AMAX, TRMAX>, lds)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_viterbi<NT, AMAX, TRMAX>), dim3(sh.B), dim3(NT), lds, st, sh, trans,
                     dur, S, lengths, bp, vbest, vcbest);
  return hipGetLastError();
}

hipError_t launch_viterbi(const ChainShape &sh, const float *trans, const float *dur,
                          const double *S, const int32_t *lengths, uint32_t *bp, double *vbest,
                          int32_t *vcbest, float *best_out, int32_t *seg_start,
                          int32_t *seg_len, int32_t *seg_label, int32_t *num_segs,
                          hipStream_t st) {
  const int trmax = sh.C <= 8 ? 8 : (sh.C <= 32 ? 32 : 64);
  hipError_t e;
  if (sh.NT == 256)
    e = trmax == 8 ? viterbi_impl<256, 32, 8>(sh, trans, dur, S, lengths, bp, vbest, vcbest, st)
        : trmax == 32 ? viterbi_impl<256, 32, 32>(sh, trans, dur, S, lengths, bp, vbest, vcbest, st)
                      : viterbi_impl<256, 32, 64>(sh, trans, dur, S, lengths, bp, vbest, vcbest, st);
  else if (sh.NT == 512)
    e = trmax == 8 ? viterbi_impl<512, 32, 8>(sh, trans, dur, S, lengths, bp, vbest, vcbest, st)
        : trmax == 32 ? viterbi_impl<512, 32, 32>(sh, trans, dur, S, lengths, bp, vbest, vcbest, st)
                      : viterbi_impl<512, 32, 64>(sh, trans, dur, S, lengths, bp, vbest, vcbest, st);
  else
    e = trmax == 8 ? viterbi_impl<1024, 16, 8>(sh, trans, dur, S, lengths, bp, vbest, vcbest, st)
        : trmax == 32 ? viterbi_impl<1024, 16, 32>(sh, trans, dur, S, lengths, bp, vbest, vcbest, st)
                      : viterbi_impl<1024, 16, 64>(sh, trans, dur, S, lengths, bp, vbest, vcbest, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_backtrack, dim3(sh.B), dim3(256), 0, st, sh, lengths, bp, vbest, vcbest,
                     best_out, seg_start, seg_len, seg_label, num_segs);
  return hipGetLastError();
}

}  // namespace semicrf
