// pitcheck.h -- the chunk-boundary check of the parallel-in-time sweeps as a
// block-wide device function: k_pit_verify (pit.hip) runs it for one chunk
// per workgroup after a parallel iteration; the sweep engines' in-order
// repair runs it chunk after chunk within one workgroup.
//
// The recursion is linear in the exp-space ring and forgets where it
// started, so a chunk swept from a guessed start reaches the true state up
// to one scalar once its start agrees in direction with its predecessor's
// end ("Streaming Structured Inference with Flash-SemiCRF", technical
// summary 2.C: the state at every checkpoint; pit.hip's header has the
// whole scheme).
#pragma once

#include "internal.h"

namespace semicrf {

constexpr double kPitTol = 1e-12;  // direction mismatch accepted, relative to the largest entry
// The same for the engine whose ring and sums are float32 (chain256.hip): two
// chains that reach one state along different paths agree to float32
// rounding there, so a float64-level bar would reject every converged chunk.
constexpr double kPitTolF32 = 1e-5;
constexpr int kPitBatch = 8;  // record entries per thread and batch of loads

struct PitMaxArg {
  double v;
  int i;
};

__device__ __forceinline__ PitMaxArg pit_max_arg(PitMaxArg a, PitMaxArg b) {
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

// Chunk j of direction `fwd` of sequence b (not the chain's exact chunk):
// compare its start record A with the end record E of the chunk before it
// in the chain (forward j - 1, backward j + 1), entry by entry relative to
// (about) E's largest entry.  Consistent -- the two agree in direction
// within the tolerance, A ~ 2^(di + df) E -- and not `force`d:
// records the scalar and clears the chunk's redo flag.  Otherwise E becomes
// the start exactly (scalar 0), redo is set and, for iter >= 0, counted in
// nbad[iter].  Returns whether it was consistent.  All NT threads of the
// block call it (the result is uniform); red and redd are LDS scratch of
// NT / 64 entries each.  Global writes of the block before the call must be
// visible to it (a fence and a barrier); its own writes are followed by a
// fence and a barrier.
template <int NT>
__device__ bool pit_check(const ChainShape &sh, const PitBufs &pb, bool fwd, int b, int j,
                          int iter, bool force, PitMaxArg *red, double *redd) {
  const int nck = sh.B * sh.nchunk;
  const int jp = fwd ? j - 1 : j + 1;  // chunk whose end must equal this chunk's start
  const int C = sh.C, K = sh.K;
  const size_t cks = ck_stride(C, K);
  double *A = (fwd ? pb.ck_fwd : pb.ck_bwd) + ((size_t)b * sh.nchunk + j) * cks;
  const double *E = (fwd ? pb.end_fwd : pb.end_bwd) + ((size_t)b * sh.nchunk + jp) * cks;
  const double *RA = A + (size_t)K * C, *RE = E + (size_t)K * C;
  const int n = K * C;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const long long re0 = (long long)RE[0];
  const int cstep = NT % C;  // label of entry i + NT from that of entry i

  // an entry of E within a factor 2^0.09 of its largest, in log2 relative to
  // E's label-0 reference (exponent plus the mantissa's chord: log2 of
  // 2m in [1, 2) taken as 2m - 1)
  // (entries in batches of kPitBatch per thread, every load of a batch
  // issued before the first use; the maximum does not depend on the order)
  PitMaxArg best = {-__builtin_huge_val(), 0x7fffffff};
  for (int i0 = tid, c = tid % C; i0 < n; i0 += kPitBatch * NT) {
    double ev[kPitBatch], rv[kPitBatch];
#pragma unroll
    for (int u = 0; u < kPitBatch; ++u) {
      const int i = i0 + u * NT;
      ev[u] = i < n ? E[i] : 0.0;
      rv[u] = RE[c];
      c += cstep;
      c -= c >= C ? C : 0;
    }
#pragma unroll
    for (int u = 0; u < kPitBatch; ++u) {
      if (ev[u] > 0.0) {
        int ex;
        const double m = frexp(ev[u], &ex);
        const double le = (double)((long long)rv[u] - re0 + ex) + (2.0 * m - 2.0);
        best = pit_max_arg(best, PitMaxArg{le, i0 + u * NT});
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    PitMaxArg o;
    o.v = __shfl_xor(best.v, off);
    o.i = __shfl_xor(best.i, off);
    best = pit_max_arg(best, o);
  }
  if (lane == 0) red[w] = best;
  __syncthreads();
  best = red[0];
  for (int q = 1; q < NT / 64; ++q) best = pit_max_arg(best, red[q]);
  const bool neutral = A[(size_t)K * C + C] != A[(size_t)K * C + C];  // o is NaN on a neutral start
  bool ok = !force && best.i != 0x7fffffff && !neutral && A[best.i] > 0.0;
  long long di = 0;
  double df = 0.0;
  double mism = 0.0;
  if (ok) {
    // scalar between the states: A ~ 2^delta E, delta = di + df
    const int cs = best.i % C;
    const double l = log2(A[best.i]) - log2(E[best.i]);
    const double fl = floor(l);
    di = (long long)RA[cs] - (long long)RE[cs] + (long long)fl;
    df = l - fl;
    // entries relative to 2^best.v: E as e 2^(RE - re0 - bv), A as
    // a 2^(RA - re0 - di - df - bv); integer parts by ldexp (exact),
    // fractional parts by two factors formed once
    const double bi = floor(best.v);
    const long long bvi = (long long)bi;
    const double fe = exp2(bi - best.v), fa = exp2(bi - best.v - df);
    auto pow2 = [](double x, long long k) {
      return ldexp(x, (int)(k < -4000 ? -4000 : (k > 4000 ? 4000 : k)));
    };
    for (int i0 = tid, c = tid % C; i0 < n; i0 += kPitBatch * NT) {
      double av[kPitBatch], ev[kPitBatch], ra[kPitBatch], re[kPitBatch];
#pragma unroll
      for (int u = 0; u < kPitBatch; ++u) {
        const int i = i0 + u * NT;
        av[u] = i < n ? A[i] : 0.0;
        ev[u] = i < n ? E[i] : 0.0;
        ra[u] = RA[c];
        re[u] = RE[c];
        c += cstep;
        c -= c >= C ? C : 0;
      }
#pragma unroll
      for (int u = 0; u < kPitBatch; ++u) {
        const double a = av[u], e = ev[u];
        if (a != 0.0 || e != 0.0) {
          const double we = e > 0.0 ? pow2(e * fe, (long long)re[u] - re0 - bvi) : 0.0;
          const double wa = a > 0.0 ? pow2(a * fa, (long long)ra[u] - re0 - di - bvi) : 0.0;
          mism = fmax(mism, fabs(wa - we));
        }
      }
    }
    for (int off = 32; off > 0; off >>= 1) mism = fmax(mism, __shfl_xor(mism, off));
    __syncthreads();
    if (lane == 0) redd[w] = mism;
    __syncthreads();
    mism = redd[0];
    for (int q = 1; q < NT / 64; ++q) mism = fmax(mism, redd[q]);
    ok = mism <= (sh.e256 ? kPitTolF32 : kPitTol);
  }
  const size_t idx = (fwd ? 0 : (size_t)nck) + (size_t)b * sh.nchunk + j;
  __syncthreads();  // every read of A above precedes the copy below
  if (ok) {
    if (tid == 0) {
      pb.corr_i[idx] = di;
      pb.corr_f[idx] = df;
      pb.redo[idx] = 0;
    }
  } else {
    // the start becomes the predecessor's end exactly: scalar 0 between them
    for (size_t i = tid; i < cks; i += NT) A[i] = E[i];
    if (tid == 0) {
      pb.corr_i[idx] = 0;
      pb.corr_f[idx] = 0.0;
      pb.redo[idx] = 1;
      if (iter >= 0) atomicAdd(&pb.nbad[iter], 1);
    }
  }
  __threadfence_block();
  __syncthreads();
  return ok;
}

// Whether v holds on any thread of the block (all NT threads call it);
// red is the same LDS scratch as pit_check's.
template <int NT>
__device__ bool pit_any(bool v, PitMaxArg *red) {
  const bool w = __any(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6].i = w ? 1 : 0;
  __syncthreads();
  int r = 0;
  for (int q = 0; q < NT / 64; ++q) r |= red[q].i;
  __syncthreads();
  return r != 0;
}

// Iterations of the parallel sweeps before an engine's in-order repair
// takes over (a chunk is consistent after the first of them unless its
// start has not been forgotten within its burn-in).
constexpr int kPitParallelIters = 2;
// The `iter` argument of a sweep launch in repair mode: one workgroup per
// (direction, sequence) walks the chunks in the chain's order, sweeping each
// chunk still marked from its (replaced) start and checking its successor
// against the new end -- so every chunk ends consistent whatever the
// parallel passes left, with one launch instead of one per iteration.
constexpr int kPitRepair = -2;

}  // namespace semicrf
