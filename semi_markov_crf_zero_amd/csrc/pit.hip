// pit.hip -- parallel-in-time sweeps: verification and normaliser fix-up.
//
// The streamed forward (and backward) state at a checkpoint boundary is the
// ring of the K newest entries of every label, in exp space relative to an
// integer log reference per label (the record layout of chain.hip /
// chain_win.hip: [K*C ring][C refs][C o][C m], float64).  The recursion is
// linear in that state, and it forgets where it started: run from two start
// states that differ, the states it reaches agree in direction (up to one
// scalar) after enough positions.  So every checkpoint interval ("chunk") is
// swept concurrently:
//   iteration 0: the chunk at the sequence end a direction starts from (the
//     first chunk forward, the last backward) starts from its exact state,
//     every other chunk from a neutral state;
//   after each iteration, k_pit_verify compares each chunk's start with the
//     end state its predecessor produced.  Equal in direction: the chunk is
//     consistent, and the scalar between the two (log2 units, kept as an
//     exact integer plus a fraction) is recorded.  Different: the
//     predecessor's end becomes the chunk's new start and the chunk is swept
//     again in the next iteration;
//   the iterations stop once one verification finds no difference.  After
//     n iterations the first n chunks have exact starts, so nchunk
//     iterations always suffice, and the last one (which can only sweep the
//     chain's last chunk) needs no verification; every kernel of an
//     iteration after convergence returns at once;
//   the register-ring engines (chain64.hip, chain256.hip, chain_win.hip) stop
//     after kPitParallelIters parallel iterations: one more launch of the
//     engine, one workgroup per (direction, sequence), walks the chain in
//     order, sweeping each chunk still marked and checking its successor
//     against the new end (pitcheck.h).  Nothing is marked after a
//     converged check, so that launch returns at once in the usual case and
//     the loop above costs two iterations instead of nchunk;
//   k_pit_fixup adds the prefix sums of the recorded scalars to the
//     checkpoint records and to log Z, which makes every record the exact
//     state with its exact log normaliser -- the checkpoint-boundary
//     normalisation of "Streaming Structured Inference with Flash-SemiCRF"
//     (abstract; technical summary, section 2.C) computed chunk-parallel.
#include "device_math.h"
#include "internal.h"
#include "pitcheck.h"

namespace semicrf {

namespace {

constexpr int kPitThreads = 256;

}  // namespace

// One workgroup per (direction, sequence, chunk).  Forward chunk j >= 1
// compares its start (state at p0_j) with the end of forward chunk j-1;
// backward chunk j compares its start (state at p1_j) with the end of
// backward chunk j+1.
__global__ __launch_bounds__(kPitThreads) void k_pit_verify(ChainShape sh,
                                                            const int32_t *__restrict__ lengths,
                                                            PitBufs pb, int iter) {
  if (iter > 0 && pb.nbad[iter - 1] == 0) return;
  __shared__ PitMaxArg red[kPitThreads / 64];
  __shared__ double redd[kPitThreads / 64];
  const int nck = sh.B * sh.nchunk;
  const bool fwd = (int)blockIdx.x < nck;
  const int rem = fwd ? blockIdx.x : blockIdx.x - nck;
  const int b = rem / sh.nchunk, j = rem % sh.nchunk;
  const int L = lengths[b];
  if (L < 1 || L > sh.T) return;
  const int nvalid = (L + sh.delta - 1) / sh.delta;
  if (j >= nvalid) return;  // past the sequence: never swept
  if (fwd ? j == 0 : j + 1 == nvalid) {
    // the chain's exact chunk: its start is exact from iteration 0, so it is
    // never swept again
    if (threadIdx.x == 0) pb.redo[(fwd ? 0 : (size_t)nck) + (size_t)b * sh.nchunk + j] = 0;
    return;
  }
  pit_check<kPitThreads>(sh, pb, fwd, b, j, iter, false, red, redd);
}

// One workgroup per (direction, sequence): prefix sums of the recorded
// scalars along the direction of the chain, giving each chunk's exact log
// correction (shift, for the rows; its integer and fractional log2 parts
// replace the chunk's scalar, for k_pit_records) and the chain's log Z.
__global__ __launch_bounds__(kPitThreads) void k_pit_fixup(ChainShape sh,
                                                           const int32_t *__restrict__ lengths,
                                                           PitBufs pb, double *logz_ws,
                                                           double *logz_bwd_ws, float *logz_out,
                                                           int with_bwd) {
  const bool fwd = (int)blockIdx.x < sh.B;
  const int b = fwd ? blockIdx.x : blockIdx.x - sh.B;
  if (!fwd && !with_bwd) return;
  const int L = lengths[b];
  const int tid = threadIdx.x;
  if (L < 1 || L > sh.T) {
    if (tid == 0) {
      if (fwd) {
        logz_ws[b] = __builtin_nan("");
        logz_out[b] = __builtin_nanf("");
      } else if (logz_bwd_ws) {
        logz_bwd_ws[b] = __builtin_nan("");
      }
    }
    return;
  }
  const int nvalid = (L + sh.delta - 1) / sh.delta;
  const size_t base = (fwd ? 0 : (size_t)sh.B * sh.nchunk) + (size_t)b * sh.nchunk;
  __shared__ long long si[kPitThreads];
  __shared__ double sf[kPitThreads];
  long long oi = 0;  // accumulated offset of the current chunk, log2 units (thread 0)
  double of = 0.0;
  if (tid == 0) pb.shift[base + (fwd ? 0 : nvalid - 1)] = 0.0;  // the chain's exact chunk
  // chunks in the chain's order, kPitThreads at a time: the scalars are read
  // in parallel, summed in order by one thread, the corrections written back
  for (int s1 = 1; s1 < nvalid; s1 += kPitThreads) {
    const int n = min(kPitThreads, nvalid - s1);
    const int j = fwd ? s1 + tid : nvalid - 1 - (s1 + tid);
    if (tid < n) {
      si[tid] = pb.corr_i[base + j];
      sf[tid] = pb.corr_f[base + j];
    }
    __syncthreads();
    if (tid == 0) {
      for (int q = 0; q < n; ++q) {
        oi += si[q];
        of += sf[q];
        const double fo = floor(of);
        oi += (long long)fo;
        of -= fo;
        // correction = -(oi + of) = ni + nf, nf in [0, 1)
        long long ni = -oi;
        double nf = -of;
        if (nf < 0.0) {
          nf += 1.0;
          ni -= 1;
        }
        si[q] = ni;
        sf[q] = nf;
      }
    }
    __syncthreads();
    if (tid < n) {
      pb.shift[base + j] = ((double)si[tid] + sf[tid]) * kLn2;
      pb.corr_i[base + j] = si[tid];  // the scalar is consumed: now the chunk's correction
      pb.corr_f[base + j] = sf[tid];
    }
    __syncthreads();
  }
  if (tid == 0) {
    // the chain's log Z was computed in the frame of its last chunk
    const double lz = pb.lz_part[fwd ? b : sh.B + b] - ((double)oi + of) * kLn2;
    if (fwd) {
      logz_ws[b] = lz;
      logz_out[b] = (float)lz;
    } else if (logz_bwd_ws) {
      logz_bwd_ws[b] = lz;
    }
  }
}

// Every checkpoint record becomes the exact state with its exact log
// normaliser: the chunk's correction (integer part to the references,
// fraction to the ring, both to the absolute o / m rows).  One workgroup
// per (direction, sequence, chunk); the chain's exact chunk has none.
__global__ __launch_bounds__(kPitThreads) void k_pit_records(ChainShape sh,
                                                             const int32_t *__restrict__ lengths,
                                                             PitBufs pb, int with_bwd) {
  const int nck = sh.B * sh.nchunk;
  const bool fwd = (int)blockIdx.x < nck;
  if (!fwd && !with_bwd) return;
  const int rem = fwd ? blockIdx.x : blockIdx.x - nck;
  const int b = rem / sh.nchunk, j = rem % sh.nchunk;
  const int L = lengths[b];
  if (L < 1 || L > sh.T || j * sh.delta >= L) return;
  const int nvalid = (L + sh.delta - 1) / sh.delta;
  if (j == (fwd ? 0 : nvalid - 1)) return;
  const size_t idx = (fwd ? 0 : (size_t)nck) + (size_t)b * sh.nchunk + j;
  const long long ni = pb.corr_i[idx];
  const double nf = pb.corr_f[idx];
  const int C = sh.C, K = sh.K;
  double *rec = (fwd ? pb.ck_fwd : pb.ck_bwd) + ((size_t)b * sh.nchunk + j) * ck_stride(C, K);
  const double scale = exp2(nf), shift = pb.shift[idx];
  for (int i = threadIdx.x; i < K * C; i += kPitThreads) rec[i] *= scale;
  for (int c = threadIdx.x; c < C; c += kPitThreads) {
    rec[(size_t)K * C + c] = (double)((long long)rec[(size_t)K * C + c] + ni);
    rec[(size_t)K * C + C + c] += shift;
    rec[(size_t)K * C + 2 * C + c] += shift;
  }
}

// nchunk iterations always suffice (after n of them the first n chunks of
// every chain have exact starts); the ones after convergence return at once.
// Each position's row correction: the log correction of the chunk that
// wrote it (forward chunk j writes alpha and u at t in (p0, p1], t = 0
// belonging to chunk 0; backward chunk j writes v and beta at t in
// [p0, p1), t = L belonging to the last chunk).  pos_shift[0][b][t] and
// pos_shift[1][b][t], t = 0..T (0 past L and for invalid lengths).  A
// table of B*(T+1) pairs instead of a pass over the four [B][T+1][C] rows.
__global__ __launch_bounds__(kPitThreads) void k_pit_pos_shift(ChainShape sh,
                                                               const int32_t *__restrict__ lengths,
                                                               PitBufs pb) {
  const int b = blockIdx.y;
  const int L = lengths[b];
  const bool ok = L >= 1 && L <= sh.T;
  const int nvalid = ok ? (L + sh.delta - 1) / sh.delta : 1;
  const size_t nck = (size_t)sh.B * sh.nchunk;
  const double *sf = pb.shift + (size_t)b * sh.nchunk, *sb = pb.shift + nck + (size_t)b * sh.nchunk;
  double *of = pb.pos_shift + (size_t)b * (sh.T + 1), *ob = of + (size_t)sh.B * (sh.T + 1);
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t <= sh.T; t += gridDim.x * blockDim.x) {
    double f = 0.0, g = 0.0;
    if (ok && t <= L) {
      f = sf[min(t >= 1 ? (t - 1) / sh.delta : 0, nvalid - 1)];
      g = sb[min(t / sh.delta, nvalid - 1)];
    }
    of[t] = f;
    ob[t] = g;
  }
}

hipError_t run_sweeps(const ChainShape &sh, const float *trans, const float *dur,
                      const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                      double *logz_ws, double *logz_bwd_ws, float *logz_out, int with_bwd,
                      hipStream_t st, hipEvent_t after_first) {
  // iteration 0 of the sweep also sets every chunk's redo flag and scalar
  // and clears the per-iteration mismatch counts
  const int niter = sh.nchunk;
  hipError_t e = hipSuccess;
  if (pb.trw) {
    e = launch_trw(sh.C, sh.CS, sh.QT, trans, pb.trw, st);
    if (e != hipSuccess) return e;
  }
  // After iteration it the first it+1 chunks of the chain are exact, so the
  // last iteration can only sweep the chain's last chunk, which has no
  // successor to verify: no verification follows it (a chunk whose start
  // was replaced carries scalar 0, set with the copy).  Engines with an
  // in-order repair run kPitParallelIters iterations, then the repair.
  const bool repair = sh.win || sh.e64 || sh.e256;
  const int npar = repair && niter > kPitParallelIters ? kPitParallelIters : niter;
  for (int it = 0; it < npar; ++it) {
    e = launch_sweep(sh, trans, dur, es, lengths, pb, with_bwd, it, st);
    if (e != hipSuccess) return e;
    if (it == 0 && after_first) (void)hipEventRecord(after_first, st);
    if (it + 1 == niter) break;
    e = launch_pit_verify(sh, lengths, pb, it, with_bwd, st);
    if (e != hipSuccess) return e;
  }
  if (npar < niter) {
    e = launch_sweep(sh, trans, dur, es, lengths, pb, with_bwd, kPitRepair, st);
    if (e != hipSuccess) return e;
  }
  e = launch_pit_fixup(sh, lengths, pb, logz_ws, logz_bwd_ws, logz_out, with_bwd, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_pit_records, dim3(2 * sh.B * sh.nchunk), dim3(kPitThreads), 0, st, sh,
                     lengths, pb, with_bwd);
  e = hipGetLastError();
  if (e != hipSuccess || !pb.row_a) return e;
  int gx = (sh.T + 1 + kPitThreads - 1) / kPitThreads;
  gx = gx > 64 ? 64 : gx;
  hipLaunchKernelGGL(k_pit_pos_shift, dim3(gx, sh.B), dim3(kPitThreads), 0, st, sh, lengths, pb);
  return hipGetLastError();
}



hipError_t launch_pit_verify(const ChainShape &sh, const int32_t *lengths, const PitBufs &pb,
                             int iter, int with_bwd, hipStream_t st) {
  const int grid = (with_bwd ? 2 : 1) * sh.B * sh.nchunk;
  hipLaunchKernelGGL(k_pit_verify, dim3(grid), dim3(kPitThreads), 0, st, sh, lengths, pb, iter);
  return hipGetLastError();
}

hipError_t launch_pit_fixup(const ChainShape &sh, const int32_t *lengths, const PitBufs &pb,
                            double *logz_ws, double *logz_bwd_ws, float *logz_out, int with_bwd,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_pit_fixup, dim3(2 * sh.B), dim3(kPitThreads), 0, st, sh, lengths, pb,
                     logz_ws, logz_bwd_ws, logz_out, with_bwd);
  return hipGetLastError();
}

}  // namespace semicrf
