// scan.hip -- zero-centred cumulative scores (the prefix-sum array).
//
// "Streaming Structured Inference with Flash-SemiCRF": the abstract replaces
// the edge-potential tensor by a prefix-sum array and centres the cumulative
// scores; the technical summary (gist.science, section 2.A) reads a segment
// score as the difference of two prefix entries and (section 2.C) subtracts a
// per-sequence, per-label baseline nu[b,c] before summing.  Here
//   nu[b,c]  = (1/L_b) sum_{t<L_b} x[b,t,c]      (0 when centring is off)
//   S[b,t,c] = sum_{i<t} (x[b,i,c] - nu[b,c]),  t = 0..T  (rows > L_b repeat L_b)
// in float64, as a three-pass tiled scan over T:
//   1. per-tile column sums of x (coalesced over C, float64 accumulation);
//   2. per (sequence, label): nu and the exclusive tile prefix (tile anchors);
//   3. per tile: anchor + in-tile prefix, written as S and, for the sweeps,
//      split into exp(+-S) = mantissa * 2^(+-n) (two float64 and an int32).
// Positions t >= L_b are never read.  HBM traffic per (b,t,c): 4 B (pass 1)
// + 4 B read + 8 B write (pass 3), + 20 B when the split is written.
#include "device_math.h"
#include "internal.h"

namespace semicrf {

// Thread (r, c) of a tile owns positions [tile*TS + r*J, +J) of label c.
// Its J scores are loaded together, before the first use (positions past
// the sequence read a valid position and count 0).
template <int J>
__device__ __forceinline__ void load_scores(const float *__restrict__ xb, int t0, int L, int C,
                                            int c, float (&v)[J]) {
#pragma unroll
  for (int i = 0; i < J; ++i) {
    const int t = t0 + i < L ? t0 + i : L - 1;
    v[i] = xb[(size_t)t * C + c];
  }
}

template <int J>
__global__ __launch_bounds__(kScanThreads) void k_scan_partial(
    const float *__restrict__ x, const int32_t *__restrict__ lengths, int T, int C, int ntile,
    double *__restrict__ tile_sum) {
  __shared__ double red[kScanThreads];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int R = kScanThreads / C, TS = R * J;
  const int tid = threadIdx.x, c = tid % C, r = tid / C;
  const int L = lengths[b];
  const bool valid_len = L >= 1 && L <= T;
  double s = 0.0;
  const int t0 = tile * TS + r * J;
  if (r < R && valid_len && t0 < L) {
    float v[J];
    load_scores<J>(x + (size_t)b * T * C, t0, L, C, c, v);
#pragma unroll
    for (int i = 0; i < J; ++i) s += t0 + i < L ? (double)v[i] : 0.0;
  }
  red[tid] = s;
  __syncthreads();
  if (r == 0) {
    double tot = 0.0;
    for (int rr = 0; rr < R; ++rr) tot += red[rr * C + c];
    tile_sum[((size_t)b * ntile + tile) * C + c] = tot;
  }
}

// One block per (sequence, label): each thread owns a contiguous range of
// tiles; the per-thread totals are combined in a fixed order (deterministic).
__global__ __launch_bounds__(kScanThreads) void k_scan_anchor(
    const int32_t *__restrict__ lengths, int T, int C, int ntile, int J, int center,
    const double *__restrict__ tile_sum, double *__restrict__ anchor, double *__restrict__ nu) {
  __shared__ double red[kScanThreads];
  const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int L = lengths[b];
  const bool valid_len = L >= 1 && L <= T;
  const int TS = (kScanThreads / C) * J;
  const int per = (ntile + kScanThreads - 1) / kScanThreads;
  const int i0 = tid * per, i1 = min(i0 + per, ntile);
  const double *ts = tile_sum + (size_t)b * ntile * C + c;
  double own = 0.0;
  for (int i = i0; i < i1; ++i) own += ts[(size_t)i * C];
  red[tid] = own;
  __syncthreads();
  // threads past nq own no tile (ranges of `per` tiles from the start)
  const int nq = min(kScanThreads, (ntile + per - 1) / per);
  if (tid == 0) {
    double total = 0.0;
    for (int q = 0; q < nq; ++q) total += red[q];
    red[0] = total;
  }
  __syncthreads();
  const double n = (valid_len && center) ? red[0] / (double)L : 0.0;
  if (tid == 0) nu[(size_t)b * C + c] = valid_len ? n : __builtin_nan("");
  // tile i contributes tile_sum - (valid positions of tile i) * nu
  double part = 0.0;
  for (int i = i0; i < i1; ++i) {
    int nvalid = valid_len ? L - i * TS : 0;
    nvalid = nvalid < 0 ? 0 : (nvalid > TS ? TS : nvalid);
    part += ts[(size_t)i * C] - (double)nvalid * n;
  }
  __syncthreads();
  red[tid] = part;
  __syncthreads();
  if (tid == 0) {  // exclusive prefix over the threads, in order
    double run = 0.0;
    for (int q = 0; q < nq; ++q) {
      const double v = red[q];
      red[q] = run;
      run += v;
    }
  }
  __syncthreads();
  double run = red[tid];
  for (int i = i0; i < i1; ++i) {
    anchor[((size_t)b * ntile + i) * C + c] = run;
    int nvalid = valid_len ? L - i * TS : 0;
    nvalid = nvalid < 0 ? 0 : (nvalid > TS ? TS : nvalid);
    run += ts[(size_t)i * C] - (double)nvalid * n;
  }
}

// S is also written split for the exp-space recursion of the sweeps
// (exp_split: exp(+-S) as a float64 in [2^-1/2, 2^1/2] times 2^(+-n)) when
// ep is given.
template <int J>
__global__ __launch_bounds__(kScanThreads) void k_scan_write(
    const float *__restrict__ x, const int32_t *__restrict__ lengths, int T, int C, int ntile,
    const double *__restrict__ anchor, const double *__restrict__ nu, double *__restrict__ S,
    double *__restrict__ ep, double *__restrict__ em, int32_t *__restrict__ en) {
  __shared__ double red[kScanThreads];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int R = kScanThreads / C, TS = R * J;
  const int tid = threadIdx.x, c = tid % C, r = tid / C;
  const int L = lengths[b];
  const bool valid_len = L >= 1 && L <= T;
  const size_t ob = (size_t)b * (T + 1) * C;
  const double n = valid_len ? nu[(size_t)b * C + c] : 0.0;
  const int t0 = tile * TS + r * J;
  double xs[J];  // x - nu of the thread's positions, 0 past the sequence
#pragma unroll
  for (int i = 0; i < J; ++i) xs[i] = 0.0;
  if (r < R && valid_len && t0 < L) {
    float v[J];
    load_scores<J>(x + (size_t)b * T * C, t0, L, C, c, v);
#pragma unroll
    for (int i = 0; i < J; ++i) xs[i] = t0 + i < L ? (double)v[i] - n : 0.0;
  }
  double local = 0.0;
#pragma unroll
  for (int i = 0; i < J; ++i) local += xs[i];
  red[tid] = local;
  __syncthreads();
  if (r >= R) return;
  double run = anchor[((size_t)b * ntile + tile) * C + c];
  for (int rr = 0; rr < r; ++rr) run += red[rr * C + c];
  if (!valid_len) run = __builtin_nan("");
  auto put = [&](int t, double v) {
    const size_t o = ob + (size_t)t * C + c;
    S[o] = v;
    if (ep) {
      double p, m;
      int k;
      exp_split(v, p, m, k);
      ep[o] = p;
      em[o] = m;
      en[o] = k;
    }
  };
  if (tile == 0 && r == 0) put(0, valid_len ? 0.0 : run);
#pragma unroll
  for (int i = 0; i < J; ++i) {
    const int t = t0 + i;
    if (t < T) {
      run += xs[i];
      put(t + 1, run);
    }
  }
}

hipError_t launch_scan(const float *x, const int32_t *lengths, int B, int T, int C, int center,
                       double *nu, double *S, double *ep, double *em, int32_t *en,
                       double *tile_sum, double *anchor, int ntile, int J, hipStream_t st) {
  dim3 grid(ntile, B);
  switch (J) {
    case 8: hipLaunchKernelGGL(k_scan_partial<8>, grid, dim3(kScanThreads), 0, st, x, lengths, T, C, ntile, tile_sum); break;
    case 16: hipLaunchKernelGGL(k_scan_partial<16>, grid, dim3(kScanThreads), 0, st, x, lengths, T, C, ntile, tile_sum); break;
    case 32: hipLaunchKernelGGL(k_scan_partial<32>, grid, dim3(kScanThreads), 0, st, x, lengths, T, C, ntile, tile_sum); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_anchor, dim3(B, C), dim3(kScanThreads), 0, st, lengths, T, C, ntile,
                     J, center, tile_sum, anchor, nu);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (J) {
    case 8: hipLaunchKernelGGL(k_scan_write<8>, grid, dim3(kScanThreads), 0, st, x, lengths, T, C, ntile, anchor, nu, S, ep, em, en); break;
    case 16: hipLaunchKernelGGL(k_scan_write<16>, grid, dim3(kScanThreads), 0, st, x, lengths, T, C, ntile, anchor, nu, S, ep, em, en); break;
    default: hipLaunchKernelGGL(k_scan_write<32>, grid, dim3(kScanThreads), 0, st, x, lengths, T, C, ntile, anchor, nu, S, ep, em, en); break;
  }
  return hipGetLastError();
}

}  // namespace semicrf
