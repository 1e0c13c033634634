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
//   2. per sequence: nu and the exclusive tile prefix (tile anchors);
//   3. per tile: anchor + in-tile prefix, written as S.
// Positions t >= L_b are never read.  HBM traffic per (b,t,c): 4 B (pass 1)
// + 4 B read + 8 B write (pass 3).
#include "internal.h"

namespace semicrf {

// Thread (r, c) of a tile owns positions [tile*TS + r*J, +J) of label c.
__global__ __launch_bounds__(kScanThreads) void k_scan_partial(
    const float *__restrict__ x, const int32_t *__restrict__ lengths, int T, int C, int ntile,
    double *__restrict__ tile_sum) {
  __shared__ double red[kScanThreads];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int R = kScanThreads / C, TS = R * kScanJ;
  const int tid = threadIdx.x, c = tid % C, r = tid / C;
  const int L = lengths[b];
  const bool valid_len = L >= 1 && L <= T;
  double s = 0.0;
  if (r < R && valid_len) {
    const int t0 = tile * TS + r * kScanJ;
    const float *xb = x + (size_t)b * T * C;
    for (int i = 0; i < kScanJ; ++i) {
      const int t = t0 + i;
      if (t < L) s += (double)xb[(size_t)t * C + c];
    }
  }
  red[tid] = s;
  __syncthreads();
  if (r == 0) {
    double tot = 0.0;
    for (int rr = 0; rr < R; ++rr) tot += red[rr * C + c];
    tile_sum[((size_t)b * ntile + tile) * C + c] = tot;
  }
}

// One block per sequence; threads loop over labels.
__global__ __launch_bounds__(kScanThreads) void k_scan_anchor(
    const int32_t *__restrict__ lengths, int T, int C, int ntile, int center,
    const double *__restrict__ tile_sum, double *__restrict__ anchor, double *__restrict__ nu) {
  const int b = blockIdx.x;
  const int L = lengths[b];
  const bool valid_len = L >= 1 && L <= T;
  const int TS = (kScanThreads / C) * kScanJ;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    double total = 0.0;
    for (int i = 0; i < ntile; ++i) total += tile_sum[((size_t)b * ntile + i) * C + c];
    const double n = (valid_len && center) ? total / (double)L : 0.0;
    nu[(size_t)b * C + c] = valid_len ? n : __builtin_nan("");
    double run = 0.0;
    for (int i = 0; i < ntile; ++i) {
      anchor[((size_t)b * ntile + i) * C + c] = run;
      int nvalid = valid_len ? L - i * TS : 0;
      nvalid = nvalid < 0 ? 0 : (nvalid > TS ? TS : nvalid);
      run += tile_sum[((size_t)b * ntile + i) * C + c] - (double)nvalid * n;
    }
  }
}

__global__ __launch_bounds__(kScanThreads) void k_scan_write(
    const float *__restrict__ x, const int32_t *__restrict__ lengths, int T, int C, int ntile,
    const double *__restrict__ anchor, const double *__restrict__ nu, double *__restrict__ S) {
  __shared__ double red[kScanThreads];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int R = kScanThreads / C, TS = R * kScanJ;
  const int tid = threadIdx.x, c = tid % C, r = tid / C;
  const int L = lengths[b];
  const bool valid_len = L >= 1 && L <= T;
  const float *xb = x + (size_t)b * T * C;
  double *Sb = S + (size_t)b * (T + 1) * C;
  const double n = valid_len ? nu[(size_t)b * C + c] : 0.0;
  const int t0 = tile * TS + r * kScanJ;
  double local = 0.0;
  if (r < R && valid_len) {
    for (int i = 0; i < kScanJ; ++i) {
      const int t = t0 + i;
      if (t < L) local += (double)xb[(size_t)t * C + c] - n;
    }
  }
  red[tid] = local;
  __syncthreads();
  if (r >= R) return;
  double run = anchor[((size_t)b * ntile + tile) * C + c];
  for (int rr = 0; rr < r; ++rr) run += red[rr * C + c];
  if (!valid_len) run = __builtin_nan("");
  if (tile == 0 && r == 0) Sb[c] = valid_len ? 0.0 : run;
  for (int i = 0; i < kScanJ; ++i) {
    const int t = t0 + i;
    if (t >= T) break;
    if (t < L) run += (double)xb[(size_t)t * C + c] - n;
    Sb[(size_t)(t + 1) * C + c] = run;
  }
}

hipError_t launch_scan(const float *x, const int32_t *lengths, int B, int T, int C, int center,
                       double *nu, double *S, double *tile_sum, double *anchor, int ntile,
                       hipStream_t st) {
  dim3 grid(ntile, B);
  hipLaunchKernelGGL(k_scan_partial, grid, dim3(kScanThreads), 0, st, x, lengths, T, C, ntile,
                     tile_sum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_anchor, dim3(B), dim3(kScanThreads), 0, st, lengths, T, C, ntile,
                     center, tile_sum, anchor, nu);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_write, grid, dim3(kScanThreads), 0, st, x, lengths, T, C, ntile,
                     anchor, nu, S);
  return hipGetLastError();
}

}  // namespace semicrf
