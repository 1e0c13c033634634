// path.hip -- score of a given labelled segmentation and its gradients.
//
// Training a semi-CRF minimises the negative log-likelihood of the gold
// segmentation, log Z - score(gold) ("Streaming Structured Inference with
// Flash-SemiCRF", technical summary at gist.science, section 3: training on
// labelled segmentations).  With the cumulative scores S of scan.hip, a
// segmentation (s_j, k_j, c_j), j < n, of [0, L) scores
//   score = sum_j (S[s_j + k_j, c_j] - S[s_j, c_j] + dur[k_j - 1, c_j])
//         + sum_{j >= 1} trans[c_{j-1}, c_j]
// (the same model as every other entry point: no transition into the first
// segment, no start/end scores).  Its gradients, for F = sum_b w_b score_b:
//   dF/dx[b,i,c]      = w_b (1[position i has label c] - n_bc / L_b)  (centred;
//                       without centring the indicator alone), n_bc the
//                       positions of label c; 0 at i >= L_b
//   dF/dtrans[c',c]   = sum_b w_b #(consecutive segments c' -> c)
//   dF/ddur[k-1,c]    = sum_b w_b #(segments of length k and label c)
// The counts are integers (integer atomics, exact); the weighted sums over
// the batch are formed in a fixed order in float64.
//
// A segmentation is valid when n is in [1, L], s_0 = 0, every segment
// starts where the previous one ended, 1 <= k_j <= K, 0 <= c_j < C and the
// last one ends at L.  Anything else (or a length outside [1, T]) gives
// score NaN and zero gradient rows, and the sequence is left out of the
// parameter gradients.
#include "device_math.h"
#include "internal.h"

namespace semicrf {

namespace {

constexpr int kPathThreads = 256;

__device__ __forceinline__ double block_sum_fixed(double v, double *red) {
  // fixed-order tree over the workgroup (deterministic)
  red[threadIdx.x] = v;
  __syncthreads();
  for (int h = kPathThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  const double s = red[0];
  __syncthreads();
  return s;
}

}  // namespace

// Zero the integer count tables (a fill kernel: the counts must start at 0).
__global__ void k_path_zero(int *p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// One workgroup per sequence: validity, the float64 score and the counts.
__global__ __launch_bounds__(kPathThreads) void k_path_score(
    ChainShape sh, const double *__restrict__ S, const int32_t *__restrict__ lengths,
    const float *__restrict__ trans, const float *__restrict__ dur,
    const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_len,
    const int32_t *__restrict__ seg_label, const int32_t *__restrict__ num_segs,
    float *__restrict__ score_out, double *__restrict__ score_ws, int *__restrict__ valid_ws,
    int *__restrict__ cnt_tr, int *__restrict__ cnt_du, int *__restrict__ cnt_lab) {
  __shared__ double red[kPathThreads];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int T = sh.T, C = sh.C, K = sh.K;
  const int L = lengths[b];
  const int n = num_segs[b];
  const size_t ob = (size_t)b * T;
  bool bad = L < 1 || L > T || n < 1 || n > L;
  double acc = 0.0;
  if (!bad) {
    const double *Sb = S + (size_t)b * (T + 1) * C;
    for (int j = tid; j < n; j += kPathThreads) {
      const int s = seg_start[ob + j], k = seg_len[ob + j], c = seg_label[ob + j];
      bool ok = k >= 1 && k <= K && c >= 0 && c < C && s >= 0 && s <= L - k;
      if (j == 0) {
        ok = ok && s == 0;
      } else {
        const int sp = seg_start[ob + j - 1], kp = seg_len[ob + j - 1], cp = seg_label[ob + j - 1];
        ok = ok && sp + kp == s && cp >= 0 && cp < C;
        if (ok) acc += (double)trans[(size_t)cp * C + c];
      }
      if (j == n - 1) ok = ok && s + k == L;
      if (ok) {
        acc += (Sb[(size_t)(s + k) * C + c] - Sb[(size_t)s * C + c]) + (double)dur[(size_t)(k - 1) * C + c];
      } else {
        bad = true;
      }
    }
  }
  bad = __syncthreads_or(bad ? 1 : 0) != 0;
  const double sc = block_sum_fixed(bad ? 0.0 : acc, red);
  if (tid == 0) {
    valid_ws[b] = bad ? 0 : 1;
    score_ws[b] = bad ? __builtin_nan("") : sc;
    score_out[b] = bad ? __builtin_nanf("") : (float)sc;
  }
  if (bad || !cnt_tr) return;
  // every segment is in range now: the counts (integer atomics: exact)
  for (int j = tid; j < n; j += kPathThreads) {
    const int k = seg_len[ob + j], c = seg_label[ob + j];
    atomicAdd(&cnt_du[((size_t)b * K + (k - 1)) * C + c], 1);
    atomicAdd(&cnt_lab[(size_t)b * C + c], k);
    if (j > 0) atomicAdd(&cnt_tr[((size_t)b * C + seg_label[ob + j - 1]) * C + c], 1);
  }
}

// Per-position label of the valid sequences: segment j of sequence b paints
// positions [s_j, s_j + k_j) (in range: the sequence passed validation).
__global__ __launch_bounds__(kPathThreads) void k_path_paint(
    ChainShape sh, const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_len,
    const int32_t *__restrict__ seg_label, const int32_t *__restrict__ num_segs,
    const int *__restrict__ valid_ws, int32_t *__restrict__ lab) {
  const int b = blockIdx.y;
  if (!valid_ws[b]) return;
  const int n = num_segs[b];
  const size_t ob = (size_t)b * sh.T;
  for (int j = blockIdx.x * kPathThreads + threadIdx.x; j < n; j += gridDim.x * kPathThreads) {
    const int s = seg_start[ob + j], k = seg_len[ob + j], c = seg_label[ob + j];
    for (int i = 0; i < k; ++i) lab[ob + s + i] = c;
  }
}

// dF/dx: coalesced over (position, label).
__global__ __launch_bounds__(kPathThreads) void k_path_grad_x(
    ChainShape sh, const int32_t *__restrict__ lengths, const float *__restrict__ w,
    const int *__restrict__ valid_ws, const int32_t *__restrict__ lab,
    const int *__restrict__ cnt_lab, float *__restrict__ grad_x) {
  const size_t n = (size_t)sh.B * sh.T * sh.C;
  for (size_t i = blockIdx.x * (size_t)kPathThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kPathThreads) {
    const int c = (int)(i % sh.C);
    const size_t bt = i / sh.C;
    const int t = (int)(bt % sh.T), b = (int)(bt / sh.T);
    float g = 0.f;
    if (valid_ws[b]) {
      const int L = lengths[b];
      if (t < L) {
        double v = lab[bt] == c ? 1.0 : 0.0;
        if (sh.center) v -= (double)cnt_lab[(size_t)b * sh.C + c] / (double)L;
        g = (float)((w ? (double)w[b] : 1.0) * v);
      }
    }
    grad_x[i] = g;
  }
}

// dF/dtrans and dF/ddur: sum over the batch in order (float64).
__global__ __launch_bounds__(kPathThreads) void k_path_grad_params(
    ChainShape sh, const float *__restrict__ w, const int *__restrict__ valid_ws,
    const int *__restrict__ cnt_tr, const int *__restrict__ cnt_du,
    float *__restrict__ grad_trans, float *__restrict__ grad_dur) {
  const int nx = sh.C * sh.C, nd = sh.K * sh.C;
  for (int e = blockIdx.x * kPathThreads + threadIdx.x; e < nx + nd; e += gridDim.x * kPathThreads) {
    const bool tx = e < nx;
    if (tx ? !grad_trans : !grad_dur) continue;
    double acc = 0.0;
    for (int b = 0; b < sh.B; ++b) {
      if (!valid_ws[b]) continue;
      const int cnt = tx ? cnt_tr[(size_t)b * nx + e] : cnt_du[(size_t)b * nd + (e - nx)];
      acc += (w ? (double)w[b] : 1.0) * (double)cnt;
    }
    if (tx)
      grad_trans[e] = (float)acc;
    else
      grad_dur[e - nx] = (float)acc;
  }
}

hipError_t launch_path_score(const ChainShape &sh, const PathArgs &pa, hipStream_t st) {
  const bool grads = pa.grad_x || pa.grad_trans || pa.grad_dur;
  hipError_t e;
  if (grads) {
    const size_t n = (size_t)sh.B * (sh.C * sh.C + sh.K * sh.C + sh.C);
    int grid = (int)((n + kPathThreads - 1) / kPathThreads);
    grid = grid > 1024 ? 1024 : grid;
    hipLaunchKernelGGL(k_path_zero, dim3(grid), dim3(kPathThreads), 0, st, pa.cnt, n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int *cnt_tr = grads ? pa.cnt : nullptr;
  int *cnt_du = grads ? pa.cnt + (size_t)sh.B * sh.C * sh.C : nullptr;
  int *cnt_lab = grads ? cnt_du + (size_t)sh.B * sh.K * sh.C : nullptr;
  hipLaunchKernelGGL(k_path_score, dim3(sh.B), dim3(kPathThreads), 0, st, sh, pa.S, pa.lengths,
                     pa.trans, pa.dur, pa.seg_start, pa.seg_len, pa.seg_label, pa.num_segs,
                     pa.score, pa.score_ws, pa.valid, cnt_tr, cnt_du, cnt_lab);
  e = hipGetLastError();
  if (e != hipSuccess || !grads) return e;
  if (pa.grad_x) {
    int gx = (sh.T + kPathThreads - 1) / kPathThreads;
    gx = gx > 256 ? 256 : gx;
    hipLaunchKernelGGL(k_path_paint, dim3(gx, sh.B), dim3(kPathThreads), 0, st, sh, pa.seg_start,
                       pa.seg_len, pa.seg_label, pa.num_segs, pa.valid, pa.lab);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n = (size_t)sh.B * sh.T * sh.C;
    long long grid = (long long)((n + kPathThreads - 1) / kPathThreads);
    grid = grid > 4096 ? 4096 : grid;
    hipLaunchKernelGGL(k_path_grad_x, dim3((int)grid), dim3(kPathThreads), 0, st, sh, pa.lengths,
                       pa.w, pa.valid, pa.lab, cnt_lab, pa.grad_x);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pa.grad_trans || pa.grad_dur) {
    const int ne = sh.C * sh.C + sh.K * sh.C;
    int grid = (ne + kPathThreads - 1) / kPathThreads;
    grid = grid > 1024 ? 1024 : grid;
    hipLaunchKernelGGL(k_path_grad_params, dim3(grid), dim3(kPathThreads), 0, st, sh, pa.w,
                       pa.valid, cnt_tr, cnt_du, pa.grad_trans, pa.grad_dur);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace semicrf
