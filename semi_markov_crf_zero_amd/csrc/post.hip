// post.hip -- posteriors and gradients from the per-position rows.
//
// With the forward rows alpha[t,c], u[t,c] and the backward rows v[t,c],
// beta[t,c] of every position (written by the parallel-in-time sweeps, see
// pit.hip), every marginal of the semi-CRF has a closed form, so this whole
// pass is data-parallel -- no recursion, no dependent chain:
//   segment     P(s,k,c)    = exp(u[s,c] + S[s+k,c] - S[s,c] + dur[k-1,c] + beta[s+k,c] - logZ)
//   transition  P(t,c'->c)  = exp(alpha[t,c'] + trans[c',c] + v[t,c] - logZ),   1 <= t < L
//   boundaries  E_start[t,c] = exp(u + v - logZ),  E_end[t,c] = exp(alpha + beta - logZ)
//   coverage    mu[i,c]     = sum_{t <= i} (E_start[t,c] - E_end[t,c])
// and with F = sum_b w_b log Z_b (technical summary of "Streaming Structured
// Inference with Flash-SemiCRF", section 2.C: exact gradients):
//   dF/d dur[k-1,c]  = sum_b w_b sum_s P(s,k,c)
//   dF/d trans[c',c] = sum_b w_b sum_t P(t,c'->c)
//   dF/d x[b,i,c]    = w_b (mu[i,c] - mean_j mu[j,c])   (centred; w_b mu[i,c] otherwise)
// Every reduction goes through per-block partials summed in a fixed order in
// float64 (deterministic; no floating-point atomics).
#include "device_math.h"
#include "internal.h"

namespace semicrf {

typedef double v4d __attribute__((ext_vector_type(4)));  // an MFMA float64 accumulator

namespace {

constexpr int kCovThreads = 256;
// consecutive positions per coverage thread: 16, halved (down to 4) while a
// batch has fewer than kCovTiles tiles (short sequences need the parallelism)
constexpr int kCovJ = 16, kCovJMin = 4, kCovTiles = 1024;  // J: a kernel instance each
constexpr int kTxThreads = 256;
constexpr int kTxTile = 64;   // output tile of the transition GEMM (64 x 64)
constexpr int kTxRows = 32;   // positions staged in LDS per batch
constexpr int kDurThreads = 256;
constexpr int kDurW = 64;     // positions per duration tile
constexpr long long kPostWorkgroups = 1024;  // grid size the posterior geometry aims for

// Row t of sequence b in the row buffers (which may cover a window only).
__device__ __forceinline__ size_t rix(const ChainShape &sh, const PostArgs &pa, int b, int t) {
  return ((size_t)b * pa.row_stride + (t - pa.row_t0)) * sh.C;
}

// The rows' chunk corrections at t (forward, backward): 0 for exact rows.
__device__ __forceinline__ double shift_f(const ChainShape &sh, const PostArgs &pa, int b, int t) {
  return pa.pos_shift ? pa.pos_shift[(size_t)b * (sh.T + 1) + t] : 0.0;
}
__device__ __forceinline__ double shift_b(const ChainShape &sh, const PostArgs &pa, int b, int t) {
  return pa.pos_shift ? pa.pos_shift[((size_t)sh.B + b) * (sh.T + 1) + t] : 0.0;
}

__device__ __forceinline__ bool valid_len(const ChainShape &sh, int L) { return L >= 1 && L <= sh.T; }

}  // namespace

// ------------------------------------------------------------ coverage
// Tiles of R x J positions (R = kCovThreads / C rows of threads, thread
// (r, c) owns J consecutive positions of label c), as in the score scan.
// delta[t,c] = E_start[t,c] - E_end[t,c] (E_end[0] = 0), float64-accurate:
// the coverage is their running sum over the whole sequence.
// The deltas of positions t0 .. t0+J-1 of label c (0 at t >= lim, lim the
// end of the sequence or of the window).  Every load is issued before the
// first exponential (indices clamped into [t0, lim)), so a thread waits for
// memory once rather than once per position.
template <int J>
__device__ __forceinline__ void cov_deltas(const PostArgs &pa, const ChainShape &sh, int b,
                                           int t0, int c, int lim, double logZ, double (&d)[J]) {
  double u[J], v[J], a[J], w[J], z[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int t = t0 + j < lim ? t0 + j : lim - 1;
    const size_t i = rix(sh, pa, b, t) + c;
    u[j] = pa.row_u[i];
    v[j] = pa.row_v[i];
    a[j] = pa.row_a[i];
    w[j] = pa.row_b[i];
    // the rows' chunk corrections, less log Z
    z[j] = shift_f(sh, pa, b, t) + shift_b(sh, pa, b, t) - logZ;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int t = t0 + j;
    double dd = exp(u[j] + v[j] + z[j]);
    if (t >= 1) dd -= exp(a[j] + w[j] + z[j]);
    d[j] = t < lim ? dd : 0.0;
  }
}

template <int J>
__global__ __launch_bounds__(kCovThreads) void k_cov_partial(ChainShape sh, PostArgs pa,
                                                             int ntile) {
  __shared__ double red1[kCovThreads], red2[kCovThreads];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int C = sh.C, R = kCovThreads / C, tid = threadIdx.x;
  const int c = tid % C, r = tid / C;
  const int L = pa.lengths[b];
  const int lim = min(L, pa.t_hi);
  double s1 = 0.0, s2 = 0.0;
  const int t0 = pa.t_lo + tile * R * J + r * J;
  if (r < R && valid_len(sh, L) && t0 < lim) {
    double d[J];
    cov_deltas<J>(pa, sh, b, t0, c, lim, pa.logz[b], d);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      s1 += d[j];
      s2 += d[j] * (double)(L - (t0 + j));  // sum_{i<L} mu[i] = sum_t delta[t] (L - t)
    }
  }
  red1[tid] = s1;
  red2[tid] = s2;
  __syncthreads();
  if (tid < C) {
    double a1 = 0.0, a2 = 0.0;
    for (int q = 0; q < R; ++q) {
      a1 += red1[q * C + tid];
      a2 += red2[q * C + tid];
    }
    const size_t o = ((size_t)b * ntile + tile) * C + tid;
    pa.cov_part[o] = a1;
    pa.cov_part2[o] = a2;
  }
}

// Exclusive prefix over tiles per (b, c) and the mean coverage.  One block
// per (sequence, label); each thread owns a contiguous range of tiles and
// the per-thread totals are combined in a fixed order.
__global__ __launch_bounds__(kCovThreads) void k_cov_anchor(ChainShape sh, PostArgs pa, int ntile) {
  __shared__ double red[kCovThreads], red2[kCovThreads];
  const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int L = pa.lengths[b];
  const int per = (ntile + kCovThreads - 1) / kCovThreads;
  const int i0 = tid * per, i1 = min(i0 + per, ntile);
  const size_t base = (size_t)b * ntile * sh.C + c;
  double own = 0.0, own2 = 0.0;
  for (int i = i0; i < i1; ++i) {
    own += pa.cov_part[base + (size_t)i * sh.C];
    own2 += pa.cov_part2[base + (size_t)i * sh.C];
  }
  red[tid] = own;
  red2[tid] = own2;
  __syncthreads();
  const int nq = min(kCovThreads, (ntile + per - 1) / per);  // threads that own tiles
  if (tid == 0) {
    // a windowed pass continues from the earlier windows' running sum
    const size_t bc = (size_t)b * sh.C + c;
    double run = pa.accumulate ? pa.cov_carry[bc] : 0.0, tot2 = 0.0;
    for (int q = 0; q < nq; ++q) {
      const double v = red[q];
      red[q] = run;
      run += v;
      tot2 += red2[q];
    }
    const double m = valid_len(sh, L) ? tot2 / (double)L : 0.0;
    pa.cov_mean[bc] = pa.accumulate ? pa.cov_mean[bc] + m : m;
    if (pa.cov_carry) pa.cov_carry[bc] = run;
  }
  __syncthreads();
  double run = red[tid];
  for (int i = i0; i < i1; ++i) {
    pa.cov_anchor[base + (size_t)i * sh.C] = run;
    run += pa.cov_part[base + (size_t)i * sh.C];
  }
}

template <int J>
__global__ __launch_bounds__(kCovThreads) void k_cov_write(ChainShape sh, PostArgs pa, int ntile) {
  __shared__ double runs[kCovThreads];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int C = sh.C, R = kCovThreads / C, tid = threadIdx.x;
  const int c = tid % C, r = tid / C;
  const int L = pa.lengths[b];
  const bool ok = valid_len(sh, L);
  const double logZ = ok ? pa.logz[b] : 0.0;
  const int lim = min(L, pa.t_hi);
  const int t0 = pa.t_lo + tile * R * J + r * J;
  double d[J];
#pragma unroll
  for (int j = 0; j < J; ++j) d[j] = 0.0;
  if (r < R && ok && t0 < lim) cov_deltas<J>(pa, sh, b, t0, c, lim, logZ, d);
  double own = 0.0;
#pragma unroll
  for (int j = 0; j < J; ++j) own += d[j];
  runs[tid] = own;
  __syncthreads();
  if (r >= R) return;
  double mu = 0.0, mean = 0.0, w = 1.0;
  if (ok) {
    mu = pa.cov_anchor[((size_t)b * ntile + tile) * C + c];
    for (int q = 0; q < r; ++q) mu += runs[q * C + c];
    mean = (sh.center && !pa.defer_mean) ? pa.cov_mean[(size_t)b * C + c] : 0.0;
    w = pa.grad_logz ? (double)pa.grad_logz[b] : 1.0;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int t = t0 + j;
    if (t < pa.t_hi) {
      float m_out = 0.f, g_out = 0.f;
      if (ok && t < L) {
        mu += d[j];
        m_out = (float)mu;
        g_out = (float)(w * (mu - mean));
      }
      const size_t o = ((size_t)b * sh.T + t) * C + c;
      pa.grad_emissions[o] = g_out;
      if (pa.marginals) pa.marginals[o] = m_out;
    }
  }
}

// ---------------------------------------------------------- transitions
// X[c',c] = sum_{t=1}^{L-1} exp(alpha[t,c'] + v[t,c] - logZ) as an exp-space
// GEMM over positions: a[t,c'] = exp(alpha[t,c'] - m_t) and
// g[t,c] = exp(v[t,c] + m_t - logZ), m_t the largest alpha of the block's
// rows (a <= 1, and g <= exp(-min trans): no overflow).  One workgroup per
// (64 x 64 output tile, sequence, position segment), four waves; the
// products run on the matrix cores in float64: wave (wi, wj) owns the
// 32 x 32 block at rows 32 wi, columns 32 wj of the tile as 2 x 2 blocks of
// 16 x 16, and every 4 staged positions add one v_mfma_f64_16x16x4 per
// block (A = a^T: lane l holds a[position 4k' + l / 16][row l % 16], B = g:
// lane l holds g[position 4k' + l / 16][column l % 16]; element r of the
// accumulator of lane l is row l / 16 + 4 r, column l % 16 -- the float64
// instruction's layout, checked on the device).
__global__ __launch_bounds__(kTxThreads) void k_trans_x(ChainShape sh, PostArgs pa, int tseg,
                                                        int nseg) {
  __shared__ double ta[kTxRows][kTxTile];
  __shared__ double tg[kTxRows][kTxTile];
  const int ntc = (sh.C + kTxTile - 1) / kTxTile;
  const int ti = blockIdx.x / ntc, tj = blockIdx.x % ntc;  // rows c' / columns c
  const int b = blockIdx.y / nseg, seg = blockIdx.y % nseg;
  const int C = sh.C, tid = threadIdx.x;
  const int L = pa.lengths[b];
  const int ci0 = ti * kTxTile, cj0 = tj * kTxTile;
  v4d acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = v4d{0.0, 0.0, 0.0, 0.0};
  int tbeg = max(1, pa.t_lo) + seg * tseg, tend = tbeg + tseg;
  if (!valid_len(sh, L)) tend = tbeg;
  if (tend > L) tend = L;  // transitions at 1 <= t < L
  if (tend > pa.t_hi) tend = pa.t_hi;
  const double logZ = valid_len(sh, L) ? pa.logz[b] : 0.0;
  // staging: wave w holds rows 4u + w of the batch (u < kTxPer), lane =
  // column, so each row's maximum is a wave reduction; every load of a batch
  // is issued before the first use (indices clamped, invalid entries masked)
  constexpr int kTxPer = kTxRows * kTxTile / kTxThreads;
  static_assert(kTxTile == 64 && kTxThreads == 256, "a staged row is one wave, four waves");
  const int lane = tid & 63, w = tid >> 6;
  const int ca = min(ci0 + lane, C - 1), cg = min(cj0 + lane, C - 1);
  for (int r0 = tbeg; r0 < tend; r0 += kTxRows) {
    const int nr = min(kTxRows, tend - r0);
    double va[kTxPer], vg[kTxPer], vz[kTxPer];
#pragma unroll
    for (int u = 0; u < kTxPer; ++u) {
      const int rr = 4 * u + w, t = r0 + min(rr, nr - 1);
      const size_t ri = rix(sh, pa, b, t);
      va[u] = pa.row_a[ri + ca];
      vg[u] = pa.row_v[ri + cg];
      // the rows' chunk corrections (alpha forward, v backward), less log Z
      vz[u] = shift_f(sh, pa, b, t) + shift_b(sh, pa, b, t) - logZ;
    }
    __syncthreads();  // the previous batch's products are done with ta / tg
#pragma unroll
    for (int u = 0; u < kTxPer; ++u) {
      const int rr = 4 * u + w;
      const bool ina = rr < nr && ci0 + lane < C;
      const bool ing = rr < nr && cj0 + lane < C;
      const double m = group_max(ina ? va[u] : -__builtin_huge_val(), 64);
      ta[rr][lane] = ina ? exp_wide(va[u] - m) : 0.0;
      tg[rr][lane] = ing ? exp_wide(vg[u] + m + vz[u]) : 0.0;
    }
    __syncthreads();
    // rows past nr were staged as zeros, so whole groups of 4 run
    const int kq = lane >> 4, li = lane & 15, wi = w >> 1, wj = w & 1;
#pragma unroll
    for (int kk = 0; kk < kTxRows; kk += 4) {
      const double a0 = ta[kk + kq][32 * wi + li], a1 = ta[kk + kq][32 * wi + 16 + li];
      const double g0 = tg[kk + kq][32 * wj + li], g1 = tg[kk + kq][32 * wj + 16 + li];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, g0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, g1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, g0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, g1, acc[1][1], 0, 0, 0);
    }
  }
  double *out = pa.tx_part + ((size_t)b * nseg + seg) * C * C;
  const int kq = lane >> 4, li = lane & 15, wi = w >> 1, wj = w & 1;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cp = ci0 + 32 * wi + 16 * x + kq + 4 * r, c = cj0 + 32 * wj + 16 * y + li;
        if (cp < C && c < C) {
          const size_t o = (size_t)cp * C + c;
          out[o] = pa.accumulate ? out[o] + acc[x][y][r] : acc[x][y][r];
        }
      }
}

// The same for C > 64 with 128 x 128 output tiles: each row element is
// staged and exponentiated by half as many tiles, and a row's maximum is one
// wave reduction over two elements per lane.  Batches of 16 positions (the
// two staged tiles take 32 KB); wave (wi, wj) accumulates the 64 x 64 block
// (64 wi, 64 wj) as 4 x 4 blocks of 16 x 16.
constexpr int kTx128 = 128, kTx128Rows = 16;
__global__ __launch_bounds__(kTxThreads, 2) void k_trans_x128(ChainShape sh, PostArgs pa, int tseg,
                                                           int nseg) {
  __shared__ double ta[kTx128Rows][kTx128];
  __shared__ double tg[kTx128Rows][kTx128];
  const int ntc = (sh.C + kTx128 - 1) / kTx128;
  const int ti = blockIdx.x / ntc, tj = blockIdx.x % ntc;  // rows c' / columns c
  const int b = blockIdx.y / nseg, seg = blockIdx.y % nseg;
  const int C = sh.C, tid = threadIdx.x;
  const int L = pa.lengths[b];
  const int ci0 = ti * kTx128, cj0 = tj * kTx128;
  v4d acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = v4d{0.0, 0.0, 0.0, 0.0};
  int tbeg = max(1, pa.t_lo) + seg * tseg, tend = tbeg + tseg;
  if (!valid_len(sh, L)) tend = tbeg;
  if (tend > L) tend = L;  // transitions at 1 <= t < L
  if (tend > pa.t_hi) tend = pa.t_hi;
  const double logZ = valid_len(sh, L) ? pa.logz[b] : 0.0;
  // staging: wave w holds rows 4u + w of the batch (u < kPer), lane l the
  // columns l and 64 + l; every load of a batch is issued before the first
  // use (indices clamped, invalid entries masked)
  constexpr int kPer = kTx128Rows / (kTxThreads / 64);
  const int lane = tid & 63, w = tid >> 6;
  const int ca0 = min(ci0 + lane, C - 1), ca1 = min(ci0 + 64 + lane, C - 1);
  const int cg0 = min(cj0 + lane, C - 1), cg1 = min(cj0 + 64 + lane, C - 1);
  for (int r0 = tbeg; r0 < tend; r0 += kTx128Rows) {
    const int nr = min(kTx128Rows, tend - r0);
    double va0[kPer], va1[kPer], vg0[kPer], vg1[kPer], vz[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int rr = 4 * u + w, t = r0 + min(rr, nr - 1);
      const size_t ri = rix(sh, pa, b, t);
      va0[u] = pa.row_a[ri + ca0];
      va1[u] = pa.row_a[ri + ca1];
      vg0[u] = pa.row_v[ri + cg0];
      vg1[u] = pa.row_v[ri + cg1];
      vz[u] = shift_f(sh, pa, b, t) + shift_b(sh, pa, b, t) - logZ;
    }
    __syncthreads();  // the previous batch's products are done with ta / tg
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int rr = 4 * u + w;
      const bool ia0 = rr < nr && ci0 + lane < C, ia1 = rr < nr && ci0 + 64 + lane < C;
      const bool ig0 = rr < nr && cj0 + lane < C, ig1 = rr < nr && cj0 + 64 + lane < C;
      const double m = group_max(fmax(ia0 ? va0[u] : -__builtin_huge_val(),
                                      ia1 ? va1[u] : -__builtin_huge_val()), 64);
      ta[rr][lane] = ia0 ? exp_wide(va0[u] - m) : 0.0;
      ta[rr][64 + lane] = ia1 ? exp_wide(va1[u] - m) : 0.0;
      tg[rr][lane] = ig0 ? exp_wide(vg0[u] + m + vz[u]) : 0.0;
      tg[rr][64 + lane] = ig1 ? exp_wide(vg1[u] + m + vz[u]) : 0.0;
    }
    __syncthreads();
    // rows past nr were staged as zeros, so whole groups of 4 run
    const int kq = lane >> 4, li = lane & 15, wi = w >> 1, wj = w & 1;
#pragma unroll
    for (int kk = 0; kk < kTx128Rows; kk += 4) {
      double a[4], g[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        a[x] = ta[kk + kq][64 * wi + 16 * x + li];
        g[x] = tg[kk + kq][64 * wj + 16 * x + li];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[x], g[y], acc[x][y], 0, 0, 0);
    }
  }
  double *out = pa.tx_part + ((size_t)b * nseg + seg) * C * C;
  const int kq = lane >> 4, li = lane & 15, wi = w >> 1, wj = w & 1;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cp = ci0 + 64 * wi + 16 * x + kq + 4 * r, c = cj0 + 64 * wj + 16 * y + li;
        if (cp < C && c < C) {
          const size_t o = (size_t)cp * C + c;
          out[o] = pa.accumulate ? out[o] + acc[x][y][r] : acc[x][y][r];
        }
      }
}

// The same for C <= 16, where a 64 x 64 tile would leave 15 of its 16
// matrix blocks empty: a staged 64-lane row holds 4 positions x 16 labels
// (lane 16p + c), each wave multiplies its own quarter of a 64-position
// batch into the one 16 x 16 block (every matrix instruction fully used,
// every staged lane live), and the four waves' blocks are added in a fixed
// order at the end.
constexpr int kTx16Rows = 64;  // positions staged per batch (C <= 16)
__global__ __launch_bounds__(kTxThreads) void k_trans_x16(ChainShape sh, PostArgs pa, int tseg,
                                                          int nseg) {
  __shared__ double ta[kTx16Rows][16];
  __shared__ double tg[kTx16Rows][16];
  __shared__ double red[kTxThreads / 64][16][17];
  const int b = blockIdx.y / nseg, seg = blockIdx.y % nseg;
  const int C = sh.C, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = pa.lengths[b];
  const int p = lane >> 4, c = lane & 15, cc = min(c, C - 1);
  v4d acc = v4d{0.0, 0.0, 0.0, 0.0};
  int tbeg = max(1, pa.t_lo) + seg * tseg, tend = tbeg + tseg;
  if (!valid_len(sh, L)) tend = tbeg;
  if (tend > L) tend = L;  // transitions at 1 <= t < L
  if (tend > pa.t_hi) tend = pa.t_hi;
  const double logZ = valid_len(sh, L) ? pa.logz[b] : 0.0;
  // staging: thread (wave w, lane 16p + c) holds label c of the positions
  // 16u + 4w + p of the batch; every load of a batch is issued before the
  // first use (indices clamped, invalid entries masked)
  constexpr int kPer = kTx16Rows * 16 / kTxThreads;
  static_assert(kTxThreads == 256 && kPer * kTxThreads == kTx16Rows * 16, "four waves");
  for (int r0 = tbeg; r0 < tend; r0 += kTx16Rows) {
    const int nr = min(kTx16Rows, tend - r0);
    double va[kPer], vg[kPer], vz[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int rr = 16 * u + 4 * w + p, t = r0 + min(rr, nr - 1);
      const size_t ri = rix(sh, pa, b, t);
      va[u] = pa.row_a[ri + cc];
      vg[u] = pa.row_v[ri + cc];
      vz[u] = shift_f(sh, pa, b, t) + shift_b(sh, pa, b, t) - logZ;
    }
    __syncthreads();  // the previous batch's products are done with ta / tg
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int rr = 16 * u + 4 * w + p;
      const bool in = rr < nr && c < C;
      const double m = group_max(in ? va[u] : -__builtin_huge_val(), 16);  // the row's maximum
      ta[rr][c] = in ? exp_wide(va[u] - m) : 0.0;
      tg[rr][c] = in ? exp_wide(vg[u] + m + vz[u]) : 0.0;
    }
    __syncthreads();
    // wave w: positions 16w .. 16w+15 of the batch, 4 per instruction
    // (rows past nr were staged as zeros)
#pragma unroll
    for (int kk = 0; kk < 16; kk += 4) {
      const double a = ta[16 * w + kk + p][c], g = tg[16 * w + kk + p][c];
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, g, acc, 0, 0, 0);
    }
  }
  // element r of lane 16p + c is entry (p + 4r, c) of the wave's block
#pragma unroll
  for (int r = 0; r < 4; ++r) red[w][p + 4 * r][c] = acc[r];
  __syncthreads();
  const int cp = tid >> 4, cq = tid & 15;
  const double v = ((red[0][cp][cq] + red[1][cp][cq]) + red[2][cp][cq]) + red[3][cp][cq];
  if (cp < C && cq < C) {
    double *out = pa.tx_part + ((size_t)b * nseg + seg) * C * C;
    const size_t o = (size_t)cp * C + cq;
    out[o] = pa.accumulate ? out[o] + v : v;
  }
}

// ------------------------------------------------------------ durations
// D[k,c] = sum_s exp(a[s,c] + b[s+k,c] + dur[k-1,c]) with
// a[s,c] = u[s,c] - S[s,c] and b[e,c] = S[e,c] + beta[e,c] - logZ, for
// s + k <= L.  One workgroup per (label group of up to 16, lag group of up
// to kDurLags lags, sequence, span of position tiles); thread (label cl, lag
// block kb) owns KB consecutive lags.  LDS: a for the tile's positions, b
// for the ends its lags reach.
//
// Each term factors as exp(a[s] - r) * exp(b[s+k] + r) * exp(dur), so per
// tile and label, with r the tile's largest a, the sum over s is an
// exp-space correlation: one float64 fused multiply-add per segment cell,
// in blocks of 8 starts x 8 lags from a register window, and exp(dur)
// applied once at the end.  Every factor stays within exp(+-(range of a
// over the tile + |dur|)): a segment starting inside the tile has
// probability at most 1, and a start and an end at most K + kDurW apart
// relate through one.  A tile whose range of a exceeds kDurRange nats (only
// with extreme scores) takes the direct path for that label: one exp per
// cell.
constexpr int kDurLags = 256;
static_assert(kDurW % 8 == 0, "duration tiles hold whole blocks of 8 starts");
constexpr double kDurRange = 600.0;

template <int KB>
__global__ __launch_bounds__(kDurThreads) void k_dur_x(ChainShape sh, PostArgs pa, int span,
                                                       int nspan, int npg) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int C = sh.C, K = sh.K, tid = threadIdx.x;
  const int cg = blockIdx.x / npg, pg = blockIdx.x % npg;
  const int b = blockIdx.y / nspan, sp = blockIdx.y % nspan;
  const int c0 = cg * 16, CG = min(16, C - c0);
  const int klo = 1 + pg * kDurLags, khi = min(K, (pg + 1) * kDurLags);  // lags [klo, khi]
  const int cl = tid % CG, kb = tid / CG;
  const int k0 = klo + kb * KB;
  const bool act = tid < CG * (kDurThreads / CG) && k0 <= khi;
  const int c = c0 + cl;
  const int L = pa.lengths[b];
  double *sa = reinterpret_cast<double *>(lds);  // [kDurW][16]
  // [kDurW + lags + KB][16], index e - s0 - klo; the rows past the tile's
  // last end are zero on the fast path, so its reads need no bound check
  // (+8: the end-row window of the fast path slides once past the tile)
  const int sbrows = kDurW + min(K, kDurLags) + KB + 8;
  double *sb = sa + (size_t)kDurW * 16;
  double *pmax = sb + (size_t)sbrows * 16;  // [4][16] per-wave max / min of a
  double *pmin = pmax + 64;
  double *rho = pmin + 64;                       // [16] reference per label
  int *fast = reinterpret_cast<int *>(rho + 16);  // [16]
  // sum over the starts of exp(a[s] + b[s+k]) per lag; exp(dur) is applied
  // once at the end, so the duration biases need no registers meanwhile
  double acc[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) acc[j] = 0.0;
  if (valid_len(sh, L)) {
    const double logZ = pa.logz[b];
    const double *Sb = pa.S + (size_t)b * (sh.T + 1) * C;
    const int sbeg = pa.t_lo + sp * span * kDurW;
    const int send = min(min(sbeg + span * kDurW, L), pa.t_hi);  // segment starts s < L
    for (int s0 = sbeg; s0 < send; s0 += kDurW) {
      const int ns = min(kDurW, send - s0);
      // ends e in [s0 + klo, min(s0 + ns - 1 + khi, L)]
      const int ne = min(ns - 1 + khi - klo + 1, L - s0 - klo + 1);
      __syncthreads();
      // staging: thread (row r0 + 16 i, label column cc); the row's index
      // and correction once per row, no division; the loads of a batch of
      // rows are all issued before the first use (row indices clamped into
      // the tile, stores masked)
      const int cc = tid & 15, r0 = tid >> 4;
      constexpr int RS = kDurThreads / 16;  // row stride
      if (cc < CG) {
        {
          constexpr int NA = kDurW / RS;  // start rows per thread
          double u[NA], f[NA], sv[NA];
#pragma unroll
          for (int i = 0; i < NA; ++i) {
            const int t = s0 + min(r0 + RS * i, ns - 1);
            u[i] = pa.row_u[rix(sh, pa, b, t) + c0 + cc];
            f[i] = shift_f(sh, pa, b, t);
            sv[i] = Sb[(size_t)t * C + c0 + cc];
          }
#pragma unroll
          for (int i = 0; i < NA; ++i)
            if (r0 + RS * i < ns) sa[(r0 + RS * i) * 16 + cc] = (u[i] + f[i]) - sv[i];
        }
        constexpr int NE = 8;  // end rows per batch
        for (int e0 = r0; e0 < ne; e0 += NE * RS) {
          double sv[NE], bv[NE], fv[NE];
#pragma unroll
          for (int i = 0; i < NE; ++i) {
            const int e = s0 + klo + min(e0 + RS * i, ne - 1);
            sv[i] = Sb[(size_t)e * C + c0 + cc];
            bv[i] = pa.row_b[rix(sh, pa, b, e) + c0 + cc];
            fv[i] = shift_b(sh, pa, b, e);
          }
#pragma unroll
          for (int i = 0; i < NE; ++i)
            if (e0 + RS * i < ne) sb[(e0 + RS * i) * 16 + cc] = (sv[i] + (bv[i] + fv[i])) - logZ;
        }
      }
      __syncthreads();
      {  // per label: the largest a of the tile and its range (rows r0 + 16 i,
         // then the wave's four row groups of the label: lanes 16 and 32 apart)
        double hi = -__builtin_huge_val(), lo = __builtin_huge_val();
        if (cc < CG)
          for (int ss = r0; ss < ns; ss += 16) {
            const double v = sa[ss * 16 + cc];
            hi = fmax(hi, v);
            lo = fmin(lo, v);
          }
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
          hi = fmax(hi, __shfl_xor(hi, off));
          lo = fmin(lo, __shfl_xor(lo, off));
        }
        if ((tid & 63) < 16) {
          pmax[(tid >> 6) * 16 + cc] = hi;
          pmin[(tid >> 6) * 16 + cc] = lo;
        }
      }
      __syncthreads();
      if (tid < 16) {
        double hi = -__builtin_huge_val(), lo = __builtin_huge_val();
        for (int q = 0; q < kDurThreads / 64; ++q) {
          hi = fmax(hi, pmax[q * 16 + tid]);
          lo = fmin(lo, pmin[q * 16 + tid]);
        }
        rho[tid] = hi;
        fast[tid] = (hi - lo <= kDurRange) ? 1 : 0;  // false for non-finite ranges
      }
      __syncthreads();
      // fast labels: the factors, zero past the tile's starts and ends
      // (a batch of rows read before the first exponential)
      if (cc < CG && fast[cc]) {
        const double rc = rho[cc];
        {
          constexpr int NA = kDurW / RS;
          double v[NA];
#pragma unroll
          for (int i = 0; i < NA; ++i) v[i] = sa[(r0 + RS * i) * 16 + cc];
#pragma unroll
          for (int i = 0; i < NA; ++i)
            sa[(r0 + RS * i) * 16 + cc] = r0 + RS * i < ns ? exp_wide(v[i] - rc) : 0.0;
        }
        constexpr int NE = 8;
        for (int e0 = r0; e0 < sbrows; e0 += NE * RS) {
          double v[NE];
#pragma unroll
          for (int i = 0; i < NE; ++i) v[i] = sb[min(e0 + RS * i, sbrows - 1) * 16 + cc];
#pragma unroll
          for (int i = 0; i < NE; ++i)
            if (e0 + RS * i < sbrows) sb[(e0 + RS * i) * 16 + cc] = e0 + RS * i < ne ? exp_wide(v[i] + rc) : 0.0;
        }
      }
      __syncthreads();
      if (!act) continue;
      const int kofs = k0 - klo;  // end index of (s0 + ss, k0 + j): ss + kofs + j
      if (fast[cl]) {
        // blocks of 8 starts x KB lags; the end factors they need, rows
        // ss0 + kofs .. ss0 + kofs + KB + 6, stay in a register window that
        // slides by 8 rows from block to block (8 new reads per block)
        constexpr int NW = KB + 7;
        double W[NW];
#pragma unroll
        for (int q = 0; q < NW; ++q) W[q] = sb[(kofs + q) * 16 + cl];
        for (int ss0 = 0; ss0 < ns; ss0 += 8) {
          double A[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) A[i] = sa[(ss0 + i) * 16 + cl];
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < KB; ++j) acc[j] = fma(A[i], W[i + j], acc[j]);
#pragma unroll
          for (int q = 0; q < NW - 8; ++q) W[q] = W[q + 8];
#pragma unroll
          for (int q = NW - 8; q < NW; ++q) W[q] = sb[(ss0 + 8 + kofs + q) * 16 + cl];
        }
      } else {
        // window w[j] = b[s + k0 + j], index (s - s0) + kofs + j
        double w[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const int ee = kofs + j;
          w[j] = ee < ne ? sb[ee * 16 + cl] : -__builtin_huge_val();
        }
        for (int ss = 0; ss < ns; ++ss) {
          const double av = sa[ss * 16 + cl];
#pragma unroll
          for (int j = 0; j < KB; ++j) acc[j] += exp_wide(av + w[j]);
#pragma unroll
          for (int j = 0; j < KB - 1; ++j) w[j] = w[j + 1];
          const int ee = ss + 1 + kofs + KB - 1;
          w[KB - 1] = ee < ne ? sb[ee * 16 + cl] : -__builtin_huge_val();
        }
      }
    }
  }
  if (act) {
    double *out = pa.dur_part + ((size_t)b * nspan + sp) * K * C;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int k = k0 + j;
      if (k <= khi) {
        const size_t o = (size_t)(k - 1) * C + c;
        const double v = exp((double)pa.dur[o]) * acc[j];
        out[o] = pa.accumulate ? out[o] + v : v;
      }
    }
  }
}

// ------------------------------------------------------------ boundaries
// boundary[b,t] = sum_c E_start[t,c] = P(a segment starts at position t)
// for t < L (1 at t = 0), 0 for t >= L: the boundary uncertainty of the
// abstract of "Streaming Structured Inference with Flash-SemiCRF".  One wave
// per position at a time (grid-stride), lanes over labels; the lanes' sums
// meet by a fixed butterfly, so the result is deterministic.
constexpr int kBndThreads = 256;
__global__ __launch_bounds__(kBndThreads) void k_boundary(ChainShape sh, PostArgs pa) {
  const int lane = threadIdx.x & 63;
  constexpr int wpb = kBndThreads / 64;
  const int Tw = pa.t_hi - pa.t_lo;  // this pass's positions
  const long long npos = (long long)sh.B * Tw;
  const long long nw = (long long)gridDim.x * wpb;
  for (long long q = (long long)blockIdx.x * wpb + (threadIdx.x >> 6); q < npos; q += nw) {
    const int b = (int)(q / Tw), t = pa.t_lo + (int)(q % Tw);
    const int L = pa.lengths[b];
    double s = 0.0;
    if (valid_len(sh, L) && t < L) {  // uniform over the wave
      const double z = shift_f(sh, pa, b, t) + shift_b(sh, pa, b, t) - pa.logz[b];
      const size_t i = rix(sh, pa, b, t);
      for (int c = lane; c < sh.C; c += 64) s += exp(pa.row_u[i + c] + pa.row_v[i + c] + z);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) pa.boundary[(size_t)b * sh.T + t] = (float)s;
  }
}

// ---------------------------------------------------------- centring term
// After the last window of a windowed pass: grad_x[b,t,c] -= w_b mean[b,c]
// for t < L_b (mean = cov_mean, summed over the windows).
__global__ __launch_bounds__(256) void k_mean_fix(ChainShape sh, PostArgs pa) {
  const size_t n = (size_t)sh.B * sh.T * sh.C;
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int c = (int)(i % sh.C);
    const size_t bt = i / sh.C;
    const int t = (int)(bt % sh.T), b = (int)(bt / sh.T);
    const int L = pa.lengths[b];
    if (valid_len(sh, L) && t < L) {
      const double w = pa.grad_logz ? (double)pa.grad_logz[b] : 1.0;
      // the window wrote (float)(w * mu); mu is re-formed from it exactly
      // enough (one float32 rounding) for the 1e-4 absolute bar
      pa.grad_emissions[i] =
          (float)((double)pa.grad_emissions[i] - w * pa.cov_mean[(size_t)b * sh.C + c]);
    }
  }
}

hipError_t launch_mean_fix(const ChainShape &sh, const PostArgs &pa, hipStream_t st) {
  if (!sh.center) return hipSuccess;
  const size_t n = (size_t)sh.B * sh.T * sh.C;
  size_t grid = (n + 255) / 256;
  grid = grid > 8192 ? 8192 : grid;
  hipLaunchKernelGGL(k_mean_fix, dim3((int)grid), dim3(256), 0, st, sh, pa);
  return hipGetLastError();
}

// ------------------------------------------------------------ reductions
// grad_trans = exp(trans) * sum_b w_b sum_seg X;  grad_dur = sum_b w_b sum_span D.
// One workgroup per kRedOut consecutive outputs (transition entries first,
// then durations); thread (o, p) sums slice p of the (sequence, partial)
// list of output o in order, and the slices meet in LDS in a fixed order.
constexpr int kRedOut = 8, kRedSlices = 32;
__global__ __launch_bounds__(kRedOut * kRedSlices) void k_post_reduce(ChainShape sh, PostArgs pa,
                                                                      int nseg, int nspan) {
  __shared__ double red[kRedSlices][kRedOut];
  const int C = sh.C, K = sh.K;
  const int nx = C * C, ng = K * C;
  const int o = threadIdx.x % kRedOut, p = threadIdx.x / kRedOut;
  const int e = blockIdx.x * kRedOut + o;
  const bool tx = e < nx;
  const int np = tx ? nseg : nspan;  // partials per sequence of this output
  const long long n = (long long)sh.B * np;
  const long long per = (n + kRedSlices - 1) / kRedSlices;
  double acc = 0.0;
  if (e < nx + ng) {
    // every load is issued unconditionally (the addresses do not depend on
    // the length), so they pipeline; an invalid sequence's term is dropped
    // by a select (its partial may hold anything)
    const double *src = tx ? pa.tx_part + e : pa.dur_part + (e - nx);
    const size_t stride = tx ? (size_t)nx : (size_t)ng;
    const long long q1 = min(n, (p + 1) * per);
    for (long long q0 = p * per; q0 < q1; q0 += 4) {  // 4 partials' loads at a time
      double v[4], w[4];
      int L[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const long long q = q0 + u < q1 ? q0 + u : q1 - 1;  // clamped: a valid partial
        const int b = (int)(q / np), j = (int)(q % np);
        L[u] = pa.lengths[b];
        w[u] = pa.grad_logz ? (double)pa.grad_logz[b] : 1.0;
        v[u] = src[((size_t)b * np + j) * stride];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (q0 + u < q1) acc += valid_len(sh, L[u]) ? w[u] * v[u] : 0.0;
    }
  }
  red[p][o] = acc;
  __syncthreads();
  if (p == 0 && e < nx + ng) {
    double s = 0.0;
    for (int q = 0; q < kRedSlices; ++q) s += red[q][o];
    if (tx)
      pa.grad_trans[e] = (float)(s * exp((double)pa.trans[e]));
    else
      pa.grad_dur[e - nx] = (float)s;
  }
}

// ------------------------------------------------------------ launch
void post_geometry(const ChainShape &sh, PostGeom &g, int Tw) {
  const int R = kCovThreads / sh.C;
  g.cov_j = kCovJ;
  while (g.cov_j > kCovJMin && (long long)sh.B * ((Tw + R * g.cov_j - 1) / (R * g.cov_j)) < kCovTiles)
    g.cov_j /= 2;
  g.cov_ntile = (Tw + R * g.cov_j - 1) / (R * g.cov_j);
  // Position segments of the transition GEMM and spans of the duration
  // kernel: as long as possible (fewer partials to reduce) while the grid
  // still has about kPostWorkgroups workgroups.
  const int ntc = (sh.C + kTxTile - 1) / kTxTile;
  long long want = (kPostWorkgroups + (long long)ntc * ntc * sh.B - 1) / ((long long)ntc * ntc * sh.B);
  int seg = (int)((Tw + want - 1) / want);
  seg = (seg + kTxRows - 1) / kTxRows * kTxRows;
  g.tx_seg = seg < kTxRows ? kTxRows : (seg > 512 ? 512 : seg);
  g.tx_nseg = (Tw + g.tx_seg - 1) / g.tx_seg;
  const int ncg = (sh.C + 15) / 16, npg = (sh.K + kDurLags - 1) / kDurLags;
  const int ntile = (Tw + kDurW - 1) / kDurW;
  want = (kPostWorkgroups + (long long)ncg * npg * sh.B - 1) / ((long long)ncg * npg * sh.B);
  int span = (int)((ntile + want - 1) / want);
  g.dur_span = span < 1 ? 1 : (span > 8 ? 8 : span);  // tiles of kDurW positions per workgroup
  g.dur_nspan = (Tw + g.dur_span * kDurW - 1) / (g.dur_span * kDurW);
  // lag blocks of KB: the smallest power of two >= 4 with CG x ceil(lags / KB) <= threads
  const int cg = sh.C < 16 ? sh.C : 16;
  const int lags = sh.K < kDurLags ? sh.K : kDurLags;
  g.dur_kb = 4;
  while (g.dur_kb < 32 && cg * ((lags + g.dur_kb - 1) / g.dur_kb) > kDurThreads) g.dur_kb *= 2;
  g.dur_npg = (sh.K + kDurLags - 1) / kDurLags;
  // a, b, partial maxima and minima of a, per-label references and paths
  g.dur_lds = (size_t)(kDurW + kDurW + lags + g.dur_kb + 8) * 16 * 8 + 2 * 64 * 8 + 16 * 8 + 16 * 4;
}

hipError_t launch_posteriors(const ChainShape &sh, const PostArgs &pa, hipStream_t st) {
  PostGeom g;
  post_geometry(sh, g, pa.geom_T);
  const dim3 gc(g.cov_ntile, sh.B);
  switch (g.cov_j) {
    case 4: hipLaunchKernelGGL(k_cov_partial<4>, gc, dim3(kCovThreads), 0, st, sh, pa, g.cov_ntile); break;
    case 8: hipLaunchKernelGGL(k_cov_partial<8>, gc, dim3(kCovThreads), 0, st, sh, pa, g.cov_ntile); break;
    default: hipLaunchKernelGGL(k_cov_partial<16>, gc, dim3(kCovThreads), 0, st, sh, pa, g.cov_ntile); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_cov_anchor, dim3(sh.B, sh.C), dim3(kCovThreads), 0, st, sh, pa,
                     g.cov_ntile);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (g.cov_j) {
    case 4: hipLaunchKernelGGL(k_cov_write<4>, gc, dim3(kCovThreads), 0, st, sh, pa, g.cov_ntile); break;
    case 8: hipLaunchKernelGGL(k_cov_write<8>, gc, dim3(kCovThreads), 0, st, sh, pa, g.cov_ntile); break;
    default: hipLaunchKernelGGL(k_cov_write<16>, gc, dim3(kCovThreads), 0, st, sh, pa, g.cov_ntile); break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ntc = (sh.C + kTxTile - 1) / kTxTile;
  if (sh.C <= 16) {
    hipLaunchKernelGGL(k_trans_x16, dim3(1, sh.B * g.tx_nseg), dim3(kTxThreads), 0, st, sh, pa,
                       g.tx_seg, g.tx_nseg);
  } else if (sh.C > kTxTile) {
    const int n128 = (sh.C + kTx128 - 1) / kTx128;
    hipLaunchKernelGGL(k_trans_x128, dim3(n128 * n128, sh.B * g.tx_nseg), dim3(kTxThreads), 0, st,
                       sh, pa, g.tx_seg, g.tx_nseg);
  } else
    hipLaunchKernelGGL(k_trans_x, dim3(ntc * ntc, sh.B * g.tx_nseg), dim3(kTxThreads), 0, st, sh,
                       pa, g.tx_seg, g.tx_nseg);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ncg = (sh.C + 15) / 16;
  const dim3 gd(ncg * g.dur_npg, sh.B * g.dur_nspan);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void *)k_dur_x<4>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    (void)hipFuncSetAttribute((const void *)k_dur_x<8>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    (void)hipFuncSetAttribute((const void *)k_dur_x<16>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    (void)hipFuncSetAttribute((const void *)k_dur_x<32>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    (void)hipGetLastError();
    attr = true;
  }
  const void *kd = g.dur_kb == 4 ? (const void *)k_dur_x<4>
                   : g.dur_kb == 8 ? (const void *)k_dur_x<8>
                   : g.dur_kb == 16 ? (const void *)k_dur_x<16> : (const void *)k_dur_x<32>;
  if (!lds_fits(kd, g.dur_lds)) return hipErrorInvalidConfiguration;
  if (pa.boundary) {
    long long nb = ((long long)sh.B * (pa.t_hi - pa.t_lo) + (kBndThreads / 64) - 1) / (kBndThreads / 64);
    nb = nb > 2048 ? 2048 : nb;
    hipLaunchKernelGGL(k_boundary, dim3((int)nb), dim3(kBndThreads), 0, st, sh, pa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (g.dur_kb) {
    case 4: hipLaunchKernelGGL(k_dur_x<4>, gd, dim3(kDurThreads), g.dur_lds, st, sh, pa, g.dur_span, g.dur_nspan, g.dur_npg); break;
    case 8: hipLaunchKernelGGL(k_dur_x<8>, gd, dim3(kDurThreads), g.dur_lds, st, sh, pa, g.dur_span, g.dur_nspan, g.dur_npg); break;
    case 16: hipLaunchKernelGGL(k_dur_x<16>, gd, dim3(kDurThreads), g.dur_lds, st, sh, pa, g.dur_span, g.dur_nspan, g.dur_npg); break;
    default: hipLaunchKernelGGL(k_dur_x<32>, gd, dim3(kDurThreads), g.dur_lds, st, sh, pa, g.dur_span, g.dur_nspan, g.dur_npg); break;
  }
  return hipGetLastError();
}

hipError_t launch_post_reduce(const ChainShape &sh, const PostArgs &pa, hipStream_t st) {
  PostGeom g;
  post_geometry(sh, g, pa.geom_T);
  const int ne = sh.C * sh.C + sh.K * sh.C;
  hipLaunchKernelGGL(k_post_reduce, dim3((ne + kRedOut - 1) / kRedOut), dim3(kRedOut * kRedSlices),
                     0, st, sh, pa, g.tx_nseg, g.dur_nspan);
  return hipGetLastError();
}

}  // namespace semicrf
