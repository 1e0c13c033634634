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

__device__ __forceinline__ size_t rix(const ChainShape &sh, int b, int t) {
  return ((size_t)b * (sh.T + 1) + t) * sh.C;
}

__device__ __forceinline__ bool valid_len(const ChainShape &sh, int L) { return L >= 1 && L <= sh.T; }

}  // namespace

// ------------------------------------------------------------ coverage
// Tiles of R x J positions (R = kCovThreads / C rows of threads, thread
// (r, c) owns J consecutive positions of label c), as in the score scan.
// delta[t,c] = E_start[t,c] - E_end[t,c] (E_end[0] = 0), float64-accurate:
// the coverage is their running sum over the whole sequence.
// The deltas of positions t0 .. t0+J-1 of label c (0 at t >= L).  Every
// load is issued before the first exponential (indices clamped into the
// sequence), so a thread waits for memory once rather than once per
// position.
template <int J>
__device__ __forceinline__ void cov_deltas(const PostArgs &pa, const ChainShape &sh, int b,
                                           int t0, int c, int L, double logZ, double (&d)[J]) {
  double u[J], v[J], a[J], w[J], z[J];
  const double *pf = pa.pos_shift + (size_t)b * (sh.T + 1);
  const double *pg = pf + (size_t)sh.B * (sh.T + 1);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int t = t0 + j < L ? t0 + j : L - 1;
    const size_t i = rix(sh, b, t) + c;
    u[j] = pa.row_u[i];
    v[j] = pa.row_v[i];
    a[j] = pa.row_a[i];
    w[j] = pa.row_b[i];
    z[j] = pf[t] + pg[t] - logZ;  // the rows' chunk corrections, less log Z
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int t = t0 + j;
    double dd = exp(u[j] + v[j] + z[j]);
    if (t >= 1) dd -= exp(a[j] + w[j] + z[j]);
    d[j] = t < L ? dd : 0.0;
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
  double s1 = 0.0, s2 = 0.0;
  const int t0 = tile * R * J + r * J;
  if (r < R && valid_len(sh, L) && t0 < L) {
    double d[J];
    cov_deltas<J>(pa, sh, b, t0, c, L, pa.logz[b], d);
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
    double run = 0.0, tot2 = 0.0;
    for (int q = 0; q < nq; ++q) {
      const double v = red[q];
      red[q] = run;
      run += v;
      tot2 += red2[q];
    }
    pa.cov_mean[(size_t)b * sh.C + c] = valid_len(sh, L) ? tot2 / (double)L : 0.0;
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
  const int t0 = tile * R * J + r * J;
  double d[J];
#pragma unroll
  for (int j = 0; j < J; ++j) d[j] = 0.0;
  if (r < R && ok && t0 < L) cov_deltas<J>(pa, sh, b, t0, c, L, logZ, d);
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
    mean = sh.center ? pa.cov_mean[(size_t)b * C + c] : 0.0;
    w = pa.grad_logz ? (double)pa.grad_logz[b] : 1.0;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int t = t0 + j;
    if (t < sh.T) {
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
// (64 x 64 output tile, sequence, position segment); each thread owns a
// 4 x 4 block of the tile.
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
  const int bi = tid / (kTxTile / 4), bj = tid % (kTxTile / 4);  // 16 x 16 thread grid
  double acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.0;
  int tbeg = 1 + seg * tseg, tend = tbeg + tseg;
  if (!valid_len(sh, L)) tend = tbeg;
  if (tend > L) tend = L;  // transitions at 1 <= t < L
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
      const size_t ri = rix(sh, b, t);
      va[u] = pa.row_a[ri + ca];
      vg[u] = pa.row_v[ri + cg];
      // the rows' chunk corrections (alpha forward, v backward), less log Z
      vz[u] = pa.pos_shift[(size_t)b * (sh.T + 1) + t] +
              pa.pos_shift[((size_t)sh.B + b) * (sh.T + 1) + t] - logZ;
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
    for (int rr = 0; rr < nr; ++rr) {
      double a[4], g[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        a[x] = ta[rr][4 * bi + x];
        g[x] = tg[rr][4 * bj + x];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fma(a[x], g[y], acc[x][y]);
    }
  }
  double *out = pa.tx_part + ((size_t)b * nseg + seg) * C * C;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int cp = ci0 + 4 * bi + x, c = cj0 + 4 * bj + y;
      if (cp < C && c < C) out[(size_t)cp * C + c] = acc[x][y];
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
  const int sbrows = kDurW + min(K, kDurLags) + KB;
  double *sb = sa + (size_t)kDurW * 16;
  double *pmax = sb + (size_t)sbrows * 16;  // [16][16] partial max / min of a
  double *pmin = pmax + 256;
  double *rho = pmin + 256;                      // [16] reference per label
  int *fast = reinterpret_cast<int *>(rho + 16);  // [16]
  double accf[KB], accs[KB], dk[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    accf[j] = 0.0;
    accs[j] = 0.0;
    const int k = k0 + j;
    dk[j] = (act && k <= khi) ? (double)pa.dur[(size_t)(k - 1) * C + c] : 0.0;
  }
  if (valid_len(sh, L)) {
    const double logZ = pa.logz[b];
    const double *Sb = pa.S + (size_t)b * (sh.T + 1) * C;
    const int sbeg = sp * span * kDurW;
    const int send = min(sbeg + span * kDurW, L);  // segment starts s < L
    for (int s0 = sbeg; s0 < send; s0 += kDurW) {
      const int ns = min(kDurW, send - s0);
      // ends e in [s0 + klo, min(s0 + ns - 1 + khi, L)]
      const int ne = min(ns - 1 + khi - klo + 1, L - s0 - klo + 1);
      __syncthreads();
      for (int i = tid; i < ns * CG; i += kDurThreads) {
        const int ss = i / CG, cc = i % CG;
        const size_t ri = rix(sh, b, s0 + ss) + c0 + cc;
        sa[ss * 16 + cc] = (pa.row_u[ri] + pa.pos_shift[(size_t)b * (sh.T + 1) + s0 + ss]) -
                           Sb[(size_t)(s0 + ss) * C + c0 + cc];
      }
      for (int i = tid; i < ne * CG; i += kDurThreads) {
        const int ee = i / CG, cc = i % CG;
        const int e = s0 + klo + ee;
        const size_t ri = rix(sh, b, e) + c0 + cc;
        sb[ee * 16 + cc] = (Sb[(size_t)e * C + c0 + cc] +
                            (pa.row_b[ri] + pa.pos_shift[((size_t)sh.B + b) * (sh.T + 1) + e])) -
                           logZ;
      }
      __syncthreads();
      {  // per label: the largest a of the tile and its range
        const int cc = tid & 15, part = tid >> 4;
        double hi = -__builtin_huge_val(), lo = __builtin_huge_val();
        if (cc < CG)
          for (int ss = part; ss < ns; ss += 16) {
            const double v = sa[ss * 16 + cc];
            hi = fmax(hi, v);
            lo = fmin(lo, v);
          }
        pmax[part * 16 + cc] = hi;
        pmin[part * 16 + cc] = lo;
      }
      __syncthreads();
      if (tid < 16) {
        double hi = -__builtin_huge_val(), lo = __builtin_huge_val();
        for (int q = 0; q < 16; ++q) {
          hi = fmax(hi, pmax[q * 16 + tid]);
          lo = fmin(lo, pmin[q * 16 + tid]);
        }
        rho[tid] = hi;
        fast[tid] = (hi - lo <= kDurRange) ? 1 : 0;  // false for non-finite ranges
      }
      __syncthreads();
      // fast labels: the factors, zero past the tile's starts and ends
      for (int i = tid; i < kDurW * CG; i += kDurThreads) {
        const int ss = i / CG, cc = i % CG;
        if (fast[cc]) sa[ss * 16 + cc] = ss < ns ? exp_wide(sa[ss * 16 + cc] - rho[cc]) : 0.0;
      }
      for (int i = tid; i < sbrows * CG; i += kDurThreads) {
        const int ee = i / CG, cc = i % CG;
        if (fast[cc]) sb[ee * 16 + cc] = ee < ne ? exp_wide(sb[ee * 16 + cc] + rho[cc]) : 0.0;
      }
      __syncthreads();
      if (!act) continue;
      const int kofs = k0 - klo;  // end index of (s0 + ss, k0 + j): ss + kofs + j
      if (fast[cl]) {
        constexpr int JB = KB < 8 ? KB : 8;
        for (int ss0 = 0; ss0 < ns; ss0 += 8) {
          double A[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) A[i] = sa[(ss0 + i) * 16 + cl];
#pragma unroll
          for (int jb = 0; jb < KB; jb += JB) {
            double W[8 + JB - 1];
#pragma unroll
            for (int q = 0; q < 8 + JB - 1; ++q) W[q] = sb[(ss0 + kofs + jb + q) * 16 + cl];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
              for (int j = 0; j < JB; ++j) accf[jb + j] = fma(A[i], W[i + j], accf[jb + j]);
          }
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
          for (int j = 0; j < KB; ++j) accs[j] += exp_wide(av + w[j] + dk[j]);
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
      if (k <= khi) out[(size_t)(k - 1) * C + c] = fma(exp(dk[j]), accf[j], accs[j]);
    }
  }
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
void post_geometry(const ChainShape &sh, PostGeom &g) {
  const int R = kCovThreads / sh.C;
  g.cov_j = kCovJ;
  while (g.cov_j > kCovJMin && (long long)sh.B * ((sh.T + R * g.cov_j - 1) / (R * g.cov_j)) < kCovTiles)
    g.cov_j /= 2;
  g.cov_ntile = (sh.T + R * g.cov_j - 1) / (R * g.cov_j);
  // Position segments of the transition GEMM and spans of the duration
  // kernel: as long as possible (fewer partials to reduce) while the grid
  // still has about kPostWorkgroups workgroups.
  const int ntc = (sh.C + kTxTile - 1) / kTxTile;
  long long want = (kPostWorkgroups + (long long)ntc * ntc * sh.B - 1) / ((long long)ntc * ntc * sh.B);
  int seg = (int)((sh.T + want - 1) / want);
  seg = (seg + kTxRows - 1) / kTxRows * kTxRows;
  g.tx_seg = seg < kTxRows ? kTxRows : (seg > 512 ? 512 : seg);
  g.tx_nseg = (sh.T + g.tx_seg - 1) / g.tx_seg;
  const int ncg = (sh.C + 15) / 16, npg = (sh.K + kDurLags - 1) / kDurLags;
  const int ntile = (sh.T + kDurW - 1) / kDurW;
  want = (kPostWorkgroups + (long long)ncg * npg * sh.B - 1) / ((long long)ncg * npg * sh.B);
  int span = (int)((ntile + want - 1) / want);
  g.dur_span = span < 1 ? 1 : (span > 8 ? 8 : span);  // tiles of kDurW positions per workgroup
  g.dur_nspan = (sh.T + g.dur_span * kDurW - 1) / (g.dur_span * kDurW);
  // lag blocks of KB: the smallest power of two >= 4 with CG x ceil(lags / KB) <= threads
  const int cg = sh.C < 16 ? sh.C : 16;
  const int lags = sh.K < kDurLags ? sh.K : kDurLags;
  g.dur_kb = 4;
  while (g.dur_kb < 32 && cg * ((lags + g.dur_kb - 1) / g.dur_kb) > kDurThreads) g.dur_kb *= 2;
  g.dur_npg = (sh.K + kDurLags - 1) / kDurLags;
  // a, b, partial maxima and minima of a, per-label references and paths
  g.dur_lds = (size_t)(kDurW + kDurW + lags + g.dur_kb) * 16 * 8 + 2 * 256 * 8 + 16 * 8 + 16 * 4;
}

hipError_t launch_posteriors(const ChainShape &sh, const PostArgs &pa, hipStream_t st) {
  PostGeom g;
  post_geometry(sh, g);
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
  post_geometry(sh, g);
  const int ne = sh.C * sh.C + sh.K * sh.C;
  hipLaunchKernelGGL(k_post_reduce, dim3((ne + kRedOut - 1) / kRedOut), dim3(kRedOut * kRedSlices),
                     0, st, sh, pa, g.tx_nseg, g.dur_nspan);
  return hipGetLastError();
}

}  // namespace semicrf
