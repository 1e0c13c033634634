// internal.h -- shapes, launch configuration and workspace layout shared by
// the host entry points (api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace semicrf {

// Thread roles of one chain workgroup (see chain.hip):
//   K-sum role   thread (c = tid % C, p = tid / C), p < P, owns the A
//                consecutive durations k = p*A+1 .. p*A+A of label c;
//   row role     thread tid < C owns label c (its log reference, outputs);
//   contraction  thread (c = tid % C, q = tid / C), q < QT, sums over the
//                previous labels c' in [CS*q, CS*q+CS).
struct ChainShape {
  int B, T, C, K;
  int NT;      // threads per workgroup (256, 512 or 1024)
  int win;     // 1: windowed engine (C <= 32), 0: LDS-ring engine
  int e64;     // 1: the engine of chain64.hip (32 < C <= 64, K <= 256)
  int e256;    // 1: the engine of chain256.hip (64 < C <= 256, K <= 64)
  int P;       // K-sum threads per label = NT / C
  int A;       // durations per K-sum thread = ceil(K / P)
  int A2;      // windowed engine: far durations per group of helper waves 2.. (A: wave 1)
  int Q;       // waves holding row threads = ceil(C / 64) (Viterbi slices)
  int QT;      // contraction slices of the LDS-ring engine
  int CS;      // previous labels per contraction slice = ceil(C / QT)
  int pf;      // positions per score-prefetch block of the LDS-ring engine (0: none)
  int nload;   // loader waves of the LDS-ring engine
  int burn;    // burn-in positions of a chunk without an exact start (iteration 0)
  int delta;   // checkpoint interval (positions)
  int nchunk;  // ceil(T / delta) chunks per sequence
  int center;  // 1 = subtract the per-label baseline nu
  // Replay (sweep launches with iteration -1): chunks rj0 .. rj0+rnf-1
  // forward and rj0 .. rj0+rnb-1 backward of every sequence, each swept once
  // from its exact checkpoint record, writing rows only (no records).
  int rj0, rnf, rnb;
  // Low-memory fwd+bwd: the posterior pass works in windows of lm_w chunks,
  // each replayed with lm_h more backward chunks (the segments that start in
  // the window end up to K positions past it); 0 when the rows are kept.
  int lm_w, lm_h;
};

constexpr int kMaxC = 256;
constexpr int kMaxPairs = 4;  // (position, label) score pairs per loader lane and block
// Rows per contraction slice in the streamed exp(trans) table (the widest
// slice instance); both directions, QT slices of kTrwRows x C float32 each.
constexpr int kTrwRows = 64;
__host__ __device__ inline size_t trw_floats(int C, int QT) { return (size_t)2 * QT * kTrwRows * C; }
constexpr int kMaxKC = 16384;
constexpr size_t kMaxLds = 163840;  // gfx950: 160 KB per workgroup (static + dynamic)
// Dynamic-LDS budget of the configurations: the hardware limit less a small
// reserve for static LDS (at most 192 bytes, in the sweep engines' repair
// instantiations; lds_fits checks the sum).
constexpr size_t kMaxDynLds = kMaxLds - 256;

// True if a launch of kernel f with `dyn` bytes of dynamic LDS fits the
// per-workgroup LDS together with the kernel's static LDS (queried once per
// kernel; a dispatch over the limit would be rejected by the queue).
inline bool lds_fits(const void *f, size_t dyn) {
  hipFuncAttributes a;
  if (hipFuncGetAttributes(&a, f) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return a.sharedSizeBytes + dyn <= kMaxLds;
}

// Scan tiles: NT_SCAN threads as R = NT_SCAN / C rows x C labels, each row
// thread owning J consecutive positions; a tile covers R*J positions.  J is
// 32, halved (down to 8) while the batch would have fewer than
// kScanWorkgroups tiles: short sequences need the parallelism, long ones
// fewer tiles for the anchor pass.
constexpr int kScanThreads = 256;
constexpr int kScanWorkgroups = 1024;

inline int scan_rows(int C) { return kScanThreads / C; }
inline int scan_j(int B, int T, int C) {
  int j = 32;
  while (j > 8 && (long long)B * ((T + scan_rows(C) * j - 1) / (scan_rows(C) * j)) < kScanWorkgroups)
    j /= 2;
  return j;
}

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Dynamic LDS bytes of one chain workgroup; the carve-up in chain.hip
// follows the same order.  pf: positions per score-prefetch block.
__host__ __device__ inline size_t chain_lds_bytes(int C, int K, int P, int QT, int pf) {
  size_t off = 0;
  off += (size_t)K * C * 8;            // ring
  off += (size_t)P * C * 8;            // K-sum partials
  off = align_up(off, 16);             // the e row is read as 16-byte pairs
  off += (size_t)(C + 64) * 8;         // e row and its zero tail
  off += 8 * 8;                        // scalars
  off += (size_t)QT * C * 8;           // contraction partials
  off += (size_t)2 * (3 * C + 1) * 8;  // row staging (two steps)
  off += (size_t)2 * pf * C * 16;      // split scores (two blocks; mantissas)
  off += (size_t)2 * pf * C * 4;       // split scores (exponents)
  off += (size_t)C * 4;                // rebase shifts
  return align_up(off, 16);
}

// Contraction split of the LDS-ring engine: up to as many slices as there
// are thread rows (NT / C, at most C), each of CS consecutive previous
// labels, CS even (a slice starts on a 16-byte pair of the e row).
__host__ __device__ inline void chain_slices(int C, int NT, int &QT, int &CS) {
  int q = NT / C;
  q = q < 1 ? 1 : (q > C ? C : q);
  CS = (C + q - 1) / q;
  CS += CS & 1;
  QT = (C + CS - 1) / CS;
}

// Viterbi LDS: ring (double), partial maxima (double), partial argmax (int),
// alpha-hat row (double), contraction partial max/arg.
__host__ __device__ inline size_t viterbi_lds_bytes(int C, int K, int P, int Q) {
  size_t off = 0;
  off += (size_t)K * C * 8;
  off += (size_t)P * C * 8;
  off += (size_t)P * C * 4;
  off += (size_t)C * 8;
  off += (size_t)Q * C * 8;
  off += (size_t)Q * C * 4;
  off += 8 * 8;
  return align_up(off, 16);
}

// Checkpoint record of one chain state (float64): [K*C ring][C ref][C o][C m].
// ring[slot][c] = exp(entry(position) - ref[c]) with slot = position mod K;
// o and m are the chain's row outputs at the checkpoint position.
__host__ __device__ inline size_t ck_stride(int C, int K) { return (size_t)(K + 3) * C; }

// Positions per block of the windowed engine (chain_win.hip).
constexpr int kWinU = 4;
// Its ring keeps a second copy of slots [0, kWinMirror) after slot K-1, so
// the far loop reads up to 8 + kWinU - 1 consecutive positions without a
// wrap.
constexpr int kWinMirror = 16;
// Far-part duration chunks (of 8) a helper thread holds in registers.
constexpr int kWinFarChunks = 6;

// LDS bytes of the windowed chain engine (chain_win.hip, 256 threads, same
// order as its carve-up): ring (with its mirror), far-part partials
// [U][groups][C], row staging of two blocks, e row (padded to the
// contraction width 8, 16 or 32), rebase shifts, flags, split scores of two
// blocks.
__host__ __device__ inline size_t win_lds_bytes(int C, int K, int P) {
  const size_t CP = (size_t)(C <= 8 ? 8 : (C <= 16 ? 16 : 32));  // contraction width
  (void)P;
  const int groups = 256 / 64 - 1;  // far-part partials: one per helper wave
  size_t off = 0;
  off += (size_t)(K + kWinMirror) * C * 8;
  off += (size_t)2 * kWinU * groups * C * 8;
  off += (size_t)2 * kWinU * (3 * C + 1) * 8;
  off = align_up(off, 16);
  off += CP * 8;
  off += (size_t)C * 4;
  off += 2 * 4;
  off = align_up(off, 16);
  off += (size_t)2 * kWinU * C * (8 + 8 + 4);
  return align_up(off, 16);
}

// Workspace layout (byte offsets, 256-aligned).
struct Layout {
  size_t S, nu, tile_sum, anchor, logz, logz_bwd;
  size_t ck_fwd, ck_bwd, end_fwd, end_bwd, redo, corr_i, corr_f, nbad, lz_part, shift, pos_shift;
  size_t row_a, row_u, row_v, row_b;
  size_t cov_part, cov_part2, cov_anchor, cov_mean, cov_carry, tx_part, dur_part, trw;
  int row_stride;  // rows per sequence in the row buffers
  size_t bp, vbest, vcbest;
  size_t p_score, p_valid, p_cnt, p_lab;
  size_t v_pred, v_rr, v_re, v_corr, v_delta, v_redo, v_nbad, v_lst_t, v_lst_c, v_mark, v_sub;
  size_t v_node;
  size_t total;
  int ntile;
  int scan_j;   // positions per scan row thread
  int vit_pit;  // Viterbi by the parallel-in-time decoder (vpit.hip)
};

// Arguments of the path score (path.hip).
struct PathArgs {
  const int32_t *lengths;
  const float *trans, *dur, *w;  // w: [B] weights of the gradients (NULL = ones)
  const double *S;
  const int32_t *seg_start, *seg_len, *seg_label, *num_segs;
  float *score;                                 // [B]
  float *grad_x, *grad_trans, *grad_dur;        // each may be NULL
  double *score_ws;                             // [B]
  int *valid;                                   // [B]
  int *cnt;  // [B][C][C] transitions, [B][K][C] durations, [B][C] positions per label
  int32_t *lab;                                 // [B][T] label of each position
};

hipError_t launch_path_score(const ChainShape &sh, const PathArgs &pa, hipStream_t st);

// Arguments of the posterior pass (post.hip).
struct PostArgs {
  const int32_t *lengths;
  const float *trans, *dur, *grad_logz;
  const double *S, *logz;
  const double *row_a, *row_u, *row_v, *row_b;
  const double *pos_shift;  // [2][B][T+1]: add to forward / backward rows at t
  double *cov_part, *cov_part2, *cov_anchor, *cov_mean;  // [B][ntile][C], [B][C]
  double *tx_part;                                       // [B][tx_nseg][C][C]
  double *dur_part;                                      // [B][dur_nspan][K][C]
  float *grad_emissions, *marginals, *grad_trans, *grad_dur;
  float *boundary;  // [B][T] P(a segment starts at t), or NULL
  // The positions of this pass, [t_lo, t_hi) (0, T: all), and the row
  // geometry (as PitBufs: row t at ((b * row_stride) + t - row_t0) * C).
  // pos_shift NULL: the rows are exact (replayed from exact records).
  int t_lo, t_hi, row_t0, row_stride;
  int geom_T;  // positions the launch geometry and partial slots are sized for
  // Windowed passes (positions in several consecutive windows): the
  // partials of every window after the first add to the earlier ones
  // (accumulate), the coverage continues from cov_carry [B][C] (the running
  // sum of all earlier windows, updated in place), cov_mean accumulates, and
  // the emission gradients are written as w * mu with the centring term
  // subtracted after the last window (defer_mean).
  int accumulate, defer_mean;
  double *cov_carry;
};

// Emission gradients minus w_b * mean (the centring term) at t < L_b, after
// the last window of a windowed posterior pass.
hipError_t launch_mean_fix(const ChainShape &sh, const PostArgs &pa, hipStream_t st);

// Launch geometry of the posterior pass (also sizes its workspace).
struct PostGeom {
  int cov_j, cov_ntile, tx_seg, tx_nseg, dur_span, dur_nspan, dur_kb, dur_npg;
  size_t dur_lds;
};

// The cumulative scores [B][T+1][C] the sweeps read (scan.hip).  The sweeps
// form the exp-space split exp(S) = ep * 2^n, exp(-S) = em * 2^-n
// (device_math.h: exp_split) themselves, in the waves that prefetch the
// scores, so no split copy of S is stored.
struct Escaled {
  const double *S;
};

// Buffers of the parallel-in-time sweeps (pit.hip).  Records have the
// checkpoint layout [K*C ring][C integer refs][C o][C m] (float64).
struct PitBufs {
  double *ck_fwd, *ck_bwd;    // chunk start records = checkpoint records [B][nchunk]
  double *end_fwd, *end_bwd;  // chunk end records [B][nchunk]
  int *redo;                  // [2][B][nchunk]: sweep the chunk in the next iteration
  long long *corr_i;          // [2][B][nchunk]: log2 scalar to the predecessor, integer part
  double *corr_f;             // [2][B][nchunk]: its fraction
  int *nbad;                  // [nchunk]: start states replaced by each verification
  double *lz_part;            // [2][B]: log Z in the frame of the chain's last chunk
  double *shift;              // [2][B][nchunk]: log correction of each chunk (fix-up)
  // Per-position rows [B][T+1][C] (float64, NULL when not wanted): forward
  // alpha (t = 1..L) and u (t = 0..L-1), backward v (t = 0..L-1) and beta
  // (t = 1..L); written in each chunk's frame.  Their readers add
  // pos_shift[0][b][t] (forward rows) and pos_shift[1][b][t] (backward rows),
  // the correction of the chunk that wrote position t (k_pit_pos_shift).
  double *row_a, *row_u, *row_v, *row_b;
  // Row geometry: row t of sequence b is at ((b * row_stride) + t - row_t0) * C
  // (row_t0 = 0, row_stride = T + 1 when the rows cover every position; a
  // replay writes a window of positions starting at row_t0).
  int row_t0, row_stride;
  double *pos_shift;          // [2][B][T+1]
  // exp(trans) in float32, [2][C][C] (forward, backward orientation), for the
  // LDS-ring instances that stream their weights (1024 threads); else NULL.
  float *trw;
};

// ---- launchers (scan.hip, chain.hip, chain_win.hip, pit.hip, post.hip,
// viterbi.hip) ------------------------------------------------------------

// ep / em / en may be NULL (then only nu and S are written).
hipError_t launch_scan(const float *x, const int32_t *lengths, int B, int T, int C, int center,
                       double *nu, double *S, double *ep, double *em, int32_t *en,
                       double *tile_sum, double *anchor, int ntile, int J, hipStream_t st);

// One iteration of the chunk-parallel sweeps (every chunk of every sequence,
// both directions when with_bwd); iteration 0 builds the start states.
hipError_t launch_sweep(const ChainShape &sh, const float *trans, const float *dur,
                        const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                        int with_bwd, int iter, hipStream_t st);

// engine for 32 < C <= 64, K <= 256 (chain64.hip); same arguments
bool sweep64_applies(int C, int K);
hipError_t launch_sweep_64(const ChainShape &sh, const float *trans, const float *dur,
                           const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                           int with_bwd, int iter, hipStream_t st);

// engine for 64 < C <= 256, K <= 64 (chain256.hip); same arguments
bool sweep256_applies(int C, int K);
hipError_t launch_sweep_256(const ChainShape &sh, const float *trans, const float *dur,
                            const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                            int with_bwd, int iter, hipStream_t st);

// windowed engine for C <= 32 (chain_win.hip); same arguments
hipError_t launch_sweep_w(const ChainShape &sh, const float *trans, const float *dur,
                          const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                          int with_bwd, int iter, hipStream_t st);

// The whole parallel-in-time sweep: init, nchunk x (sweep, verify), fix-up
// of the records, log Z and (when wanted) the per-position rows.
// after_first (may be NULL) is recorded on st right after the first sweep
// launch (iteration 0, which sweeps every chunk).
hipError_t run_sweeps(const ChainShape &sh, const float *trans, const float *dur,
                      const Escaled &es, const int32_t *lengths, const PitBufs &pb,
                      double *logz_ws, double *logz_bwd_ws, float *logz_out, int with_bwd,
                      hipStream_t st, hipEvent_t after_first = nullptr);

// exp(trans) for the weight-streaming instances (chain.hip).
hipError_t launch_trw(int C, int CS, int QT, const float *trans, float *trw, hipStream_t st);

hipError_t launch_pit_verify(const ChainShape &sh, const int32_t *lengths, const PitBufs &pb,
                             int iter, int with_bwd, hipStream_t st);
hipError_t launch_pit_fixup(const ChainShape &sh, const int32_t *lengths, const PitBufs &pb,
                            double *logz_ws, double *logz_bwd_ws, float *logz_out, int with_bwd,
                            hipStream_t st);
// Tw: positions the posterior pass covers at once (T, or a window's length).
void post_geometry(const ChainShape &sh, PostGeom &g, int Tw);

// Coverage, emission gradients and marginals; transition and duration
// posterior sums (per-block partials) ...
hipError_t launch_posteriors(const ChainShape &sh, const PostArgs &pa, hipStream_t st);
// ... and their fixed-order reduction into grad_trans / grad_dur.
hipError_t launch_post_reduce(const ChainShape &sh, const PostArgs &pa, hipStream_t st);

hipError_t launch_viterbi(const ChainShape &sh, const float *trans, const float *dur,
                          const double *S, const int32_t *lengths, uint32_t *bp, double *vbest,
                          int32_t *vcbest, float *best_out, int32_t *seg_start,
                          int32_t *seg_len, int32_t *seg_label, int32_t *num_segs,
                          hipStream_t st);

// Parallel-in-time Viterbi (vpit.hip).  Threads of a sweep workgroup form
// label groups of NG consecutive lanes: group c owns label c, its lanes
// split the durations (lane g: k = g + 1 + NG*a) and the previous labels
// (c' = g + NG*i) of that label.
struct VShape {
  int B, T, C, K;
  int NT;      // sweep threads (256 or 1024)
  int NG;      // lanes per label group (power of two, 4..64)
  int A;       // durations per lane = ceil(K / NG)
  int CA;      // previous labels per lane = ceil(C / NG)
  int U;       // positions per score-staging block (power of two, 2..min(16, NG))
  int delta;   // positions per sweep chunk
  int nchunk;  // ceil(T / delta)
  int burn;    // burn-in positions of a chunk's first sweep
  int dbt;     // positions per backtrack sub-chunk (>= K)
  int nsub;    // ceil(T / dbt)
  int center;
  // Decisions of the absolute sweep (kAbs): chunks aj0 .. aj0+anj-1 of every
  // sequence; the decision of (t, c) at bp[(b*C + c)*bp_stride + t - bp_t0].
  // The whole sequence: aj0 = 0, anj = nchunk, bp_t0 = 0, bp_stride = T+1;
  // the low-memory decoder sweeps one window of chunks at a time.
  int aj0, anj, bp_t0, bp_stride;
  int lm_w;    // low-memory decoder: chunks per window (0: decisions kept whole)
  // Backtrack range: positions (wp0, wp1] in wsub sub-chunks of dbt, their
  // predecessor words and marks at (t - bp_t0) with stride bp_stride as the
  // decisions, walk lists at (t - wp0) with stride lst_stride.  The whole
  // sequence: wp0 = 0, wp1 = T, wsub = nsub, lst_stride = T.
  int wp0, wp1, wsub, lst_stride;
};

constexpr int kVitIters = 2;     // parallel verification passes before the serial repair
constexpr int kVSubFields = 10;  // int32 fields per backtrack sub-chunk (vpit.hip)

struct VBufs {
  uint32_t *bp;        // [B][C][T+1] decisions at (t, c): k | c' << 16
  uint32_t *pred;      // [B][C][T+1] predecessor of segment end (t, c): k | previous label << 16
  double *rec_r;       // [B][nchunk][C][K] chunk start states (ring slots by position mod K)
  double *rec_e;       // [B][nchunk][C][K] chunk end states
  double *corr;        // [B][nchunk] offset between a chunk's start and its predecessor's end
  double *delta;       // [B][nchunk] accumulated offset of a chunk's frame
  int *redo;           // [B][nchunk]
  int *nbad;           // [kVitIters]
  double *vbest;       // [B]
  int32_t *vcbest;     // [B]
  int32_t *lst_t, *lst_c;  // [B][T] guessed backtrack walks, by sub-chunk
  int32_t *mark;       // [B][T+1] walk index * 512 + label of the node ending at t, or -1
  int32_t *sub;        // [B][nsub][kVSubFields]
  int32_t *node;       // low-memory decoder: [B][3] entry node (t, label) of the next
                       // window's walk (t = -1: not started), segments found so far
};

inline size_t vit_lds_bytes(int C, int K, int U) {
  return (size_t)C * K * 8 + (size_t)2 * C * 8 + (size_t)2 * U * C * 8 + 256;
}
bool vit_config(int B, int T, int C, int K, VShape &vs);
hipError_t launch_vit_pit(const VShape &vs, const float *trans, const float *dur,
                          const double *S, const int32_t *lengths, const VBufs &vb,
                          float *best_out, int32_t *seg_start, int32_t *seg_len,
                          int32_t *seg_label, int32_t *num_segs, hipStream_t st);

}  // namespace semicrf
