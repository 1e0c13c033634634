/*
 * semicrf.h -- C ABI of the MI355X (gfx950) semi-CRF hot path.
 *
 * Method: "Streaming Structured Inference with Flash-SemiCRF" (Johnson et
 * al., abstract; technical summary at gist.science/es/paper/2604.18780,
 * section 2.A-2.C).  A semi-CRF scores a labelled segmentation of [0, L) into
 * segments of length 1..K.  With the centring baseline
 *     nu[b,c] = (1/L_b) sum_{t<L_b} x[b,t,c]            (section 2.C)
 * and the cumulative scores
 *     S[b,t,c] = sum_{i<t} (x[b,i,c] - nu[b,c])          (section 2.A)
 * a segment [s, s+k) with label c, preceded by a segment of label c', scores
 *     S[b,s+k,c] - S[b,s,c] + dur[k-1,c] + trans[c',c]
 * (no transition term for the first segment; no start/end scores).  log Z is
 * the log-sum-exp of the total score over every segmentation.  Edge
 * potentials are never materialised: every segment score is read on the fly
 * from S (abstract: "prefix-sum lookup").
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers (HIP), row-major, contiguous,
 *     4-byte aligned (doubles 8-byte aligned); the caller owns every buffer,
 *     including the workspace.  The library allocates, frees and
 *     synchronises nothing and keeps no state between calls; it is reentrant.
 *   - emissions x [B][T][C] float32 (C fastest); lengths [B] int32;
 *     trans [C][C] float32, trans[c'][c] = score of previous label c' -> c;
 *     dur [K][C] float32, dur[k-1][c] = bias of a length-k segment of label c.
 *   - Positions t >= lengths[b] are never read into any result (they may
 *     hold NaN).  A length outside [1, T] makes logz[b] (or best_score[b])
 *     NaN; its gradient rows are zero and it is left out of grad_trans and
 *     grad_dur.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Outputs are overwritten, never accumulated, and must
 *     not alias inputs or each other.
 *   - Host-detectable errors are returned BEFORE anything is launched, so no
 *     output is touched: NULL pointers, sizes < 1, unsupported sizes, a
 *     workspace that is NULL or too small, an invalid checkpoint interval.
 *     A failed launch returns SEMICRF_ERR_HIP (outputs then undefined).
 *   - Non-finite inputs are not checked; they propagate.
 *
 * Supported sizes: 1 <= C <= 256; 1 <= K; K*C <= 16384; K <= 32*floor(512/C)
 * for fwd/bwd and log Z; B*T*C < 2^31.  (The streaming ring of K rows of C
 * float64 values lives in the 160 KB LDS of one compute unit.)
 */
#ifndef SEMICRF_H
#define SEMICRF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SEMICRF_OK = 0,
    SEMICRF_ERR_NULL = 1,        /* a required pointer is NULL */
    SEMICRF_ERR_SHAPE = 2,       /* B, T, C or K < 1, or B*T*C too large */
    SEMICRF_ERR_UNSUPPORTED = 3, /* C or K outside the supported sizes above */
    SEMICRF_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
    SEMICRF_ERR_HIP = 5,         /* a kernel launch failed */
    SEMICRF_ERR_ARG = 6          /* unknown op or flag, negative checkpoint interval */
} semicrf_status_t;

/* operations, for semicrf_workspace_size */
enum {
    SEMICRF_OP_SCAN = 0,    /* semicrf_cumulative_scores */
    SEMICRF_OP_LOGZ = 1,    /* semicrf_logz_fwd */
    SEMICRF_OP_FWD_BWD = 2, /* semicrf_fwd_bwd */
    SEMICRF_OP_VITERBI = 3  /* semicrf_viterbi */
};

/* flags */
enum {
    SEMICRF_NO_CENTER = 1u << 0 /* nu = 0: the textbook, uncentred semi-CRF */
};

/* Human-readable name of a status code (static string, never NULL). */
const char *semicrf_status_string(semicrf_status_t status);

/* Default checkpoint interval: ceil(sqrt(T*K)) positions (technical summary,
 * section 2.C: checkpoints every ~sqrt(TK)). */
int semicrf_default_checkpoint_interval(int T, int K);

/* The checkpoint interval semicrf_logz_fwd and semicrf_fwd_bwd use when
 * given 0: the default above, halved while the sweeps (one workgroup per
 * direction, sequence and interval; every interval is swept concurrently)
 * would have fewer than 256 workgroups, and never below max(2K, 32).
 * Returns 0 for B, T or K < 1. */
int semicrf_checkpoint_interval(int B, int T, int K);

/* Bytes of device workspace `op` needs for these sizes.  checkpoint_interval
 * is the one passed to semicrf_fwd_bwd (0 = default; ignored by other ops).
 * Writes *bytes; returns an error for invalid sizes exactly as the op would. */
semicrf_status_t semicrf_workspace_size(int op, int B, int T, int C, int K, unsigned flags,
                                        int checkpoint_interval, size_t *bytes);

/* Row (a) alone: centring baseline and cumulative scores (abstract:
 * "zero-centered cumulative scores"; technical summary 2.A, 2.C).
 *   nu [B][C] float64 (device), S [B][T+1][C] float64 (device);
 *   S[b,0,:] = 0, S[b,t,:] for t <= L_b as defined above, rows t > L_b repeat
 *   row L_b.  (K is irrelevant here; pass any K >= 1.) */
semicrf_status_t semicrf_cumulative_scores(const float *emissions, const int32_t *lengths,
                                           int B, int T, int C, unsigned flags,
                                           double *nu, double *S,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream);

/* log Z per sequence (abstract: exact inference; forward pass with a K-deep
 * ring, technical summary 2.B).  logz [B] float32 (device). */
semicrf_status_t semicrf_logz_fwd(const float *emissions, const int32_t *lengths,
                                  const float *trans, const float *dur,
                                  int B, int T, int C, int K, unsigned flags,
                                  float *logz, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Forward-backward (abstract: streaming forward-backward with
 * checkpoint-boundary normalisation, exact gradients; technical summary
 * 2.B-2.C).  With F = sum_b w_b log Z_b (w = grad_logz, NULL = all ones):
 *   logz [B] float32            log Z_b
 *   grad_emissions [B][T][C]    dF/dx; with centring this is the exact
 *                               derivative through nu:
 *                               w_b (mu[b,t,c] - (1/L_b) sum_j mu[b,j,c])
 *   grad_trans [C][C]           dF/dtrans  (summed over the batch)
 *   grad_dur [K][C]             dF/ddur    (summed over the batch)
 *   marginals [B][T][C] or NULL coverage mu[b,t,c] = P(position t lies in a
 *                               segment of label c); sums to 1 over c.
 * checkpoint_interval: positions between stored forward/backward states
 * (0 = semicrf_checkpoint_interval(B, T, K)).  Results do not depend on it
 * beyond rounding. */
semicrf_status_t semicrf_fwd_bwd(const float *emissions, const int32_t *lengths,
                                 const float *trans, const float *dur,
                                 int B, int T, int C, int K, unsigned flags,
                                 int checkpoint_interval, const float *grad_logz,
                                 float *logz, float *grad_emissions, float *grad_trans,
                                 float *grad_dur, float *marginals,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* semicrf_fwd_bwd with phase timing: `phase_events` (may be NULL) points to
 * SEMICRF_FWD_BWD_PHASES + 1 hipEvent_t handles created by the caller; event
 * i is recorded on `stream` when phase i is enqueued and the last one after
 * the final phase.  Phases: 0 cumulative scores (3 kernels); 1 the
 * parallel-in-time forward and backward sweeps (one sweep launch per
 * iteration, at most one iteration per checkpoint interval, with their
 * verification, normaliser fix-up and row correction); 2 the posteriors
 * (coverage scan, transition and duration sums: 5 kernels); 3 the
 * parameter-gradient reduction (1 kernel).  Everything else is identical to
 * semicrf_fwd_bwd. */
enum { SEMICRF_FWD_BWD_PHASES = 4 };
semicrf_status_t semicrf_fwd_bwd_timed(const float *emissions, const int32_t *lengths,
                                       const float *trans, const float *dur,
                                       int B, int T, int C, int K, unsigned flags,
                                       int checkpoint_interval, const float *grad_logz,
                                       float *logz, float *grad_emissions, float *grad_trans,
                                       float *grad_dur, float *marginals,
                                       void *workspace, size_t workspace_bytes, void *stream,
                                       void *const *phase_events);

/* Viterbi: the same model in the (max,+) semiring.  The pages give no
 * decoder; this is the maximising segmentation of the scores above.
 * Ties: smallest duration k, then smallest previous label c'; at the end the
 * smallest final label c.
 *   best_score [B] float32; seg_start/seg_len/seg_label [B][T] int32: segment
 *   j of sequence b at index b*T + j for j < num_segs[b], in increasing
 *   start order, remaining slots -1; num_segs [B] int32. */
semicrf_status_t semicrf_viterbi(const float *emissions, const int32_t *lengths,
                                 const float *trans, const float *dur,
                                 int B, int T, int C, int K, unsigned flags,
                                 float *best_score, int32_t *seg_start, int32_t *seg_len,
                                 int32_t *seg_label, int32_t *num_segs,
                                 void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SEMICRF_H */
