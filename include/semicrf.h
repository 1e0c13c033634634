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
    SEMICRF_ERR_ARG = 6,         /* unknown op or flag, negative checkpoint interval */
    SEMICRF_ERR_SCRATCH = 7      /* semicrf_fwd_bwd_static: sizes beyond its scratch */
} semicrf_status_t;

/* operations, for semicrf_workspace_size */
enum {
    SEMICRF_OP_SCAN = 0,    /* semicrf_cumulative_scores */
    SEMICRF_OP_LOGZ = 1,    /* semicrf_logz_fwd */
    SEMICRF_OP_FWD_BWD = 2, /* semicrf_fwd_bwd */
    SEMICRF_OP_VITERBI = 3, /* semicrf_viterbi */
    SEMICRF_OP_PATH_SCORE = 4 /* semicrf_path_score */
};

/* flags */
enum {
    SEMICRF_NO_CENTER = 1u << 0,  /* nu = 0: the textbook, uncentred semi-CRF */
    /* semicrf_fwd_bwd / _ex: working memory sublinear in T beyond the
     * cumulative scores (abstract: checkpoint-boundary normalisation keeps
     * working memory sublinear in sequence length; technical summary 2.C:
     * forward messages recomputed between checkpoints).  The sweeps keep only
     * the checkpoint records (default interval ceil(sqrt(T*K)), raised to K
     * when smaller); the posterior pass then replays the intervals window by
     * window from their exact records -- ceil(sqrt(#intervals)) intervals
     * forward, one more backward (the durations reach past the window) --
     * and consumes each window's messages before the next, so they take
     * O(sqrt(T/interval) * interval * C) memory.  Slower (the windows run
     * one after another); same results up to rounding.
     * semicrf_viterbi: the decisions are not kept for every position.  The
     * parallel sweeps keep only each chunk's start state; then, window by
     * window from the end (ceil(sqrt(#chunks)) chunks a window), the
     * decisions of the window and of the chunk before it are recomputed
     * from those states and the optimal path is followed back through the
     * window, one thread per sequence.  Decision memory
     * O(sqrt(T/chunk) * chunk * C) instead of O(T * C); the same
     * segmentation as without the flag.  Slower (the windows run one after
     * another; the walk is serial per sequence).  Shapes the parallel
     * decoder does not take (see semicrf_viterbi) ignore the flag.
     * Ignored by the other operations. */
    SEMICRF_LOW_MEMORY = 1u << 1,
    /* semicrf_logz_fwd / semicrf_fwd_bwd: every sweep in float64.  Without
     * it, shapes with 64 < C <= 256 and K <= 64 run a sweep whose ring
     * entries, K-sums and transition contraction are float32 (integer
     * references, scales, the combination of partial sums and every output
     * stay float64): a relative rounding of about 1e-7 per position, and
     * the parameters must keep 2 |dur| + |trans| below about 60 nats (a
     * larger spread overflows the float32 ring).  The pages fix no
     * precision; this flag selects the float64 engine for those shapes
     * (slower).  Ignored by the other operations. */
    SEMICRF_FLOAT64 = 1u << 2
};

/* Human-readable name of a status code (static string, never NULL). */
const char *semicrf_status_string(semicrf_status_t status);

/* Default checkpoint interval: ceil(sqrt(T*K)) positions (technical summary,
 * section 2.C: checkpoints every ~sqrt(TK)). */
int semicrf_default_checkpoint_interval(int T, int K);

/* The checkpoint interval semicrf_logz_fwd and semicrf_fwd_bwd use when
 * given 0: the default above, halved while the sweeps (one workgroup per
 * direction, sequence and interval; every interval is swept concurrently)
 * would have fewer workgroups than the GPU runs at once -- 256, or 512 for
 * the C <= 16 engine while two of its workgroups fit one compute unit's LDS
 * (C = 16 up to K of about 550) -- and never below max(2K, 32).  Depends on C
 * through the engine.  Returns 0 for B, T, C or K < 1. */
int semicrf_checkpoint_interval(int B, int T, int C, int K);

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
 * 2.B-2.C).  With F = sum_b w_b log Z_b (w = grad_logz [B] float32,
 * contiguous; NULL = all ones):
 *   logz [B] float32            log Z_b
 *   grad_emissions [B][T][C]    dF/dx; with centring this is the exact
 *                               derivative through nu:
 *                               w_b (mu[b,t,c] - (1/L_b) sum_j mu[b,j,c])
 *   grad_trans [C][C]           dF/dtrans  (summed over the batch)
 *   grad_dur [K][C]             dF/ddur    (summed over the batch)
 *   marginals [B][T][C] or NULL coverage mu[b,t,c] = P(position t lies in a
 *                               segment of label c); sums to 1 over c.
 * checkpoint_interval: positions between stored forward/backward states
 * (0 = semicrf_checkpoint_interval(B, T, C, K)).  Results do not depend on it
 * beyond rounding. */
semicrf_status_t semicrf_fwd_bwd(const float *emissions, const int32_t *lengths,
                                 const float *trans, const float *dur,
                                 int B, int T, int C, int K, unsigned flags,
                                 int checkpoint_interval, const float *grad_logz,
                                 float *logz, float *grad_emissions, float *grad_trans,
                                 float *grad_dur, float *marginals,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* semicrf_fwd_bwd with two optional extras.
 *   boundary [B][T] float32 or NULL: P(a segment starts at position t)
 *     = sum_c P(a segment of label c starts at t) -- the uncertainty of the
 *     segment boundaries (abstract: "uncertainty estimates at their
 *     boundaries").  1 at t = 0, 0 at t >= L_b; P(a segment ends at t) is
 *     boundary[b, t] for 0 < t < L_b.
 *   phase_events (may be NULL): SEMICRF_FWD_BWD_PHASES + 1 hipEvent_t handles
 *     created by the caller; event i is recorded on `stream` where phase i
 *     begins and the last one after the final phase.  Phases: 0 cumulative
 *     scores (3 kernels); 1 the first parallel-in-time sweep launch (every
 *     checkpoint interval of both directions); 2 the rest of the sweeps
 *     (verification, further iterations -- no-ops once converged --,
 *     normaliser fix-up, record and row corrections); 3 the posteriors
 *     (coverage scan, boundaries, transition and duration sums); 4 the
 *     parameter-gradient reduction.
 * Everything else is identical to semicrf_fwd_bwd. */
enum { SEMICRF_FWD_BWD_PHASES = 5 };
semicrf_status_t semicrf_fwd_bwd_ex(const float *emissions, const int32_t *lengths,
                                    const float *trans, const float *dur,
                                    int B, int T, int C, int K, unsigned flags,
                                    int checkpoint_interval, const float *grad_logz,
                                    float *logz, float *grad_emissions, float *grad_trans,
                                    float *grad_dur, float *marginals, float *boundary,
                                    void *workspace, size_t workspace_bytes, void *stream,
                                    void *const *phase_events);

/* semicrf_fwd_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The workspace is a static
 * device array of 64 MiB inside the library (SEMICRF_STATIC_SCRATCH_BYTES),
 * which every GPU the library runs on holds until the process ends; its
 * address is looked up once per device on the first call with that device
 * current.  Sizes whose workspace (semicrf_workspace_size with op
 * SEMICRF_OP_FWD_BWD) exceeds it return SEMICRF_ERR_SCRATCH before
 * anything is launched (e.g. the NLP shape B=32 T=512 C=24 K=32 fits,
 * T = 4096 with C = 256 does not).  The call allocates nothing: no
 * hipMalloc, no hipFree, no allocating library routine.
 * All calls on one GPU share its array and it keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on
 * one GPU -- concurrent streams or threads -- race and must be serialised
 * by the caller.  Everything else is identical to semicrf_fwd_bwd. */
enum { SEMICRF_STATIC_SCRATCH_BYTES = 64 << 20 };
semicrf_status_t semicrf_fwd_bwd_static(const float *emissions, const int32_t *lengths,
                                        const float *trans, const float *dur,
                                        int B, int T, int C, int K, unsigned flags,
                                        int checkpoint_interval, const float *grad_logz,
                                        float *logz, float *grad_emissions, float *grad_trans,
                                        float *grad_dur, float *marginals, void *stream);

/* Score of a given labelled segmentation under the same model, and its
 * gradients: the second term of the training loss log Z - score(gold)
 * (technical summary, section 3: training on labelled segmentations).
 *   score_b = sum_j (S[b, s_j + k_j, c_j] - S[b, s_j, c_j] + dur[k_j - 1, c_j])
 *           + sum_{j >= 1} trans[c_{j-1}, c_j]
 * Segments in the Viterbi output layout: seg_start / seg_len / seg_label
 * [B][T] int32, segment j of sequence b at index b*T + j for j < num_segs[b]
 * (entries past num_segs[b] are not read).  A segmentation is valid when
 * 1 <= num_segs[b] <= L_b, s_0 = 0, each segment starts where the previous
 * one ends, 1 <= k_j <= K, 0 <= c_j < C and the last one ends at L_b; an
 * invalid one (or a length outside [1, T]) gives score NaN, zero gradient
 * rows, and no share of grad_trans / grad_dur.
 * Gradients of F = sum_b w_b score_b (weights [B] or NULL = all ones), each
 * output optional (NULL skips it):
 *   grad_emissions [B][T][C]: w_b (1[position t has label c] - n_bc / L_b)
 *     with centring (n_bc = positions of label c), the indicator without;
 *     0 at t >= L_b;
 *   grad_trans [C][C]: sum_b w_b #(consecutive segments c' -> c);
 *   grad_dur [K][C]: sum_b w_b #(segments of length k and label c).
 * score [B] float32 (required).  The workspace is
 * semicrf_workspace_size(SEMICRF_OP_PATH_SCORE, ...). */
semicrf_status_t semicrf_path_score(const float *emissions, const int32_t *lengths,
                                    const float *trans, const float *dur,
                                    int B, int T, int C, int K, unsigned flags,
                                    const int32_t *seg_start, const int32_t *seg_len,
                                    const int32_t *seg_label, const int32_t *num_segs,
                                    const float *weights, float *score,
                                    float *grad_emissions, float *grad_trans, float *grad_dur,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Viterbi: the same model in the (max,+) semiring.  The pages give no
 * decoder; this is the maximising segmentation of the scores above.
 * Ties: segmentations that only reorder segment lengths inside a run of one
 * label score the same in exact arithmetic, so the recursion compares in
 * float64 with a tolerance: a candidate within 1e-11 * (|max| + 1) of the
 * maximum at a decision ties with it (at |max| ~ 5e6 candidates up to ~5e-5
 * apart tie).  Among tied candidates the smallest duration k wins, then the
 * smallest previous label c'; at the end the smallest final label c among
 * the tied final scores.
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
