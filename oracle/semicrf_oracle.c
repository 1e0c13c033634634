/*
 * semicrf_oracle.c -- plain float64 CPU semi-CRF: log-partition, gradients,
 * coverage marginals and Viterbi.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this code.  It shares no code,
 * header, table or helper with the HIP library and includes nothing from it.
 *
 * Source of the method: "Streaming Structured Inference with Flash-SemiCRF"
 * (Johnson et al.), as summarised on the pages
 *   - abstract (mlsanity.com/paper/2604.18780): segment scores read from a
 *     prefix-sum array; zero-centred cumulative scores; exact gradients;
 *   - gist.science/es/paper/2604.18780, "Resumen Tecnico" section 2.A: the score
 *     of segment [s, s+k) is the difference of two cumulative-score entries;
 *     section 2.C: a per-sequence, per-label emission baseline nu_{b,c} is
 *     subtracted before the prefix sum.
 * The pages give no recursions.  This file writes out the plain definition:
 *
 *   nu[c]     = (1/L) sum_{t<L} x[t,c]              (0 when centring is off)
 *   S[t,c]    = sum_{i<t} (x[i,c] - nu[c])          t = 0..L
 *   score(seg [s,s+k), label c) = S[s+k,c] - S[s,c] + dur[k-1,c]
 *   a segmentation of [0,L) is a sequence of such segments with 1<=k<=K;
 *   consecutive segments with labels c', c add trans[c',c]; the first
 *   segment has no transition term, and there are no start/end scores.
 *   log Z = log sum over all segmentations of exp(total score).
 *
 * log Z is evaluated by the textbook dynamic programme over segment end
 * points, kept as full (T+1) x C float64 tables -- no ring buffer, no
 * checkpointing:
 *   u[0,c] = 0;  alpha[t,c] = LSE_{k=1..min(K,t)} (u[t-k,c] + S[t,c]-S[t-k,c] + dur[k-1,c])
 *   u[t,c] = LSE_{c'} (alpha[t,c'] + trans[c',c])          1 <= t < L
 *   log Z = LSE_c alpha[L,c]
 * and its mirror image from the right:
 *   beta[L,c] = 0;  v[t,c] = LSE_{k=1..min(K,L-t)} (S[t+k,c]-S[t,c] + dur[k-1,c] + beta[t+k,c])
 *   beta[t,c'] = LSE_c (trans[c',c] + v[t,c])               1 <= t < L
 * The log values grow roughly linearly with t (log Z reaches ~5e6 at a
 * million positions), and a float64 number that large carries only ~1e-9
 * absolute precision, which every step of the recursion would add to.  So
 * each table row t stores its values minus an exact integer offset (zf[t]
 * forward, zb[t] backward: the previous row's offset plus the floor of the
 * new row's maximum), and the integers are combined exactly before the small
 * parts are added: log Z = zf[L] + LSE_c (alpha[L,c] - zf[L]), and every
 * posterior exponent below is (zf[s] + zb[e] - zf[L]) plus small terms.  In
 * exact arithmetic this is the same programme.
 * Posteriors follow from the definition of a marginal:
 *   P(segment s,k,c) = exp(u[s,c] + S[s+k,c]-S[s,c] + dur[k-1,c] + beta[s+k,c] - log Z)
 *   P(transition c'->c at boundary t) = exp(alpha[t,c'] + trans[c',c] + v[t,c] - log Z)
 *   coverage mu[i,c] = sum of P(segment) over the segments of label c that
 *                      contain position i (accumulated with a difference array)
 *   boundary   P(a segment starts at s) = sum over every segment (s, k, c)
 *              that starts at s of P(segment)  (the boundary uncertainty of
 *              the abstract)
 * and the gradients of F = sum_b w_b log Z_b are
 *   dF/d dur[k-1,c]    = sum_b w_b sum_s P(s,k,c)
 *   dF/d trans[c',c]   = sum_b w_b sum_t P(t,c'->c)
 *   dF/d x[b,i,c]      = w_b (mu[i,c] - (1/L) sum_j mu[j,c])   (centred: nu depends on x)
 *                      = w_b mu[i,c]                          (centring off)
 * Viterbi is the same programme in the (max,+) semiring.  Segmentations that
 * differ only in the order of segment lengths inside a run of one label score
 * exactly the same in real arithmetic, so ties are structural; in floating
 * point such tied candidates differ by rounding only.  A candidate therefore
 * ties with the maximum when it lies within eps = 1e-11 * (|max| + 1) of it;
 * among tied candidates the smallest duration k wins, then the smallest
 * previous label c', and at the end the smallest final label c.  The stored
 * programme value is the maximum itself.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py
 * (brute-force enumeration, K=1 linear-chain reduction, closed forms,
 * invariances, finite differences).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_NEG_INF (-INFINITY)

/* ---------------------------------------------------------------- helpers */

/* log(sum_i exp(v_i)) over n values, max-shifted; -inf when all are -inf. */
static double lse_array(const double *v, int n)
{
    double m = ORACLE_NEG_INF;
    for (int i = 0; i < n; ++i)
        if (v[i] > m) m = v[i];
    if (m == ORACLE_NEG_INF) return ORACLE_NEG_INF;
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += exp(v[i] - m);
    return m + log(s);
}

/* tie tolerance of the Viterbi decisions (see the file header) */
static double tie_eps(double best)
{
    return 1e-11 * (fabs(best) + 1.0);
}

static int pick_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* nu and S for one sequence (x is [T][C], S is [T+1][C]).  Rows t > L are
 * copies of row L; they are never read by any result. */
static void prefix_one(int T, int C, int L, const float *x, int center,
                       double *nu, double *S)
{
    for (int c = 0; c < C; ++c) {
        double sum = 0.0;
        for (int t = 0; t < L; ++t) sum += (double)x[(size_t)t * C + c];
        nu[c] = center ? sum / (double)L : 0.0;
    }
    for (int c = 0; c < C; ++c) S[c] = 0.0;
    for (int t = 0; t < L; ++t)
        for (int c = 0; c < C; ++c)
            S[(size_t)(t + 1) * C + c] =
                S[(size_t)t * C + c] + ((double)x[(size_t)t * C + c] - nu[c]);
    for (int t = L + 1; t <= T; ++t)
        for (int c = 0; c < C; ++c)
            S[(size_t)t * C + c] = S[(size_t)L * C + c];
}

/* ------------------------------------------------------ per-sequence tables */

typedef struct {
    double *S, *alpha, *u, *v, *beta, *zf, *zb, *tmp;
} tables_t;

static int tables_alloc(tables_t *tb, int T, int C, int K, int nth)
{
    size_t n = (size_t)(T + 1) * C;
    size_t ntmp = (size_t)nth * (size_t)(K > C ? K : C);
    tb->S = malloc(n * sizeof(double));
    tb->alpha = malloc(n * sizeof(double));
    tb->u = malloc(n * sizeof(double));
    tb->v = malloc(n * sizeof(double));
    tb->beta = malloc(n * sizeof(double));
    tb->zf = malloc((size_t)(T + 1) * sizeof(double));
    tb->zb = malloc((size_t)(T + 1) * sizeof(double));
    tb->tmp = malloc(ntmp * sizeof(double));
    return tb->S && tb->alpha && tb->u && tb->v && tb->beta && tb->zf && tb->zb && tb->tmp;
}

static void tables_free(tables_t *tb)
{
    free(tb->S); free(tb->alpha); free(tb->u); free(tb->v); free(tb->beta);
    free(tb->zf); free(tb->zb); free(tb->tmp);
}

/* Largest value of a row (-inf when all are -inf). */
static double row_max(const double *v, int n)
{
    double m = ORACLE_NEG_INF;
    for (int i = 0; i < n; ++i)
        if (v[i] > m) m = v[i];
    return m;
}

/* Forward table: alpha[t,c] for t=1..L, u[t,c] for t=0..L-1, each stored
 * minus the integer offset zf[t].  Returns LSE_c (alpha[L,c] - zf[L]); log Z
 * is zf[L] plus that. */
static double forward_one(int L, int C, int K, const double *S, const double *tr,
                          const double *du, double *alpha, double *u, double *zf, double *tmp,
                          int nth)
{
    for (int c = 0; c < C; ++c) { u[c] = 0.0; alpha[c] = ORACLE_NEG_INF; }
    zf[0] = 0.0;
#pragma omp parallel num_threads(nth) if (nth > 1)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *buf = tmp + (size_t)tid * (size_t)(K > C ? K : C);
        for (int t = 1; t <= L; ++t) {
            int kmax = t < K ? t : K;
            /* alpha[t,c] relative to zf[t-1] */
#pragma omp for schedule(static)
            for (int c = 0; c < C; ++c) {
                for (int k = 1; k <= kmax; ++k)
                    buf[k - 1] = u[(size_t)(t - k) * C + c] + (zf[t - k] - zf[t - 1])
                               + (S[(size_t)t * C + c] - S[(size_t)(t - k) * C + c])
                               + du[(size_t)(k - 1) * C + c];
                alpha[(size_t)t * C + c] = lse_array(buf, kmax);
            }
#pragma omp single
            {
                double n = floor(row_max(alpha + (size_t)t * C, C));
                zf[t] = zf[t - 1] + n;
                for (int c = 0; c < C; ++c) alpha[(size_t)t * C + c] -= n;
            }
            if (t < L) {
#pragma omp for schedule(static)
                for (int c = 0; c < C; ++c) {
                    for (int cp = 0; cp < C; ++cp)
                        buf[cp] = alpha[(size_t)t * C + cp] + tr[(size_t)cp * C + c];
                    u[(size_t)t * C + c] = lse_array(buf, C);
                }
            }
        }
    }
    return lse_array(alpha + (size_t)L * C, C);
}

/* Backward table: v[t,c] for t=0..L-1, beta[t,c] for t=1..L, each stored
 * minus the integer offset zb[t].  Returns LSE_c (v[0,c] - zb[0]); the
 * right-to-left log Z is zb[0] plus that. */
static double backward_one(int L, int C, int K, const double *S, const double *tr,
                           const double *du, double *v, double *beta, double *zb, double *tmp,
                           int nth)
{
    for (int c = 0; c < C; ++c) beta[(size_t)L * C + c] = 0.0;
    zb[L] = 0.0;
#pragma omp parallel num_threads(nth) if (nth > 1)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *buf = tmp + (size_t)tid * (size_t)(K > C ? K : C);
        for (int t = L - 1; t >= 0; --t) {
            int kmax = (L - t) < K ? (L - t) : K;
            /* v[t,c] relative to zb[t+1] */
#pragma omp for schedule(static)
            for (int c = 0; c < C; ++c) {
                for (int k = 1; k <= kmax; ++k)
                    buf[k - 1] = (S[(size_t)(t + k) * C + c] - S[(size_t)t * C + c])
                               + du[(size_t)(k - 1) * C + c]
                               + beta[(size_t)(t + k) * C + c] + (zb[t + k] - zb[t + 1]);
                v[(size_t)t * C + c] = lse_array(buf, kmax);
            }
#pragma omp single
            {
                double n = floor(row_max(v + (size_t)t * C, C));
                zb[t] = zb[t + 1] + n;
                for (int c = 0; c < C; ++c) v[(size_t)t * C + c] -= n;
            }
            if (t >= 1) {
#pragma omp for schedule(static)
                for (int cp = 0; cp < C; ++cp) {
                    for (int c = 0; c < C; ++c)
                        buf[c] = tr[(size_t)cp * C + c] + v[(size_t)t * C + c];
                    beta[(size_t)t * C + cp] = lse_array(buf, C);
                }
            }
        }
    }
    return lse_array(v, C);
}

/* Posteriors of one sequence.  Adds w * (its contribution) into gtrans/gdur
 * (local per-sequence buffers supplied by the caller) and writes mu / grad_x
 * rows [0,T) (zeros at t >= L).  Each label's sums are taken in arrays of
 * that label alone (one thread per label) and stored once at the end, so no
 * two threads write the same cache line while they add; every sum adds the
 * same terms in the same order as the formulas state. */
static void posteriors_one(int T, int L, int C, int K, int center, double w, double lzs,
                           const double *S, const double *tr, const double *du,
                           const double *alpha, const double *u, const double *v,
                           const double *beta, const double *zf, const double *zb,
                           double *gtrans, double *gdur, double *mu_out, double *gx_out,
                           double *bnd_out, int nth)
{
    double *start = bnd_out ? calloc((size_t)T * C, sizeof(double)) : NULL;
#pragma omp parallel for num_threads(nth) if (nth > 1) schedule(static)
    for (int c = 0; c < C; ++c) {
        double *diff = calloc((size_t)T + 1, sizeof(double)); /* difference array of mu[., c] */
        double *mu = calloc((size_t)T, sizeof(double));
        double *st = start ? calloc((size_t)T, sizeof(double)) : NULL;
        double *gd = calloc((size_t)K, sizeof(double));
        double *gt = calloc((size_t)C, sizeof(double));
        /* every segment (s, k, c) */
        for (int s = 0; s < L; ++s) {
            int kmax = (L - s) < K ? (L - s) : K;
            for (int k = 1; k <= kmax; ++k) {
                double lp = u[(size_t)s * C + c]
                          + (S[(size_t)(s + k) * C + c] - S[(size_t)s * C + c])
                          + du[(size_t)(k - 1) * C + c]
                          + beta[(size_t)(s + k) * C + c]
                          + ((zf[s] + zb[s + k] - zf[L]) - lzs);
                double p = exp(lp);
                gd[k - 1] += w * p;
                if (st) st[s] += p;
                diff[s] += p;
                diff[s + k] -= p;
            }
        }
        double run = 0.0;
        for (int i = 0; i < L; ++i) {
            run += diff[i];
            mu[i] = run;
        }
        /* every transition c' -> c at an interior boundary t */
        for (int t = 1; t < L; ++t)
            for (int cp = 0; cp < C; ++cp) {
                double lp = alpha[(size_t)t * C + cp] + tr[(size_t)cp * C + c]
                          + v[(size_t)t * C + c] + ((zf[t] + zb[t] - zf[L]) - lzs);
                gt[cp] += w * exp(lp);
            }
        double mean = 0.0;
        if (center) {
            for (int i = 0; i < L; ++i) mean += mu[i];
            mean /= (double)L;
        }
        for (int i = 0; i < T; ++i) {
            double m = i < L ? mu[i] : 0.0;
            if (mu_out) mu_out[(size_t)i * C + c] = m;
            if (gx_out) gx_out[(size_t)i * C + c] = i < L ? w * (m - mean) : 0.0;
            if (st) start[(size_t)i * C + c] = st[i];
        }
        if (gdur)
            for (int k = 0; k < K; ++k) gdur[(size_t)k * C + c] += gd[k];
        if (gtrans)
            for (int cp = 0; cp < C; ++cp) gtrans[(size_t)cp * C + c] += gt[cp];
        free(diff);
        free(mu);
        free(st);
        free(gd);
        free(gt);
    }
    if (bnd_out) {
        for (int s = 0; s < T; ++s) {
            double b = 0.0;
            if (s < L)
                for (int c = 0; c < C; ++c) b += start[(size_t)s * C + c];
            bnd_out[s] = b;
        }
    }
    free(start);
}

/* --------------------------------------------------------------- public API */

/* Centring baseline nu [B][C] and cumulative scores S [B][T+1][C]. */
int oracle_prefix(int B, int T, int C, const float *x, const int32_t *lengths, int center,
                  double *nu, double *S)
{
    for (int b = 0; b < B; ++b) {
        int L = lengths[b];
        if (L < 1 || L > T) return 2;
        prefix_one(T, C, L, x + (size_t)b * T * C, center, nu + (size_t)b * C,
                   S + (size_t)b * (T + 1) * C);
    }
    return 0;
}

/* Full forward-backward.  Output pointers other than logz may be NULL.
 * logz_bwd (optional) receives the right-to-left log Z for consistency checks;
 * boundary (optional, [B][T]) the probability that a segment starts at t. */
int oracle_fwd_bwd(int B, int T, int C, int K, const float *x, const int32_t *lengths,
                   const float *trans, const float *dur, int center, const double *w,
                   double *logz, double *logz_bwd, double *grad_x, double *grad_trans,
                   double *grad_dur, double *marginals, double *boundary, int nthreads)
{
    if (B < 1 || T < 1 || C < 1 || K < 1) return 2;
    int nth = pick_threads(nthreads);
    double *tr = malloc((size_t)C * C * sizeof(double));
    double *du = malloc((size_t)K * C * sizeof(double));
    for (size_t i = 0; i < (size_t)C * C; ++i) tr[i] = trans[i];
    for (size_t i = 0; i < (size_t)K * C; ++i) du[i] = dur[i];
    int want_post = grad_x || grad_trans || grad_dur || marginals || boundary;
    /* per-sequence parameter-gradient buffers, summed in sequence order */
    double *gt_all = want_post ? calloc((size_t)B * C * C, sizeof(double)) : NULL;
    double *gd_all = want_post ? calloc((size_t)B * K * C, sizeof(double)) : NULL;

    int outer = (B >= nth && nth > 1) ? nth : 1;
    int inner = outer > 1 ? 1 : nth;
    int rc = 0;
#pragma omp parallel for num_threads(outer) if (outer > 1) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int L = lengths[b];
        const float *xb = x + (size_t)b * T * C;
        double wb = w ? w[b] : 1.0;
        if (L < 1 || L > T) {
            logz[b] = NAN;
            if (logz_bwd) logz_bwd[b] = NAN;
            for (size_t i = 0; i < (size_t)T * C; ++i) {
                if (grad_x) grad_x[(size_t)b * T * C + i] = 0.0;
                if (marginals) marginals[(size_t)b * T * C + i] = 0.0;
            }
            if (boundary)
                for (int i = 0; i < T; ++i) boundary[(size_t)b * T + i] = 0.0;
            continue;
        }
        tables_t tb;
        if (!tables_alloc(&tb, T, C, K, inner)) {
            rc = 3;
            continue;
        }
        double *nu = malloc((size_t)C * sizeof(double));
        prefix_one(T, C, L, xb, center, nu, tb.S);
        double lzs = forward_one(L, C, K, tb.S, tr, du, tb.alpha, tb.u, tb.zf, tb.tmp, inner);
        logz[b] = tb.zf[L] + lzs;
        if (want_post || logz_bwd) {
            double lzb = backward_one(L, C, K, tb.S, tr, du, tb.v, tb.beta, tb.zb, tb.tmp, inner);
            if (logz_bwd) logz_bwd[b] = tb.zb[0] + lzb;
        }
        if (want_post)
            posteriors_one(T, L, C, K, center, wb, lzs, tb.S, tr, du, tb.alpha, tb.u, tb.v,
                           tb.beta, tb.zf, tb.zb, gt_all + (size_t)b * C * C,
                           gd_all + (size_t)b * K * C,
                           marginals ? marginals + (size_t)b * T * C : NULL,
                           grad_x ? grad_x + (size_t)b * T * C : NULL,
                           boundary ? boundary + (size_t)b * T : NULL, inner);
        free(nu);
        tables_free(&tb);
    }
    if (want_post) {
        if (grad_trans) {
            memset(grad_trans, 0, (size_t)C * C * sizeof(double));
            for (int b = 0; b < B; ++b)
                for (size_t i = 0; i < (size_t)C * C; ++i) grad_trans[i] += gt_all[(size_t)b * C * C + i];
        }
        if (grad_dur) {
            memset(grad_dur, 0, (size_t)K * C * sizeof(double));
            for (int b = 0; b < B; ++b)
                for (size_t i = 0; i < (size_t)K * C; ++i) grad_dur[i] += gd_all[(size_t)b * K * C + i];
        }
    }
    free(gt_all); free(gd_all); free(tr); free(du);
    return rc;
}

/* Viterbi (max,+) decoding.  Segments of sequence b are written at
 * [b*T + j] for j < num_segs[b]; remaining slots are set to -1.
 * min_margin (optional): over the decisions on the returned path, the
 * smallest gap between the maximum and the best candidate outside its tie
 * set (+inf when every candidate tied). */
int oracle_viterbi(int B, int T, int C, int K, const float *x, const int32_t *lengths,
                   const float *trans, const float *dur, int center, double *best_score,
                   int32_t *seg_start, int32_t *seg_len, int32_t *seg_label,
                   int32_t *num_segs, double *min_margin, int nthreads)
{
    if (B < 1 || T < 1 || C < 1 || K < 1) return 2;
    int nth = pick_threads(nthreads);
    int rc = 0;
#pragma omp parallel for num_threads(nth) if (nth > 1 && B > 1) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int L = lengths[b];
        for (int j = 0; j < T; ++j) {
            seg_start[(size_t)b * T + j] = -1;
            seg_len[(size_t)b * T + j] = -1;
            seg_label[(size_t)b * T + j] = -1;
        }
        if (L < 1 || L > T) {
            best_score[b] = NAN;
            num_segs[b] = 0;
            if (min_margin) min_margin[b] = NAN;
            continue;
        }
        size_t n = (size_t)(T + 1) * C;
        double *S = malloc(n * sizeof(double));
        double *nu = malloc((size_t)C * sizeof(double));
        double *ah = malloc(n * sizeof(double));
        double *uh = malloc(n * sizeof(double));
        int32_t *bk = malloc(n * sizeof(int32_t));
        int32_t *bc = malloc(n * sizeof(int32_t));
        double *mk = malloc(n * sizeof(double)); /* margin of the k decision at (t,c) */
        double *mc = malloc(n * sizeof(double)); /* margin of the c' decision at (t,c) */
        if (!S || !nu || !ah || !uh || !bk || !bc || !mk || !mc) {
            rc = 3;
            continue;
        }
        prefix_one(T, C, L, x + (size_t)b * T * C, center, nu, S);
        for (int c = 0; c < C; ++c) { uh[c] = 0.0; bc[c] = -1; mc[c] = INFINITY; }
        for (int t = 1; t <= L; ++t) {
            int kmax = t < K ? t : K;
            for (int c = 0; c < C; ++c) {
                double best = ORACLE_NEG_INF;
                for (int k = 1; k <= kmax; ++k) {
                    double val = ((S[(size_t)t * C + c] - S[(size_t)(t - k) * C + c])
                                  + (double)dur[(size_t)(k - 1) * C + c])
                               + uh[(size_t)(t - k) * C + c];
                    if (val > best) best = val;
                }
                double eps = tie_eps(best), outside = ORACLE_NEG_INF;
                int arg = 0;
                for (int k = 1; k <= kmax; ++k) {
                    double val = ((S[(size_t)t * C + c] - S[(size_t)(t - k) * C + c])
                                  + (double)dur[(size_t)(k - 1) * C + c])
                               + uh[(size_t)(t - k) * C + c];
                    if (val >= best - eps) { if (arg == 0) arg = k; }
                    else if (val > outside) outside = val;
                }
                ah[(size_t)t * C + c] = best;
                bk[(size_t)t * C + c] = arg;
                mk[(size_t)t * C + c] = best - outside;
            }
            if (t < L) {
                for (int c = 0; c < C; ++c) {
                    double best = ORACLE_NEG_INF;
                    for (int cp = 0; cp < C; ++cp) {
                        double val = ah[(size_t)t * C + cp] + (double)trans[(size_t)cp * C + c];
                        if (val > best) best = val;
                    }
                    double eps = tie_eps(best), outside = ORACLE_NEG_INF;
                    int arg = -1;
                    for (int cp = 0; cp < C; ++cp) {
                        double val = ah[(size_t)t * C + cp] + (double)trans[(size_t)cp * C + c];
                        if (val >= best - eps) { if (arg < 0) arg = cp; }
                        else if (val > outside) outside = val;
                    }
                    uh[(size_t)t * C + c] = best;
                    bc[(size_t)t * C + c] = arg;
                    mc[(size_t)t * C + c] = best - outside;
                }
            }
        }
        double best = ORACLE_NEG_INF, outside = ORACLE_NEG_INF;
        for (int c = 0; c < C; ++c)
            if (ah[(size_t)L * C + c] > best) best = ah[(size_t)L * C + c];
        int cbest = -1;
        for (int c = 0; c < C; ++c) {
            double val = ah[(size_t)L * C + c];
            if (val >= best - tie_eps(best)) { if (cbest < 0) cbest = c; }
            else if (val > outside) outside = val;
        }
        best_score[b] = best;
        double margin = best - outside;
        /* backtrack, then reverse into the output slots */
        int nseg = 0;
        int t = L, c = cbest;
        int32_t *tmp_s = malloc((size_t)L * sizeof(int32_t));
        int32_t *tmp_k = malloc((size_t)L * sizeof(int32_t));
        int32_t *tmp_c = malloc((size_t)L * sizeof(int32_t));
        while (t > 0) {
            int k = bk[(size_t)t * C + c];
            if (k < 1 || k > t) k = t; /* only with non-finite scores */
            double m1 = mk[(size_t)t * C + c];
            if (m1 < margin) margin = m1;
            tmp_s[nseg] = t - k; tmp_k[nseg] = k; tmp_c[nseg] = c;
            ++nseg;
            int s = t - k;
            if (s > 0) {
                double m2 = mc[(size_t)s * C + c];
                if (m2 < margin) margin = m2;
                c = bc[(size_t)s * C + c];
                if (c < 0) c = 0; /* only with non-finite scores */
            }
            t = s;
        }
        for (int j = 0; j < nseg; ++j) {
            seg_start[(size_t)b * T + j] = tmp_s[nseg - 1 - j];
            seg_len[(size_t)b * T + j] = tmp_k[nseg - 1 - j];
            seg_label[(size_t)b * T + j] = tmp_c[nseg - 1 - j];
        }
        num_segs[b] = nseg;
        if (min_margin) min_margin[b] = margin;
        free(tmp_s); free(tmp_k); free(tmp_c);
        free(S); free(nu); free(ah); free(uh); free(bk); free(bc); free(mk); free(mc);
    }
    return rc;
}
