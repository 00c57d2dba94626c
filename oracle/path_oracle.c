/*
 * PaTH attention CPU oracle (fp64).  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code with the HIP path: it is a plain,
 * slow and obviously correct evaluation of what PaTH attention computes.
 *
 * Definitions followed (PaTH paper; pages "PaTH Attention: Position Encoding
 * via Accumulating Householder Transformations"):
 *   - transition  H_t = I - beta_t w_t w_t^T               (Dutch technical
 *     summary, section 2 "Kernmechanisme"; Chinese notes, "key design")
 *   - logit       A_ij ~ exp(k_j^T (H_{j+1} ... H_i) q_i),  j <= i
 *     (same sections; the product runs from s = j+1 to s = i)
 *   - output      o_t = (1/Z_t) sum_{j<=t} v_j exp(logit_tj)
 *     (Chinese notes, "relation to linear RNNs", softmax form)
 *   - PaTH-FoX    the weight is additionally multiplied by prod_{s=j+1}^{i} f_s,
 *     i.e. an additive bias sum_{s=j+1}^{i} log f_s on the logit
 *     (Chinese notes, "PaTH-FoX extension")
 *   - inference   cached keys are updated in place at every step,
 *     k_j <- (I - beta_t w_t w_t^T) k_j  (Dutch summary section 3
 *     "Inferentie"; Chinese notes, training/inference strategy)
 *
 * Readings adopted where the pages are silent: 0-based token index (so H_0,
 * beta_0 and f_0 never enter a logit); the softmax scale multiplies only the
 * bilinear term; lse is the natural-log log-sum-exp of the (scaled, gated)
 * logits of a row.
 *
 * Layout: q, k, v, w are [BH][Lt][d] row-major doubles; beta, log_f are
 * [BH][Lt].  log_f may be NULL (PaTH without the forget gate).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double dot(const double* a, const double* b, long d) {
    double s = 0.0;
    for (long i = 0; i < d; ++i) s += a[i] * b[i];
    return s;
}

/* x <- (I - beta w w^T) x */
static void apply_h(double* x, const double* w, double beta, long d) {
    double a = beta * dot(w, x, d);
    for (long i = 0; i < d; ++i) x[i] -= a * w[i];
}

/* softmax-weighted sum of rows v[0..n) with logits s[0..n) */
static void softmax_rows(const double* s, long n, const double* v, long d,
                         double* out, double* lse) {
    double m = -INFINITY;
    for (long j = 0; j < n; ++j) if (s[j] > m) m = s[j];
    double z = 0.0;
    for (long i = 0; i < d; ++i) out[i] = 0.0;
    for (long j = 0; j < n; ++j) {
        double p = exp(s[j] - m);
        z += p;
        for (long i = 0; i < d; ++i) out[i] += p * v[j * d + i];
    }
    for (long i = 0; i < d; ++i) out[i] /= z;
    if (lse) *lse = m + log(z);
}

int path_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Recurrent (in-place key update) evaluation of every output row.
 * At step t: every cached key j < t is multiplied by H_t, key t is appended
 * unchanged, then query t attends over keys 0..t.
 * If kcache != NULL, the transformed key cache as it stands after step
 * Lcache-1 (i.e. H_{Lcache-1}...H_{j+1} k_j for j < Lcache) is written to
 * kcache [BH][Lcache][d].
 * Returns the number of threads used.
 */
int path_oracle_recurrent(long BH, long Lt, long d,
                          const double* q, const double* k, const double* v,
                          const double* w, const double* beta,
                          const double* log_f, double scale,
                          double* out, double* lse,
                          long Lcache, double* kcache, int nthreads) {
    int used = 1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long h = 0; h < BH; ++h) {
#ifdef _OPENMP
        if (h == 0) used = omp_get_num_threads();
#endif
        const double* qh = q + h * Lt * d;
        const double* kh = k + h * Lt * d;
        const double* vh = v + h * Lt * d;
        const double* wh = w + h * Lt * d;
        const double* bh = beta + h * Lt;
        const double* fh = log_f ? log_f + h * Lt : NULL;
        double* khat = (double*)malloc(sizeof(double) * Lt * d);
        double* F = (double*)malloc(sizeof(double) * Lt);
        double* s = (double*)malloc(sizeof(double) * Lt);
        for (long t = 0; t < Lt; ++t) {
            F[t] = (t ? F[t - 1] : 0.0) + (fh ? fh[t] : 0.0);
            for (long j = 0; j < t; ++j) apply_h(khat + j * d, wh + t * d, bh[t], d);
            memcpy(khat + t * d, kh + t * d, sizeof(double) * d);
            if (kcache && t == Lcache - 1)
                memcpy(kcache + h * Lcache * d, khat, sizeof(double) * Lcache * d);
            for (long j = 0; j <= t; ++j)
                s[j] = scale * dot(qh + t * d, khat + j * d, d) + (fh ? F[t] - F[j] : 0.0);
            softmax_rows(s, t + 1, vh, d, out + (h * Lt + t) * d,
                         lse ? lse + h * Lt + t : NULL);
        }
        free(khat);
        free(F);
        free(s);
    }
    return used;
}

/*
 * Selected output rows from the definition itself: the query is carried
 * leftwards, x_j = H_{j+1} ... H_i q_i, and the logit with key j is
 * scale * k_j . x_j + sum_{s=j+1}^{i} log f_s.   O(i d) per row.
 * rows: nrows pairs (head index, row index).  out_rows [nrows][d],
 * lse_rows [nrows]; logits (optional) [nrows][Lt], entries j > i set to NaN.
 */
int path_oracle_rows(long BH, long Lt, long d,
                     const double* q, const double* k, const double* v,
                     const double* w, const double* beta,
                     const double* log_f, double scale,
                     long nrows, const long* head_idx, const long* row_idx,
                     double* out_rows, double* lse_rows, double* logits,
                     int nthreads) {
    int used = 1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long r = 0; r < nrows; ++r) {
#ifdef _OPENMP
        if (r == 0) used = omp_get_num_threads();
#endif
        long h = head_idx[r], i = row_idx[r];
        const double* kh = k + h * Lt * d;
        const double* wh = w + h * Lt * d;
        const double* bh = beta + h * Lt;
        const double* fh = log_f ? log_f + h * Lt : NULL;
        double* x = (double*)malloc(sizeof(double) * d);
        double* s = (double*)malloc(sizeof(double) * (i + 1));
        memcpy(x, q + (h * Lt + i) * d, sizeof(double) * d);
        double g = 0.0;
        for (long j = i; j >= 0; --j) {
            s[j] = scale * dot(kh + j * d, x, d) + g;
            apply_h(x, wh + j * d, bh[j], d);   /* x_{j-1} = H_j x_j */
            if (fh) g += fh[j];                 /* sum_{s=j}^{i} log f_s */
        }
        softmax_rows(s, i + 1, v + h * Lt * d, d, out_rows + r * d,
                     lse_rows ? lse_rows + r : NULL);
        if (logits) {
            for (long j = 0; j < Lt; ++j)
                logits[r * Lt + j] = (j <= i) ? s[j] : NAN;
        }
        free(x);
        free(s);
    }
    return used;
}

/*
 * Selected transformed keys  H_T ... H_{j+1} k_j  (the in-place updated key
 * cache entry j as it stands after step T).  out [nrows][d].
 */
int path_oracle_transported_keys(long BH, long Lt, long d,
                                 const double* k, const double* w,
                                 const double* beta, long T, long nrows,
                                 const long* head_idx, const long* key_idx,
                                 double* out) {
    for (long r = 0; r < nrows; ++r) {
        long h = head_idx[r], j = key_idx[r];
        double* x = out + r * d;
        memcpy(x, k + (h * Lt + j) * d, sizeof(double) * d);
        for (long s = j + 1; s <= T; ++s)
            apply_h(x, w + (h * Lt + s) * d, beta[h * Lt + s], d);
    }
    return 0;
}
