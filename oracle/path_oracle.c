/*
 * path_oracle.c -- plain fp64 CPU oracle for PaTH attention (forward).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is the mathematical
 * definition written out, slowly and in double precision.
 *
 * Source of the definition (the discussion slides "PaTH Attention: Position
 * Encoding via Accumulating Householder Transformations", arXiv:2505.16381v2):
 *   - frame "PaTH inserts a learned transformation along every path"
 *     (paper Sec. 2.2): H_t = I - beta_t w_t w_t^T, and for j <= i the
 *     un-normalised logit is  k_j^T H_{j+1} H_{j+2} ... H_i q_i ; the row is
 *     soft-maxed over j <= i and o_i = sum_j A_ij v_j.  The product is empty
 *     on the diagonal j = i.
 *   - frame "FoX adds a separate mechanism for forgetting" (paper Sec. 2.2):
 *     PaTH-FoX multiplies the un-normalised weight by prod_{s=j+1..i} f_s,
 *     i.e. adds sum_{s=j+1..i} log f_s to the logit, outside the scale.
 *   - the authors' response page ("Implementation detail"): the logits are
 *     multiplied by `scale` before the softmax, with a causal -inf mask.
 *
 * Reading of the pages used here: logit s_ij = scale * c_ij + sum_{s=j+1..i}
 * log f_s, with the gate term not scaled; lse_i = ln sum_{j<=i} exp(s_ij).
 *
 * Algorithm (per query row i, rows independent):
 *   z <- q_i ; g <- 0
 *   for j = i, i-1, ..., 0:
 *       s_j <- scale * (k_j . z) + g        z = H_{j+1} ... H_i q_i
 *       if j == 0: stop
 *       z <- z - beta_j (w_j . z) w_j       apply H_j
 *       g <- g + log f_j
 *   two-pass softmax over s_0..s_i, then the value sum.
 * The factor H_0 and f_0 never enter any logit.
 *
 * All arrays are row-major, double precision:
 *   q, k, v, w : [n_heads, T, d]      beta, logf : [n_heads, T]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double dot(const double *a, const double *b, int d) {
    double s = 0.0;
    for (int t = 0; t < d; ++t) s += a[t] * b[t];
    return s;
}

/* Apply H = I - beta w w^T to z in place. */
static void apply_householder(double *z, const double *w, double beta, int d) {
    double a = beta * dot(w, z, d);
    for (int t = 0; t < d; ++t) z[t] -= a * w[t];
}

/*
 * Scaled, gated logits of one query row:  s[j] for j = 0..i.
 * z must have room for d doubles.
 */
static void row_logits(const double *q, const double *k, const double *w,
                       const double *beta, const double *logf, int i, int d,
                       double scale, double *z, double *s) {
    memcpy(z, q + (size_t)i * d, sizeof(double) * (size_t)d);
    double g = 0.0;
    for (int j = i; j >= 0; --j) {
        s[j] = scale * dot(k + (size_t)j * d, z, d) + g;
        if (j == 0) break;
        apply_householder(z, w + (size_t)j * d, beta[j], d);
        if (logf) g += logf[j];
    }
}

/*
 * Logit matrix of one head: S[i*T + j] = scale * c_ij + gate_ij for j <= i and
 * -INFINITY above the diagonal (the causal mask).  With scale = 1 and
 * logf = NULL this is the raw path logit c_ij = k_j^T H_{j+1}...H_i q_i.
 */
void oracle_path_logits(const double *q, const double *k, const double *w,
                        const double *beta, const double *logf, int T, int d,
                        double scale, double *S) {
    double *z = (double *)malloc(sizeof(double) * (size_t)d);
    for (int i = 0; i < T; ++i) {
        double *row = S + (size_t)i * T;
        row_logits(q, k, w, beta, logf, i, d, scale, z, row);
        for (int j = i + 1; j < T; ++j) row[j] = -INFINITY;
    }
    free(z);
}

/*
 * The walked query vector of one row: Z[(i-j)*d + t] = (H_{j+1}...H_i q_i)_t
 * for j = i, i-1, ..., 0 (so Z row 0 is q_i itself).  Exposed so that the
 * invariants of the transition (norm, erasure) can be checked directly.
 */
void oracle_path_walk(const double *q, const double *w, const double *beta,
                      int i, int d, double *Z) {
    double *z = (double *)malloc(sizeof(double) * (size_t)d);
    memcpy(z, q + (size_t)i * d, sizeof(double) * (size_t)d);
    for (int j = i; j >= 0; --j) {
        memcpy(Z + (size_t)(i - j) * d, z, sizeof(double) * (size_t)d);
        if (j == 0) break;
        apply_householder(z, w + (size_t)j * d, beta[j], d);
    }
    free(z);
}

/*
 * Attention outputs for a list of rows.  rows[2r] = head index, rows[2r+1] =
 * query index i.  out[r*d + t] = o_i, lse[r] = ln sum_{j<=i} exp(s_ij).
 * n_threads <= 0 uses the OpenMP default.  Returns 0, or -1 on a bad row.
 */
int oracle_path_attn_rows(const double *q, const double *k, const double *v,
                          const double *w, const double *beta,
                          const double *logf, int n_heads, int T, int d,
                          double scale, const int64_t *rows, int64_t n_rows,
                          double *out, double *lse, int n_threads) {
    for (int64_t r = 0; r < n_rows; ++r) {
        if (rows[2 * r] < 0 || rows[2 * r] >= n_heads || rows[2 * r + 1] < 0 ||
            rows[2 * r + 1] >= T)
            return -1;
    }
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)d);
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t h = rows[2 * r];
            const int i = (int)rows[2 * r + 1];
            const size_t off = (size_t)h * T * d;
            const double *qh = q + off, *kh = k + off, *vh = v + off;
            const double *wh = w + off;
            const double *bh = beta + (size_t)h * T;
            const double *fh = logf ? logf + (size_t)h * T : NULL;
            row_logits(qh, kh, wh, bh, fh, i, d, scale, z, s);
            double m = -INFINITY;
            for (int j = 0; j <= i; ++j) m = s[j] > m ? s[j] : m;
            double Z = 0.0;
            for (int j = 0; j <= i; ++j) {
                s[j] = exp(s[j] - m);
                Z += s[j];
            }
            double *o = out + (size_t)r * d;
            for (int t = 0; t < d; ++t) o[t] = 0.0;
            for (int j = 0; j <= i; ++j) {
                const double a = s[j] / Z;
                const double *vj = vh + (size_t)j * d;
                for (int t = 0; t < d; ++t) o[t] += a * vj[t];
            }
            lse[r] = m + log(Z);
        }
        free(s);
        free(z);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
