/*
 * gmm_oracle.c - plain fp64 CPU reference for one EM iteration of a
 * diagonal-covariance Gaussian mixture model.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load or call this library. The product path never
 * does: it shares no code, header, table or helper with the HIP library.
 *
 * What it computes (the textbook diagonal-GMM EM that the Flash-GMM pages
 * apply their tiling to: "Flash-GMM: A Memory-Efficient Kernel for Scalable
 * Soft Clustering", section 1 (responsibility matrix) and section 3 (EM with
 * per-tile statistics accumulated globally, O(KD) memory)). The pages print
 * no equations; these are the standard ones, written step by step:
 *
 *   1. log-density   l[n][k] = log w[k]
 *                              - 1/2 sum_d ( log(2 pi) + log v[k][d]
 *                                            + (x[n][d] - mu[k][d])^2 / v[k][d] )
 *                    (direct subtract-then-square form; w[k] = 0 gives -inf)
 *   2. normaliser    lse[n] = M + log sum_k exp(l[n][k] - M),  M = max_k l[n][k]
 *   3. log-likelihood L = sum_n lse[n]   (natural log, total, input parameters)
 *   4. responsibilities r[n][k] = exp(l[n][k] - lse[n])
 *   5. statistics    N[k]     = sum_n r[n][k]
 *                    T1[k][d] = sum_n r[n][k] (x[n][d] - mu[k][d])
 *                    T2[k][d] = sum_n r[n][k] (x[n][d] - mu[k][d])^2
 *                    (moments taken about the input mean: exact in maths)
 *   6. M-step        w'[k] = N[k] / N
 *                    N[k] > 0:  mu'[k] = mu[k] + T1[k] / N[k]
 *                               v'[k]  = max(T2[k]/N[k] - (T1[k]/N[k])^2, floor)
 *                    N[k] = 0:  mu'[k] = mu[k], v'[k] = v[k], w'[k] = 0
 *
 * Determinism: rows are taken in fixed blocks of ORACLE_BLOCK_ROWS rows.
 * Each block's fp64 partial sums are formed serially in row order, and the
 * block partials are added into the total strictly in block order, so the
 * result does not depend on the number of threads. Terms with r == 0.0
 * exactly are skipped in step 5 (adding an exact zero changes nothing).
 *
 * Loop order: the log-density loop runs over components innermost so that
 * the compiler can vectorise across components; for every (n, k) the sum
 * over d is still formed in order d = 0, 1, ..., D-1.
 *
 * Inputs X are fp32 (bf16 data is widened to fp32 exactly by the caller) and
 * are converted to fp64 exactly. Parameters are fp64.
 *
 * Return codes: 0 ok, 1 invalid sizes, 2 invalid parameters, 3 out of memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BLOCK_ROWS 4096
#define LOG_2PI 1.8378770664093454835606594728112

/* Parameters laid out for the log-density loop: transposed means and
 * variances (D x K) and the per-component constant
 *   log w[k] - 1/2 (D log 2 pi + sum_d log v[k][d]). */
typedef struct {
    int d, k;
    double* mu_t;   /* [d][k] */
    double* var_t;  /* [d][k] */
    double* cst;    /* [k] */
} prepared;

static void prepared_free(prepared* p) {
    free(p->mu_t);
    free(p->var_t);
    free(p->cst);
}

static int check_params(int d, int k, const double* w, const double* mu, const double* var) {
    int any_positive = 0;
    for (int j = 0; j < k; ++j) {
        if (!(w[j] >= 0.0) || !isfinite(w[j])) return 2;
        if (w[j] > 0.0) any_positive = 1;
        for (int t = 0; t < d; ++t) {
            double m = mu[(int64_t)j * d + t], v = var[(int64_t)j * d + t];
            if (!isfinite(m) || !isfinite(v) || !(v > 0.0)) return 2;
        }
    }
    return any_positive ? 0 : 2;
}

static int prepare(int d, int k, const double* w, const double* mu, const double* var, prepared* p) {
    p->d = d;
    p->k = k;
    p->mu_t = (double*)malloc(sizeof(double) * (size_t)d * k);
    p->var_t = (double*)malloc(sizeof(double) * (size_t)d * k);
    p->cst = (double*)malloc(sizeof(double) * (size_t)k);
    if (!p->mu_t || !p->var_t || !p->cst) {
        prepared_free(p);
        return 3;
    }
    for (int j = 0; j < k; ++j) {
        double logdet = 0.0;
        for (int t = 0; t < d; ++t) {
            p->mu_t[(int64_t)t * k + j] = mu[(int64_t)j * d + t];
            p->var_t[(int64_t)t * k + j] = var[(int64_t)j * d + t];
            logdet += log(var[(int64_t)j * d + t]);
        }
        p->cst[j] = log(w[j]) - 0.5 * ((double)d * LOG_2PI + logdet);
    }
    return 0;
}

/* Step 1 for one row: out[k] = l[n][k]. acc is scratch of length k. */
static void row_logdensity(const prepared* p, const float* xr, double* acc, double* out) {
    const int d = p->d, k = p->k;
    for (int j = 0; j < k; ++j) acc[j] = 0.0;
    for (int t = 0; t < d; ++t) {
        const double xv = (double)xr[t];
        const double* m = p->mu_t + (int64_t)t * k;
        const double* v = p->var_t + (int64_t)t * k;
        for (int j = 0; j < k; ++j) {
            const double diff = xv - m[j];
            acc[j] += diff * diff / v[j];
        }
    }
    for (int j = 0; j < k; ++j) out[j] = p->cst[j] - 0.5 * acc[j];
}

/* Step 2 for one row. */
static double row_lse(const double* l, int k) {
    double m = -INFINITY;
    for (int j = 0; j < k; ++j)
        if (l[j] > m) m = l[j];
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += exp(l[j] - m);
    return m + log(s);
}

static int threads_for(int64_t units) {
#ifdef _OPENMP
    int t = omp_get_max_threads();
    return (int64_t)t > units ? (int)(units > 0 ? units : 1) : t;
#else
    (void)units;
    return 1;
#endif
}

/* Per-row log-likelihood (optional) and the total L = sum_n lse[n]. */
int oracle_loglik(const float* x, int64_t n, int d, int k, const double* w, const double* mu,
                  const double* var, double* total, double* per_row) {
    if (n < 0 || d < 1 || k < 1) return 1;
    int rc = check_params(d, k, w, mu, var);
    if (rc) return rc;
    *total = 0.0;
    if (n == 0) return 0;
    prepared p;
    if ((rc = prepare(d, k, w, mu, var, &p))) return rc;
    const int64_t nblocks = (n + ORACLE_BLOCK_ROWS - 1) / ORACLE_BLOCK_ROWS;
    double* block_sum = (double*)calloc((size_t)nblocks, sizeof(double));
    if (!block_sum) {
        prepared_free(&p);
        return 3;
    }
    int fail = 0;
#pragma omp parallel num_threads(threads_for(nblocks))
    {
        double* acc = (double*)malloc(sizeof(double) * k);
        double* l = (double*)malloc(sizeof(double) * k);
        if (!acc || !l) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < nblocks; ++b) {
            if (!acc || !l) continue;
            const int64_t lo = b * ORACLE_BLOCK_ROWS;
            const int64_t hi = lo + ORACLE_BLOCK_ROWS < n ? lo + ORACLE_BLOCK_ROWS : n;
            double s = 0.0;
            for (int64_t i = lo; i < hi; ++i) {
                row_logdensity(&p, x + i * d, acc, l);
                const double v = row_lse(l, k);
                if (per_row) per_row[i] = v;
                s += v;
            }
            block_sum[b] = s;
        }
        free(acc);
        free(l);
    }
    if (!fail)
        for (int64_t b = 0; b < nblocks; ++b) *total += block_sum[b];
    free(block_sum);
    prepared_free(&p);
    return fail ? 3 : 0;
}

/* Full log-density matrix for a small set of rows (n x k, row-major). */
int oracle_logdensity(const float* x, int64_t n, int d, int k, const double* w, const double* mu,
                      const double* var, double* out) {
    if (n < 0 || d < 1 || k < 1) return 1;
    int rc = check_params(d, k, w, mu, var);
    if (rc) return rc;
    prepared p;
    if ((rc = prepare(d, k, w, mu, var, &p))) return rc;
    double* acc = (double*)malloc(sizeof(double) * k);
    if (!acc) {
        prepared_free(&p);
        return 3;
    }
    for (int64_t i = 0; i < n; ++i) row_logdensity(&p, x + i * d, acc, out + i * k);
    free(acc);
    prepared_free(&p);
    return 0;
}

/* One EM iteration (steps 1-6). Outputs the new parameters, the log-likelihood
 * of the INPUT parameters and the responsibility mass N[k] per component. */
int oracle_em_step(const float* x, int64_t n, int d, int k, const double* w, const double* mu,
                   const double* var, double var_floor, double* w_out, double* mu_out,
                   double* var_out, double* loglik, double* nk_out) {
    if (n < 1 || d < 1 || k < 1) return 1;
    if (!(var_floor >= 0.0) || !isfinite(var_floor)) return 1;
    int rc = check_params(d, k, w, mu, var);
    if (rc) return rc;
    prepared p;
    if ((rc = prepare(d, k, w, mu, var, &p))) return rc;

    const int64_t nblocks = (n + ORACLE_BLOCK_ROWS - 1) / ORACLE_BLOCK_ROWS;
    const int64_t stride = 1 + (int64_t)k * (1 + 2 * (int64_t)d); /* L, N[k], T1[k][d], T2[k][d] */
    /* blocks are processed in batches; the batch size only bounds memory */
    int64_t batch = threads_for(nblocks);
    const int64_t budget = (int64_t)2 << 30;
    while (batch > 1 && batch * stride * (int64_t)sizeof(double) > budget) batch /= 2;

    double* total = (double*)calloc((size_t)stride, sizeof(double));
    double* part = (double*)malloc(sizeof(double) * (size_t)(batch * stride));
    if (!total || !part) {
        free(total);
        free(part);
        prepared_free(&p);
        return 3;
    }
    int fail = 0;
    for (int64_t b0 = 0; b0 < nblocks && !fail; b0 += batch) {
        const int64_t b1 = b0 + batch < nblocks ? b0 + batch : nblocks;
#pragma omp parallel num_threads(threads_for(b1 - b0))
        {
            double* acc = (double*)malloc(sizeof(double) * k);
            double* l = (double*)malloc(sizeof(double) * k);
            if (!acc || !l) {
#pragma omp atomic write
                fail = 1;
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t b = b0; b < b1; ++b) {
                if (!acc || !l) continue;
                double* s = part + (b - b0) * stride;
                memset(s, 0, sizeof(double) * (size_t)stride);
                double* sL = s;
                double* sN = s + 1;
                double* sT1 = sN + k;
                double* sT2 = sT1 + (int64_t)k * d;
                const int64_t lo = b * ORACLE_BLOCK_ROWS;
                const int64_t hi = lo + ORACLE_BLOCK_ROWS < n ? lo + ORACLE_BLOCK_ROWS : n;
                for (int64_t i = lo; i < hi; ++i) {
                    const float* xr = x + i * d;
                    row_logdensity(&p, xr, acc, l);
                    const double lse = row_lse(l, k);
                    *sL += lse;
                    for (int j = 0; j < k; ++j) {
                        const double r = exp(l[j] - lse);
                        if (r == 0.0) continue;
                        sN[j] += r;
                        const double* m = mu + (int64_t)j * d;
                        double* t1 = sT1 + (int64_t)j * d;
                        double* t2 = sT2 + (int64_t)j * d;
                        for (int t = 0; t < d; ++t) {
                            const double diff = (double)xr[t] - m[t];
                            t1[t] += r * diff;
                            t2[t] += r * (diff * diff);
                        }
                    }
                }
            }
            free(acc);
            free(l);
        }
        for (int64_t b = b0; b < b1 && !fail; ++b) {
            const double* s = part + (b - b0) * stride;
            for (int64_t e = 0; e < stride; ++e) total[e] += s[e];
        }
    }
    if (!fail) {
        const double* N = total + 1;
        const double* T1 = N + k;
        const double* T2 = T1 + (int64_t)k * d;
        *loglik = total[0];
        for (int j = 0; j < k; ++j) {
            if (nk_out) nk_out[j] = N[j];
            w_out[j] = N[j] / (double)n;
            for (int t = 0; t < d; ++t) {
                const int64_t e = (int64_t)j * d + t;
                if (N[j] > 0.0) {
                    const double m1 = T1[e] / N[j];
                    const double v = T2[e] / N[j] - m1 * m1;
                    mu_out[e] = mu[e] + m1;
                    var_out[e] = v > var_floor ? v : var_floor;
                } else {
                    mu_out[e] = mu[e];
                    var_out[e] = var[e];
                }
            }
            if (!(N[j] > 0.0)) w_out[j] = 0.0;
        }
    }
    free(total);
    free(part);
    prepared_free(&p);
    return fail ? 3 : 0;
}

/* The m most responsible components of each row, most responsible first
 * (equivalently the m largest log-densities; ties go to the smaller index),
 * with their responsibilities r[n][k] = exp(l[n][k] - lse[n]). gap[n], if
 * given, receives l_(m) - l_(m+1) (the margin of the m-th choice; +inf when
 * m == k). */
int oracle_topm(const float* x, int64_t n, int d, int k, const double* w, const double* mu,
                const double* var, int m, int32_t* idx, double* resp, double* gap) {
    if (n < 0 || d < 1 || k < 1 || m < 1 || m > k) return 1;
    int rc = check_params(d, k, w, mu, var);
    if (rc) return rc;
    if (n == 0) return 0;
    prepared p;
    if ((rc = prepare(d, k, w, mu, var, &p))) return rc;
    int fail = 0;
#pragma omp parallel num_threads(threads_for((n + ORACLE_BLOCK_ROWS - 1) / ORACLE_BLOCK_ROWS))
    {
        double* acc = (double*)malloc(sizeof(double) * k);
        double* l = (double*)malloc(sizeof(double) * k);
        char* taken = (char*)malloc((size_t)k);
        if (!acc || !l || !taken) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, ORACLE_BLOCK_ROWS)
        for (int64_t i = 0; i < n; ++i) {
            if (!acc || !l || !taken) continue;
            row_logdensity(&p, x + i * d, acc, l);
            const double lse = row_lse(l, k);
            memset(taken, 0, (size_t)k);
            double last = 0.0;
            for (int s = 0; s <= m && s < k; ++s) {
                int best = -1;
                for (int j = 0; j < k; ++j)
                    if (!taken[j] && (best < 0 || l[j] > l[best])) best = j;
                if (s < m) {
                    taken[best] = 1;
                    idx[i * m + s] = best;
                    resp[i * m + s] = exp(l[best] - lse);
                    last = l[best];
                } else if (gap) {
                    gap[i] = last - l[best];
                }
            }
            if (gap && m == k) gap[i] = INFINITY;
        }
        free(acc);
        free(l);
        free(taken);
    }
    prepared_free(&p);
    return fail ? 3 : 0;
}

/* One Lloyd (k-means) step: the hard-assignment quantizer the Flash-GMM
 * pages replace with a GMM in the IVF coarse quantizer ("Flash-GMM: A
 * Memory-Efficient Kernel for Scalable Soft Clustering", section 3, the
 * comparison with K-Means). It is the limit of the EM step with equal
 * weights and equal spherical variances as the variance goes to zero. Steps:
 *
 *   1. distance    D[n][k] = sum_d (x[n][d] - c[k][d])^2   (direct form)
 *   2. assignment  z[n] = argmin_k D[n][k]  (ties: the smaller k)
 *   3. inertia     I = sum_n D[n][z[n]]     (for the input centroids)
 *   4. update      N[k] = #{n : z[n] = k}
 *                  N[k] > 0: c'[k] = c[k] + (1/N[k]) sum_{z[n]=k} (x[n] - c[k])
 *                  N[k] = 0: c'[k] = c[k]
 *
 * Same fixed-block determinism as oracle_em_step. z_out and nk_out may be
 * NULL. */
int oracle_kmeans_step(const float* x, int64_t n, int d, int k, const double* c,
                       double* c_out, int32_t* z_out, double* inertia, double* nk_out) {
    if (n < 1 || d < 1 || k < 1) return 1;
    for (int64_t e = 0; e < (int64_t)k * d; ++e)
        if (!isfinite(c[e])) return 2;
    double* c_t = (double*)malloc(sizeof(double) * (size_t)d * k); /* [d][k] */
    if (!c_t) return 3;
    for (int j = 0; j < k; ++j)
        for (int t = 0; t < d; ++t) c_t[(int64_t)t * k + j] = c[(int64_t)j * d + t];

    const int64_t nblocks = (n + ORACLE_BLOCK_ROWS - 1) / ORACLE_BLOCK_ROWS;
    const int64_t stride = 1 + (int64_t)k * (1 + (int64_t)d); /* I, N[k], T1[k][d] */
    int64_t batch = threads_for(nblocks);
    const int64_t budget = (int64_t)2 << 30;
    while (batch > 1 && batch * stride * (int64_t)sizeof(double) > budget) batch /= 2;
    double* total = (double*)calloc((size_t)stride, sizeof(double));
    double* part = (double*)malloc(sizeof(double) * (size_t)(batch * stride));
    if (!total || !part) {
        free(total);
        free(part);
        free(c_t);
        return 3;
    }
    int fail = 0;
    for (int64_t b0 = 0; b0 < nblocks && !fail; b0 += batch) {
        const int64_t b1 = b0 + batch < nblocks ? b0 + batch : nblocks;
#pragma omp parallel num_threads(threads_for(b1 - b0))
        {
            double* dist = (double*)malloc(sizeof(double) * k);
            if (!dist) {
#pragma omp atomic write
                fail = 1;
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t b = b0; b < b1; ++b) {
                if (!dist) continue;
                double* s = part + (b - b0) * stride;
                memset(s, 0, sizeof(double) * (size_t)stride);
                double* sI = s;
                double* sN = s + 1;
                double* sT1 = sN + k;
                const int64_t lo = b * ORACLE_BLOCK_ROWS;
                const int64_t hi = lo + ORACLE_BLOCK_ROWS < n ? lo + ORACLE_BLOCK_ROWS : n;
                for (int64_t i = lo; i < hi; ++i) {
                    const float* xr = x + i * d;
                    for (int j = 0; j < k; ++j) dist[j] = 0.0;
                    for (int t = 0; t < d; ++t) {
                        const double xv = (double)xr[t];
                        const double* ct = c_t + (int64_t)t * k;
                        for (int j = 0; j < k; ++j) {
                            const double diff = xv - ct[j];
                            dist[j] += diff * diff;
                        }
                    }
                    int z = 0;
                    for (int j = 1; j < k; ++j)
                        if (dist[j] < dist[z]) z = j;
                    if (z_out) z_out[i] = z;
                    *sI += dist[z];
                    sN[z] += 1.0;
                    const double* cz = c + (int64_t)z * d;
                    double* t1 = sT1 + (int64_t)z * d;
                    for (int t = 0; t < d; ++t) t1[t] += (double)xr[t] - cz[t];
                }
            }
            free(dist);
        }
        for (int64_t b = b0; b < b1 && !fail; ++b) {
            const double* s = part + (b - b0) * stride;
            for (int64_t e = 0; e < stride; ++e) total[e] += s[e];
        }
    }
    if (!fail) {
        const double* N = total + 1;
        const double* T1 = N + k;
        *inertia = total[0];
        for (int j = 0; j < k; ++j) {
            if (nk_out) nk_out[j] = N[j];
            for (int t = 0; t < d; ++t) {
                const int64_t e = (int64_t)j * d + t;
                c_out[e] = N[j] > 0.0 ? c[e] + T1[e] / N[j] : c[e];
            }
        }
    }
    free(total);
    free(part);
    free(c_t);
    return fail ? 3 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
