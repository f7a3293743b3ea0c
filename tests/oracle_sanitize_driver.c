/*
 * oracle_sanitize_driver.c - calls every entry point of the fp64 CPU oracle
 * (oracle/gmm_oracle.c) on small seeded inputs, including the edge cases
 * (one row, one component, a zero-weight component, a component too far away
 * to receive any mass, row counts around the oracle's 4096-row block), so
 * that an AddressSanitizer / UndefinedBehaviorSanitizer build of the oracle
 * exercises all of its loops. Test infrastructure only: built and run by
 * tests/test_oracle_sanitize.py with gcc; prints "ok" and exits 0 when every
 * call returns its expected status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_loglik(const float* x, int64_t n, int d, int k, const double* w, const double* mu,
                  const double* var, double* total, double* per_row);
int oracle_logdensity(const float* x, int64_t n, int d, int k, const double* w, const double* mu,
                      const double* var, double* out);
int oracle_em_step(const float* x, int64_t n, int d, int k, const double* w, const double* mu,
                   const double* var, double var_floor, double* w_out, double* mu_out,
                   double* var_out, double* loglik, double* nk_out);
int oracle_topm(const float* x, int64_t n, int d, int k, const double* w, const double* mu,
                const double* var, int m, int32_t* idx, double* resp, double* gap);
int oracle_kmeans_step(const float* x, int64_t n, int d, int k, const double* c, double* c_out,
                       int32_t* z_out, double* inertia, double* nk_out);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uni(void) { /* xorshift64*, uniform in [0, 1) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}

static int run_case(int64_t n, int d, int k, int zero_weight, int far) {
    float* x = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * d);
    double* w = malloc(sizeof(double) * k);
    double* mu = malloc(sizeof(double) * (size_t)k * d);
    double* var = malloc(sizeof(double) * (size_t)k * d);
    double* w2 = malloc(sizeof(double) * k);
    double* mu2 = malloc(sizeof(double) * (size_t)k * d);
    double* v2 = malloc(sizeof(double) * (size_t)k * d);
    double* nk = malloc(sizeof(double) * k);
    double* rows = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* ell = malloc(sizeof(double) * (size_t)k * 3);
    int m = k < 3 ? k : 3;
    int32_t* idx = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1) * m);
    double* resp = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * m);
    double* gap = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    int32_t* z = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int bad = 0;
    for (int64_t i = 0; i < n * d; ++i) x[i] = (float)(4.0 * uni() - 2.0);
    for (int j = 0; j < k; ++j) {
        w[j] = 0.1 + uni();
        for (int t = 0; t < d; ++t) {
            mu[(int64_t)j * d + t] = 4.0 * uni() - 2.0;
            var[(int64_t)j * d + t] = 0.2 + uni();
        }
    }
    if (zero_weight && k > 1) w[1] = 0.0;
    if (far && k > 2)
        for (int t = 0; t < d; ++t) mu[2 * (int64_t)d + t] = 1e5;
    double L = 0.0, inertia = 0.0;
    if (oracle_loglik(x, n, d, k, w, mu, var, &L, rows) != 0) bad |= 1;
    if (n > 0) {
        int64_t nl = n < 3 ? n : 3;
        if (oracle_logdensity(x, nl, d, k, w, mu, var, ell) != 0) bad |= 2;
        if (oracle_em_step(x, n, d, k, w, mu, var, 1e-6, w2, mu2, v2, &L, nk) != 0) bad |= 4;
        if (oracle_topm(x, n, d, k, w, mu, var, m, idx, resp, gap) != 0) bad |= 8;
        if (oracle_kmeans_step(x, n, d, k, mu, mu2, z, &inertia, nk) != 0) bad |= 16;
        if (!isfinite(L) || !isfinite(inertia)) bad |= 32;
    }
    free(x); free(w); free(mu); free(var); free(w2); free(mu2); free(v2); free(nk);
    free(rows); free(ell); free(idx); free(resp); free(gap); free(z);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run_case(0, 3, 2, 0, 0);
    bad |= run_case(1, 1, 1, 0, 0);
    bad |= run_case(5, 2, 4, 1, 1);
    bad |= run_case(4095, 3, 5, 1, 1);
    bad |= run_case(4097, 5, 3, 0, 1);
    bad |= run_case(9000, 7, 6, 1, 0);
    /* invalid inputs return a status and touch nothing */
    double w = -1.0, mu = 0.0, var = 1.0, L = 0.0;
    float x = 0.0f;
    if (oracle_loglik(&x, 1, 1, 1, &w, &mu, &var, &L, NULL) != 2) bad |= 64;
    if (oracle_em_step(&x, 0, 1, 1, &w, &mu, &var, 0.0, &w, &mu, &var, &L, NULL) != 1) bad |= 128;
    if (bad) {
        printf("failed %d\n", bad);
        return 1;
    }
    printf("ok\n");
    return 0;
}
