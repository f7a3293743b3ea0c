// gmm_api.hip - the C ABI declared in include/gmm_em.h: argument checks,
// workspace planning and the launch sequence of each entry point.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <new>
#include <stdlib.h>
#include <string.h>

#include "gmm_em.h"
#include "gmm_internal.h"

namespace gmm {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool make_plan(int d, int k, void* ws, Plan* pl) {
    if (d < 1 || k < 1 || k > (1 << 22)) return false;
    Plan p;
    p.d = d;
    p.dp = (d + 15) / 16 * 16;
    if (p.dp > MAX_DP) {
        p.wide = true;
        p.dp = (d + 127) / 128 * 128;
        if (p.dp > WIDE_MAX_DP) return false;
    }
    p.k = k;
    p.kp = (k + 127) / 128 * 128;  // whole 8-tile groups of the statistics pass
    p.ntiles = p.kp / 16;
    // narrow: one block per (row group, K-group of waves); wide: one block per
    // (row group, K-tile)
    const int kgroups = p.wide ? p.ntiles : p.ntiles / waves_per_stats_block(p.dp);
    p.kgroups = kgroups;
    int g = (1024 + kgroups - 1) / kgroups;
    p.ngroups = g < 1 ? 1 : (g > 512 ? 512 : g);
    p.chunk = p.wide ? WIDE_CHUNK_ROWS : CHUNK_ROWS;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t o_status = take(16 * sizeof(int));
    const size_t o_shift = take((size_t)p.dp * sizeof(double));
    const size_t o_pg = take((size_t)p.kp * 2 * p.dp * sizeof(double));
    const size_t o_c = take((size_t)p.kp * sizeof(double));
    const size_t o_lse = take((size_t)CHUNK_ROWS * sizeof(double));
    const size_t o_ll = take((size_t)(CHUNK_ROWS / LL_ROWS) * sizeof(double));
    const size_t o_np = take((size_t)p.ngroups * p.kp * sizeof(double));
    const size_t o_part = take((size_t)p.ngroups * p.kp * 2 * p.dp * sizeof(double));
    const size_t o_lt = take(sizeof(double));
    const size_t o_xb = take((size_t)p.ngroups * 4 * kgroups * 32 * sizeof(double2));
    const size_t o_cnt = take((size_t)p.ngroups * kgroups * sizeof(unsigned));
    const size_t wpart = p.wide ? (size_t)WIDE_CHUNK_ROWS * p.ntiles : 0;
    const size_t o_wl = take(wpart * sizeof(double2));
    const size_t o_wv = take(wpart * WIDE_TM * sizeof(double));
    const size_t o_wi = take(wpart * WIDE_TM * sizeof(int32_t));
    p.bytes = off;
    if (ws) {
        char* b = (char*)ws;
        p.status = (int*)(b + o_status);
        p.shift = (double*)(b + o_shift);
        p.Pg = (double*)(b + o_pg);
        p.cvec = (double*)(b + o_c);
        p.lse = (double*)(b + o_lse);
        p.llpart = (double*)(b + o_ll);
        p.npart = (double*)(b + o_np);
        p.part = (double*)(b + o_part);
        p.ll_tmp = (double*)(b + o_lt);
        p.xbuf = (double2*)(b + o_xb);
        p.counters = (unsigned*)(b + o_cnt);
        if (p.wide) {
            p.wlpart = (double2*)(b + o_wl);
            p.wtval = (double*)(b + o_wv);
            p.wtidx = (int32_t*)(b + o_wi);
        }
    }
    *pl = p;
    return true;
}

}  // namespace gmm

using namespace gmm;

static int check_common(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                        const void* w, const void* mu, const void* var, int32_t k, void* ws,
                        size_t ws_bytes, Plan* pl) {
    if (n < 0 || d < 1 || k < 1 || ldx < d) return GMM_E_INVALID;
    // the statistics pass addresses a 32-row tile with 32-bit byte offsets
    if (ldx > MAX_LDX) return GMM_E_UNSUPPORTED;
    if (n > 0 && !x) return GMM_E_INVALID;
    if (!w || !mu || !var) return GMM_E_INVALID;
    if (x_dtype != GMM_F32 && x_dtype != GMM_BF16) return GMM_E_DTYPE;
    if (!make_plan(d, k, nullptr, pl)) return GMM_E_UNSUPPORTED;
    if (!ws || ws_bytes < pl->bytes) return GMM_E_WORKSPACE;
    if ((uintptr_t)ws % 256 != 0) return GMM_E_WORKSPACE;
    make_plan(d, k, ws, pl);
    return GMM_OK;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? GMM_OK : GMM_E_HIP; }

// Optional event recording around the two passes (gmm_profile_begin/end).
struct Prof {
    bool on = false;
    int cap = 0;
    int n1 = 0, n2 = 0;
    hipEvent_t* ev1 = nullptr;  // [2*cap] start/stop pairs, pass 1
    hipEvent_t* ev2 = nullptr;  // [2*cap] pass 2
};
static Prof g_prof;

static void prof_mark(int pass, bool start, hipStream_t st) {
    if (!g_prof.on) return;
    int& cnt = pass == 1 ? g_prof.n1 : g_prof.n2;
    hipEvent_t* ev = pass == 1 ? g_prof.ev1 : g_prof.ev2;
    if (cnt >= g_prof.cap) return;
    (void)hipEventRecord(ev[2 * cnt + (start ? 0 : 1)], st);
    if (!start) ++cnt;
}

// E-step over all rows in chunks of CHUNK_ROWS: per-row normalisers into the
// workspace scratch and the log-likelihood partials; with `stats`, each
// chunk's statistics pass follows its normaliser pass; with m > 0, the top-m
// components of each row are written to idx/resp; lse_rows, if given,
// receives every row's normaliser instead of the chunk scratch.
static hipError_t run_passes(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                             bool stats, hipStream_t st, int m = 0, int32_t* idx = nullptr,
                             float* resp = nullptr, double* lse_rows = nullptr) {
    const size_t esz = dtype == GMM_BF16 ? 2 : 4;
    for (int64_t c0 = 0, ci = 0; c0 < n; c0 += pl.chunk, ++ci) {
        const int64_t cn = n - c0 < pl.chunk ? n - c0 : pl.chunk;
        const void* xc = (const char*)x + (size_t)c0 * (size_t)ldx * esz;
        double* lse = lse_rows ? lse_rows + c0 : pl.lse;
        int32_t* ic = m > 0 ? idx + c0 * m : nullptr;
        float* rc = m > 0 ? resp + c0 * m : nullptr;
        prof_mark(1, true, st);
        hipError_t e = pl.wide ? launch_wide_lse(pl, xc, cn, ldx, dtype, lse, ci > 0, m, ic, rc, st)
                               : launch_lse(pl, xc, cn, ldx, dtype, lse, ci > 0, m, ic, rc, st);
        prof_mark(1, false, st);
        if (e != hipSuccess) return e;
        if (stats) {
            prof_mark(2, true, st);
            e = pl.wide ? launch_wide_stats(pl, xc, cn, ldx, dtype, lse, ci > 0, st)
                        : launch_stats(pl, xc, cn, ldx, dtype, lse, ci > 0, st);
            prof_mark(2, false, st);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// Schedule of the EM step. The default is the two-pass schedule; the
// cooperative single pass (GMM_EM_SCHEDULE=coop) removes the normaliser
// pass but pays a cross-workgroup exchange per 32-row tile, which measured
// slower on MI355X at the headline shape (321 vs 217 ms per step at N=1e7,
// D=96, K=1024). coop fails with GMM_E_UNSUPPORTED where the grid cannot be
// co-resident.
enum { SCHED_TWO_PASS = 1, SCHED_COOP = 2 };

static int schedule_choice() {
    const char* v = getenv("GMM_EM_SCHEDULE");
    if (v && !strcmp(v, "coop")) return SCHED_COOP;
    return SCHED_TWO_PASS;
}

// Row groups of the cooperative pass for the current device, or 0 if it
// cannot run: every block must be co-resident, and each XCD (8 of them,
// workgroups dispatched round-robin) must hold whole row groups.
static int coop_groups(const Plan& pl) {
    static int cached_dev = -1, cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev != cached_dev) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess || !prop.cooperativeLaunch) return 0;
        cached_cus = prop.multiProcessorCount;
        cached_dev = dev;
    }
    if (pl.wide) return 0;  // the cooperative kernel holds a K-group's rows in registers
    const int bpc = coop_blocks_per_cu(pl.dp);
    if (bpc < 1 || pl.kgroups < 1 || pl.kgroups > 64) return 0;  // one wave watches the flags
    int groups = (cached_cus * bpc) / pl.kgroups;
    groups = groups / 8 * 8;
    if (groups > pl.ngroups) groups = pl.ngroups / 8 * 8;
    return groups >= 8 ? groups : 0;
}

static int ll_parts(const Plan& pl, int64_t n) {
    const int64_t first = n < pl.chunk ? n : pl.chunk;
    return (int)((first + LL_ROWS - 1) / LL_ROWS);
}

extern "C" {

size_t gmm_workspace_bytes(int32_t d, int32_t k) {
    Plan p;
    return make_plan(d, k, nullptr, &p) ? p.bytes : 0;
}

int gmm_em_step(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype, float* weights,
                float* means, float* variances, int32_t k, float var_floor, double* loglik_dev,
                void* workspace, size_t workspace_bytes, void* stream) {
    Plan pl;
    int rc = check_common(x, n, d, ldx, x_dtype, weights, means, variances, k, workspace,
                          workspace_bytes, &pl);
    if (rc) return rc;
    if (n < 1 || !(var_floor >= 0.0f) || !isfinite(var_floor)) return GMM_E_INVALID;
    hipStream_t st = (hipStream_t)stream;
    const int sched = schedule_choice();
    const int cg = sched == SCHED_TWO_PASS ? 0 : coop_groups(pl);
    if (sched == SCHED_COOP && cg == 0) return GMM_E_UNSUPPORTED;
    double* ll_out = loglik_dev ? loglik_dev : pl.ll_tmp;
    hipError_t e = launch_prologue(pl, weights, means, variances, st);
    if (e != hipSuccess) return GMM_E_HIP;
    if (cg > 0) {
        prof_mark(2, true, st);
        e = launch_coop(pl, x, n, ldx, x_dtype, cg, st);
        prof_mark(2, false, st);
        if (e == hipSuccess) {
            e = launch_ll_final(pl, cg, ll_out, st);
            if (e == hipSuccess) e = launch_finalize(pl, cg, n, var_floor, weights, means, variances, st);
            return hip_status(e);
        }
        if (sched == SCHED_COOP) return GMM_E_HIP;
        (void)hipGetLastError();  // fall back to the two-pass schedule
    }
    e = run_passes(pl, x, n, ldx, x_dtype, true, st);
    if (e == hipSuccess) e = launch_ll_final(pl, ll_parts(pl, n), ll_out, st);
    if (e == hipSuccess) e = launch_finalize(pl, pl.ngroups, n, var_floor, weights, means, variances, st);
    return hip_status(e);
}

int gmm_fit(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype, float* weights,
            float* means, float* variances, int32_t k, float var_floor, int32_t max_iter,
            double tol, double* loglik_hist_dev, int32_t* iters_done, void* workspace,
            size_t workspace_bytes, void* stream) {
    if (max_iter < 0 || !(tol >= 0.0) || !isfinite(tol)) return GMM_E_INVALID;
    Plan pl;
    int rc = check_common(x, n, d, ldx, x_dtype, weights, means, variances, k, workspace,
                          workspace_bytes, &pl);
    if (rc) return rc;
    if (n < 1 || !(var_floor >= 0.0f) || !isfinite(var_floor)) return GMM_E_INVALID;
    hipStream_t st = (hipStream_t)stream;
    double prev = 0.0;
    int done = 0;
    for (int it = 0; it < max_iter; ++it) {
        double* ll = loglik_hist_dev ? loglik_hist_dev + it : pl.ll_tmp;
        rc = gmm_em_step(x, n, d, ldx, x_dtype, weights, means, variances, k, var_floor, ll,
                         workspace, workspace_bytes, stream);
        if (rc) break;
        ++done;
        if (tol > 0.0) {
            double cur = 0.0;
            if (hipMemcpyAsync(&cur, ll, sizeof(double), hipMemcpyDeviceToHost, st) != hipSuccess ||
                hipStreamSynchronize(st) != hipSuccess) {
                rc = GMM_E_HIP;
                break;
            }
            if (it > 0 && cur - prev < tol * fabs(cur)) break;
            prev = cur;
        }
    }
    if (iters_done) *iters_done = done;
    return rc;
}

int gmm_loglik(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
               const float* weights, const float* means, const float* variances, int32_t k,
               double* total_dev, double* per_row_dev, void* workspace, size_t workspace_bytes,
               void* stream) {
    Plan pl;
    int rc = check_common(x, n, d, ldx, x_dtype, weights, means, variances, k, workspace,
                          workspace_bytes, &pl);
    if (rc) return rc;
    if (!total_dev) return GMM_E_INVALID;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = launch_prologue(pl, weights, means, variances, st);
    if (e == hipSuccess)
        e = run_passes(pl, x, n, ldx, x_dtype, false, st, 0, nullptr, nullptr, per_row_dev);
    if (e == hipSuccess) e = launch_ll_final(pl, ll_parts(pl, n), total_dev, st);
    return hip_status(e);
}

int gmm_assign_topm(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                    const float* weights, const float* means, const float* variances, int32_t k,
                    int32_t m, int32_t* idx_dev, float* resp_dev, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (m < 1 || m > 4 || m > k || ((!idx_dev || !resp_dev) && n > 0)) return GMM_E_INVALID;
    Plan pl;
    int rc = check_common(x, n, d, ldx, x_dtype, weights, means, variances, k, workspace,
                          workspace_bytes, &pl);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = launch_prologue(pl, weights, means, variances, st);
    if (e == hipSuccess) e = run_passes(pl, x, n, ldx, x_dtype, false, st, m, idx_dev, resp_dev);
    return hip_status(e);
}

int gmm_kmeans_step(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                    float* centroids, int32_t k, int32_t* assign_dev, double* inertia_dev,
                    void* workspace, size_t workspace_bytes, void* stream) {
    if (n < 1 || !centroids) return GMM_E_INVALID;
    Plan pl;
    // (the check wants three parameter pointers; k-means has only centroids)
    int rc = check_common(x, n, d, ldx, x_dtype, centroids, centroids, centroids, k, workspace,
                          workspace_bytes, &pl);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    // weights and variances null: the k-means coefficients (2c, -1, -|c|^2)
    hipError_t e = launch_prologue(pl, nullptr, centroids, nullptr, st);
    const size_t esz = x_dtype == GMM_BF16 ? 2 : 4;
    for (int64_t c0 = 0, ci = 0; e == hipSuccess && c0 < n; c0 += pl.chunk, ++ci) {
        const int64_t cn = n - c0 < pl.chunk ? n - c0 : pl.chunk;
        const void* xc = (const char*)x + (size_t)c0 * (size_t)ldx * esz;
        // without an output array the chunk's assignments live in the
        // normaliser scratch (CHUNK_ROWS doubles hold CHUNK_ROWS int32)
        int32_t* zc = assign_dev ? assign_dev + c0 : (int32_t*)pl.lse;
        prof_mark(1, true, st);
        e = pl.wide ? launch_wide_lse(pl, xc, cn, ldx, x_dtype, nullptr, ci > 0, 1, zc, nullptr, st, 1)
                    : launch_lse(pl, xc, cn, ldx, x_dtype, nullptr, ci > 0, 1, zc, nullptr, st, 1);
        prof_mark(1, false, st);
        if (e != hipSuccess) break;
        prof_mark(2, true, st);
        e = pl.wide ? launch_wide_km_stats(pl, xc, cn, ldx, x_dtype, zc, ci > 0, st)
                    : launch_km_stats(pl, xc, cn, ldx, x_dtype, zc, ci > 0, st);
        prof_mark(2, false, st);
    }
    if (e == hipSuccess) e = launch_ll_final(pl, ll_parts(pl, n), inertia_dev ? inertia_dev : pl.ll_tmp, st, -1.0);
    if (e == hipSuccess) e = launch_kmfinal(pl, centroids, st);
    return hip_status(e);
}

int gmm_kmeans_fit(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                   float* centroids, int32_t k, int32_t max_iter, double tol,
                   double* inertia_hist_dev, int32_t* iters_done, void* workspace,
                   size_t workspace_bytes, void* stream) {
    if (max_iter < 0 || !(tol >= 0.0) || !isfinite(tol)) return GMM_E_INVALID;
    hipStream_t st = (hipStream_t)stream;
    double prev = 0.0;
    int done = 0, rc = GMM_OK;
    for (int it = 0; it < max_iter; ++it) {
        double* in = inertia_hist_dev ? inertia_hist_dev + it : nullptr;
        double* tmp = nullptr;
        if (!in && tol > 0.0) {
            Plan pl;
            if (!make_plan(d, k, workspace, &pl)) return GMM_E_UNSUPPORTED;
            tmp = pl.ll_tmp;  // (checked by gmm_kmeans_step below)
        }
        rc = gmm_kmeans_step(x, n, d, ldx, x_dtype, centroids, k, nullptr, in ? in : tmp,
                             workspace, workspace_bytes, stream);
        if (rc) break;
        ++done;
        if (tol > 0.0) {
            double cur = 0.0;
            if (hipMemcpyAsync(&cur, in ? in : tmp, sizeof(double), hipMemcpyDeviceToHost, st) !=
                    hipSuccess ||
                hipStreamSynchronize(st) != hipSuccess) {
                rc = GMM_E_HIP;
                break;
            }
            if (it > 0 && prev - cur < tol * cur) break;
            prev = cur;
        }
    }
    if (iters_done) *iters_done = done;
    return rc;
}

int gmm_device_status(const void* workspace, void* stream) {
    if (!workspace) return GMM_E_INVALID;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return GMM_E_HIP;
    int st2[4] = {0, 0, 0, 0};
    if (hipMemcpy(st2, workspace, sizeof(st2), hipMemcpyDeviceToHost) != hipSuccess) return GMM_E_HIP;
    if (st2[2] != 0) return GMM_E_SYNC;
    return (st2[0] != 0 || st2[1] == 0) ? GMM_E_PARAMS : GMM_OK;
}

const char* gmm_status_string(int status) {
    switch (status) {
        case GMM_OK: return "ok";
        case GMM_E_INVALID: return "invalid argument";
        case GMM_E_DTYPE: return "unsupported data type";
        case GMM_E_WORKSPACE: return "workspace missing, misaligned or too small";
        case GMM_E_PARAMS: return "invalid parameter values";
        case GMM_E_HIP: return "HIP runtime error";
        case GMM_E_UNSUPPORTED: return "shape or schedule not supported by this build or device";
        case GMM_E_SYNC: return "cooperative exchange between workgroups timed out";
        default: return "unknown status";
    }
}

int gmm_profile_begin(int32_t max_launches) {
    if (max_launches < 1 || max_launches > (1 << 16)) return GMM_E_INVALID;
    if (g_prof.cap < max_launches) {
        hipEvent_t* e1 = new (std::nothrow) hipEvent_t[2 * max_launches];
        hipEvent_t* e2 = new (std::nothrow) hipEvent_t[2 * max_launches];
        if (!e1 || !e2) {
            delete[] e1;
            delete[] e2;
            return GMM_E_INVALID;
        }
        for (int i = 0; i < 2 * g_prof.cap; ++i) {
            (void)hipEventDestroy(g_prof.ev1[i]);
            (void)hipEventDestroy(g_prof.ev2[i]);
        }
        delete[] g_prof.ev1;
        delete[] g_prof.ev2;
        g_prof.ev1 = e1;
        g_prof.ev2 = e2;
        for (int i = 0; i < 2 * max_launches; ++i) {
            if (hipEventCreate(&e1[i]) != hipSuccess || hipEventCreate(&e2[i]) != hipSuccess) {
                g_prof.cap = 0;
                return GMM_E_HIP;
            }
        }
        g_prof.cap = max_launches;
    }
    g_prof.n1 = g_prof.n2 = 0;
    g_prof.on = true;
    return GMM_OK;
}

int gmm_profile_end(double* ms1, int32_t* n1, double* ms2, int32_t* n2) {
    g_prof.on = false;
    double t1 = 0.0, t2 = 0.0;
    for (int i = 0; i < g_prof.n1; ++i) {
        float ms = 0.0f;
        if (hipEventSynchronize(g_prof.ev1[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_prof.ev1[2 * i], g_prof.ev1[2 * i + 1]) != hipSuccess)
            return GMM_E_HIP;
        t1 += ms;
    }
    for (int i = 0; i < g_prof.n2; ++i) {
        float ms = 0.0f;
        if (hipEventSynchronize(g_prof.ev2[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_prof.ev2[2 * i], g_prof.ev2[2 * i + 1]) != hipSuccess)
            return GMM_E_HIP;
        t2 += ms;
    }
    if (ms1) *ms1 = t1;
    if (n1) *n1 = g_prof.n1;
    if (ms2) *ms2 = t2;
    if (n2) *n2 = g_prof.n2;
    return GMM_OK;
}

int32_t gmm_version(void) { return 100; }

}  // extern "C"
