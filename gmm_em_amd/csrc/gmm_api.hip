// gmm_api.hip - the C ABI declared in include/gmm_em.h: argument checks,
// workspace planning and the launch sequence of each entry point.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <new>

#include "gmm_em.h"
#include "gmm_internal.h"

namespace gmm {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool make_plan(int d, int k, void* ws, Plan* pl, int64_t chunk_rows, int max_groups, int64_t b16_rows) {
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
    p.ngroups = g < 1 ? 1 : (g > max_groups ? max_groups : g);
    p.chunk = p.wide ? WIDE_CHUNK_ROWS : chunk_rows;
    // per-row scratch: the narrow chunk, and at least the wide chunk
    const int64_t srows = chunk_rows > WIDE_CHUNK_ROWS ? chunk_rows : WIDE_CHUNK_ROWS;
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
    const size_t o_lse = take((size_t)srows * sizeof(double));
    const size_t o_ll = take((size_t)(srows / LL_ROWS) * sizeof(double));
    const size_t o_np = take((size_t)p.ngroups * p.kp * sizeof(double));
    const size_t o_part = take((size_t)p.ngroups * p.kp * 2 * p.dp * sizeof(double));
    const size_t o_lt = take(sizeof(double));
    const bool i8 = !p.wide;  // the int8-slice E-step serves the narrow path
    const size_t o_ia = take(i8 ? MAX_DP * sizeof(unsigned long long) : 0);
    const size_t o_il = take(i8 ? MAX_DP * sizeof(int) : 0);
    const size_t o_ip = take(i8 ? I8P_SIZE * sizeof(int) : 0);
    const size_t o_id = take(i8 ? sizeof(double) : 0);
    const size_t o_ic = take(i8 ? (size_t)p.ntiles * I8_MAX_LEV * I8_MAX_NC * 1024 : 0);
    const size_t o_ie = take(i8 ? (size_t)p.kp * sizeof(int) : 0);
    const size_t o_it = take(i8 ? (size_t)p.ntiles * I8_TINFO * sizeof(int) : 0);
    p.i8_nc = i8 ? i8_nc_for(d) : 0;
    p.i8_stats = i8 && i8_stats_for(p.dp);
    // one region for the int8 pass's packed digit rows and the split-bf16
    // statistics pass's operand pieces (a call uses one of them)
    p.b16_chunk = i8 ? (b16_rows < chunk_rows ? b16_rows : chunk_rows) : 0;
    const size_t rows8 = p.i8_stats ? (size_t)chunk_rows * S8_FLG : 0;
    const size_t rows16 = (size_t)p.b16_chunk * B16_PIECE_ROW_BYTES * (size_t)((d + 31) / 32);
    const size_t o_ir = take(rows8 > rows16 ? rows8 : rows16);
    const size_t o_bc = take(i8 ? (size_t)p.ntiles * B16_TILE_BYTES : 0);
    const size_t o_bv = take(i8 ? (size_t)p.kp * sizeof(double) : 0);
    const size_t o_ba = take(i8 ? MAX_DP * sizeof(unsigned long long) : 0);
    const size_t o_bl = take(i8 ? MAX_DP * sizeof(int) : 0);
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
        if (i8) {
            p.i8_amax = (unsigned long long*)(b + o_ia);
            p.i8_lsb = (int*)(b + o_il);
            p.i8_plan = (int*)(b + o_ip);
            p.i8_dbl = (double*)(b + o_id);
            p.i8_coef = (int8_t*)(b + o_ic);
            p.i8_ek = (int*)(b + o_ie);
            p.i8_tinfo = (int*)(b + o_it);
            if (p.i8_stats) p.i8_rows = (int8_t*)(b + o_ir);
            p.b16_pieces = (uint32_t*)(b + o_ir);
            p.b16_coef = (uint16_t*)(b + o_bc);
            p.b16_cvec = (double*)(b + o_bv);
            p.b16_amax = (unsigned long long*)(b + o_ba);
            p.b16_lsb = (int*)(b + o_bl);
        }
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
// This is the library's only process-wide state: a measurement aid outside
// the compute calls' re-entrancy promise. A mutex keeps concurrent calls from
// corrupting it; the events exist only between begin and end.
struct Prof {
    bool on = false;
    int cap = 0;
    int n1 = 0, n2 = 0;
    hipEvent_t* ev1 = nullptr;  // [2*cap] start/stop pairs, pass 1
    hipEvent_t* ev2 = nullptr;  // [2*cap] pass 2
};
static Prof g_prof;
static std::mutex g_prof_mu;

static void prof_release() {
    for (int i = 0; i < 2 * g_prof.cap; ++i) {
        if (g_prof.ev1 && g_prof.ev1[i]) (void)hipEventDestroy(g_prof.ev1[i]);
        if (g_prof.ev2 && g_prof.ev2[i]) (void)hipEventDestroy(g_prof.ev2[i]);
    }
    delete[] g_prof.ev1;
    delete[] g_prof.ev2;
    g_prof = Prof();
}

static void prof_mark(int pass, bool start, hipStream_t st) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
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
// receives every row's normaliser instead of the chunk scratch. With i8 (the
// int8-slice prologue has run), pass 1 is the int8-slice kernel when the
// prologue selected it.
// Rows per chunk of run_passes: an EM step on bf16 data on the narrow path
// takes the split-bf16 statistics pass's chunk (its operand pieces fill the
// workspace region for that many rows).
static int64_t chunk_for(const Plan& pl, int dtype, bool stats) {
    return stats && dtype == GMM_BF16 && !pl.wide ? pl.b16_chunk : pl.chunk;
}

static hipError_t run_passes(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                             bool stats, hipStream_t st, int m = 0, int32_t* idx = nullptr,
                             float* resp = nullptr, double* lse_rows = nullptr,
                             bool i8 = false) {
    const size_t esz = dtype == GMM_BF16 ? 2 : 4;
    const int64_t chunk = chunk_for(pl, dtype, stats);
    for (int64_t c0 = 0, ci = 0; c0 < n; c0 += chunk, ++ci) {
        const int64_t cn = n - c0 < chunk ? n - c0 : chunk;
        const void* xc = (const char*)x + (size_t)c0 * (size_t)ldx * esz;
        double* lse = lse_rows ? lse_rows + c0 : pl.lse;
        int32_t* ic = m > 0 ? idx + c0 * m : nullptr;
        float* rc = m > 0 ? resp + c0 * m : nullptr;
        prof_mark(1, true, st);
        hipError_t e = hipSuccess;
        if (pl.wide) {
            e = launch_wide_lse(pl, xc, cn, ldx, dtype, lse, ci > 0, m, ic, rc, st);
        } else if (i8) {
            // every variant is launched; the mode flag the prologue wrote
            // lets exactly one of them do the work
            if (m > 0) {  // top-m lists (fp32 rows)
                e = launch_lse8_topm(pl, xc, cn, ldx, lse, ci > 0, m, ic, rc, st);
            } else {
                e = launch_lse8(pl, xc, cn, ldx, dtype, lse, ci > 0, st);
                if (e == hipSuccess && dtype == GMM_BF16)
                    e = launch_lse16(pl, xc, cn, ldx, lse, ci > 0, stats, st);
            }
            if (e == hipSuccess)
                e = launch_lse(pl, xc, cn, ldx, dtype, lse, ci > 0, m, ic, rc, st, 0,
                               pl.status + I8S_MODE);
        } else {
            e = launch_lse(pl, xc, cn, ldx, dtype, lse, ci > 0, m, ic, rc, st);
        }
        prof_mark(1, false, st);
        if (e != hipSuccess) return e;
        if (stats) {
            prof_mark(2, true, st);
            if (pl.wide) {
                e = launch_wide_stats(pl, xc, cn, ldx, dtype, lse, ci > 0, st);
            } else if (i8) {
                // as for pass 1: the mode flag lets one of them work
                if (pl.i8_stats) e = launch_stats8(pl, xc, cn, ldx, dtype, lse, ci > 0, st);
                if (e == hipSuccess && dtype == GMM_BF16)
                    e = launch_stats16(pl, cn, lse, ci > 0, st);
                if (e == hipSuccess)
                    e = launch_stats(pl, xc, cn, ldx, dtype, lse, ci > 0, st, pl.status + I8S_MODE2);
            } else {
                e = launch_stats(pl, xc, cn, ldx, dtype, lse, ci > 0, st);
            }
            prof_mark(2, false, st);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

static int ll_parts(const Plan& pl, int64_t n, int64_t chunk) {
    const int64_t first = n < chunk ? n : chunk;
    return (int)((first + LL_ROWS - 1) / LL_ROWS);
}

// The launch sequence of one EM step on a planned workspace.
static int em_step_planned(const Plan& pl, const void* x, int64_t n, int64_t ldx, int x_dtype,
                           float* weights, float* means, float* variances, float var_floor,
                           double* loglik_dev, hipStream_t st) {
    double* ll_out = loglik_dev ? loglik_dev : pl.ll_tmp;
    hipError_t e = launch_prologue(pl, weights, means, variances, st);
    if (e == hipSuccess && !pl.wide)
        e = launch_i8_prologue(pl, weights, means, variances, x, n, ldx, x_dtype, st);
    if (e != hipSuccess) return GMM_E_HIP;
    e = run_passes(pl, x, n, ldx, x_dtype, true, st, 0, nullptr, nullptr, nullptr, !pl.wide);
    if (e == hipSuccess) e = launch_ll_final(pl, ll_parts(pl, n, chunk_for(pl, x_dtype, true)), ll_out, st);
    if (e == hipSuccess) e = launch_finalize(pl, pl.ngroups, n, var_floor, weights, means, variances, st);
    return hip_status(e);
}

// Device scratch of the allocation-free EM step: one copy per GPU, held for
// the life of the process, shared by every gmm_em_step_noalloc call on that
// GPU. Host code never passes this symbol to a kernel (on the host it is only
// a stand-in): scratch_address() looks up the device address once per device,
// with that device current, and every use goes through that address.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
constexpr int SCRATCH_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[SCRATCH_MAX_DEVICES];

static int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GMM_E_HIP;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return GMM_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GMM_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GMM_OK;
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
    return em_step_planned(pl, x, n, ldx, x_dtype, weights, means, variances, var_floor, loglik_dev,
                           (hipStream_t)stream);
}

int gmm_em_step_noalloc(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                        float* weights, float* means, float* variances, int32_t k, float var_floor,
                        double* loglik_dev, void* stream) {
    if (n < 0 || d < 1 || k < 1 || ldx < d) return GMM_E_INVALID;
    if (ldx > MAX_LDX) return GMM_E_UNSUPPORTED;
    if ((n > 0 && !x) || !weights || !means || !variances) return GMM_E_INVALID;
    if (x_dtype != GMM_F32 && x_dtype != GMM_BF16) return GMM_E_DTYPE;
    if (n < 1 || !(var_floor >= 0.0f) || !isfinite(var_floor)) return GMM_E_INVALID;
    // the plan with the scratch's row chunk, and as many statistics row
    // groups as fit the scratch
    Plan pl;
    int groups = 512;
    for (;;) {
        if (!make_plan(d, k, nullptr, &pl, NOALLOC_CHUNK_ROWS, groups, NOALLOC_B16_CHUNK_ROWS))
            return GMM_E_UNSUPPORTED;
        if (pl.bytes <= NOALLOC_SCRATCH_BYTES) break;
        if (groups == 1) return GMM_E_UNSUPPORTED;  // (d, k) too large for the scratch
        groups = groups / 2 > 1 ? groups / 2 : 1;
    }
    void* scr = nullptr;
    const int rc = scratch_address(&scr);
    if (rc) return rc;
    make_plan(d, k, scr, &pl, NOALLOC_CHUNK_ROWS, groups, NOALLOC_B16_CHUNK_ROWS);
    return em_step_planned(pl, x, n, ldx, x_dtype, weights, means, variances, var_floor, loglik_dev,
                           (hipStream_t)stream);
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
    if (e == hipSuccess && !pl.wide)
        e = launch_i8_prologue(pl, weights, means, variances, x, n, ldx, x_dtype, st);
    if (e == hipSuccess)
        e = run_passes(pl, x, n, ldx, x_dtype, false, st, 0, nullptr, nullptr, per_row_dev,
                       !pl.wide);
    if (e == hipSuccess) e = launch_ll_final(pl, ll_parts(pl, n, pl.chunk), total_dev, st);
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
    // the int8-slice pass with top-m lists serves fp32 rows up to 128 dims
    // (where its error bound holds; the fp64 pass otherwise)
    const bool i8 = !pl.wide && x_dtype == GMM_F32;
    if (e == hipSuccess && i8)
        e = launch_i8_prologue(pl, weights, means, variances, x, n, ldx, x_dtype, st, false);
    if (e == hipSuccess)
        e = run_passes(pl, x, n, ldx, x_dtype, false, st, m, idx_dev, resp_dev, nullptr, i8);
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
    // weights and variances null: the k-means coefficients (2c, -1, -|c|^2);
    // the distances on int8 slices where they are exact, as for the EM step
    hipError_t e = launch_prologue(pl, nullptr, centroids, nullptr, st);
    if (e == hipSuccess && !pl.wide)
        e = launch_i8_prologue(pl, nullptr, centroids, nullptr, x, n, ldx, x_dtype, st, false);
    const size_t esz = x_dtype == GMM_BF16 ? 2 : 4;
    for (int64_t c0 = 0, ci = 0; e == hipSuccess && c0 < n; c0 += pl.chunk, ++ci) {
        const int64_t cn = n - c0 < pl.chunk ? n - c0 : pl.chunk;
        const void* xc = (const char*)x + (size_t)c0 * (size_t)ldx * esz;
        // without an output array the chunk's assignments live in the
        // normaliser scratch (CHUNK_ROWS doubles hold CHUNK_ROWS int32)
        int32_t* zc = assign_dev ? assign_dev + c0 : (int32_t*)pl.lse;
        prof_mark(1, true, st);
        if (pl.wide) {
            e = launch_wide_lse(pl, xc, cn, ldx, x_dtype, nullptr, ci > 0, 1, zc, nullptr, st, 1);
        } else {
            // both variants; the mode flag lets one of them work
            e = launch_lse8_km(pl, xc, cn, ldx, x_dtype, zc, ci > 0, st);
            if (e == hipSuccess)
                e = launch_lse(pl, xc, cn, ldx, x_dtype, nullptr, ci > 0, 1, zc, nullptr, st, 1,
                               pl.status + I8S_MODE);
        }
        prof_mark(1, false, st);
        if (e != hipSuccess) break;
        prof_mark(2, true, st);
        e = pl.wide ? launch_wide_km_stats(pl, xc, cn, ldx, x_dtype, zc, ci > 0, st)
                    : launch_km_stats(pl, xc, cn, ldx, x_dtype, zc, ci > 0, st);
        prof_mark(2, false, st);
    }
    if (e == hipSuccess) e = launch_ll_final(pl, ll_parts(pl, n, pl.chunk), inertia_dev ? inertia_dev : pl.ll_tmp, st, -1.0);
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
    return (st2[0] != 0 || st2[1] == 0) ? GMM_E_PARAMS : GMM_OK;
}

int gmm_estep_arithmetic(const void* workspace, void* stream) {
    if (!workspace) return -1;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return -1;
    int st2[16] = {0};
    if (hipMemcpy(st2, workspace, sizeof(st2), hipMemcpyDeviceToHost) != hipSuccess) return -1;
    if (st2[I8S_MODE] == MODE1_B16) return GMM_ESTEP_BF16_SPLIT;
    if (st2[I8S_MODE] != 1) return GMM_ESTEP_FP64;
    if (st2[I8S_MODE2] == 2) return GMM_ESTEP_INT8_SLICES_MSTEP;
    return st2[I8S_MODE2] == 1 ? GMM_ESTEP_INT8_SLICES_BOTH : GMM_ESTEP_INT8_SLICES;
}

const char* gmm_status_string(int status) {
    switch (status) {
        case GMM_OK: return "ok";
        case GMM_E_INVALID: return "invalid argument";
        case GMM_E_DTYPE: return "unsupported data type";
        case GMM_E_WORKSPACE: return "workspace missing, misaligned or too small";
        case GMM_E_PARAMS: return "invalid parameter values";
        case GMM_E_HIP: return "HIP runtime error";
        case GMM_E_UNSUPPORTED: return "shape not supported by this build";
        default: return "unknown status";
    }
}

int gmm_profile_begin(int32_t max_launches) {
    if (max_launches < 1 || max_launches > (1 << 16)) return GMM_E_INVALID;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    prof_release();
    g_prof.ev1 = new (std::nothrow) hipEvent_t[2 * max_launches]();
    g_prof.ev2 = new (std::nothrow) hipEvent_t[2 * max_launches]();
    g_prof.cap = max_launches;
    if (!g_prof.ev1 || !g_prof.ev2) {
        prof_release();
        return GMM_E_INVALID;
    }
    for (int i = 0; i < 2 * max_launches; ++i) {
        if (hipEventCreate(&g_prof.ev1[i]) != hipSuccess ||
            hipEventCreate(&g_prof.ev2[i]) != hipSuccess) {
            prof_release();
            return GMM_E_HIP;
        }
    }
    g_prof.on = true;
    return GMM_OK;
}

int gmm_profile_end(double* ms1, int32_t* n1, double* ms2, int32_t* n2) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof.on) return GMM_E_INVALID;
    g_prof.on = false;
    double t[2] = {0.0, 0.0};
    int rc = GMM_OK;
    for (int pass = 0; pass < 2 && rc == GMM_OK; ++pass) {
        hipEvent_t* ev = pass == 0 ? g_prof.ev1 : g_prof.ev2;
        const int cnt = pass == 0 ? g_prof.n1 : g_prof.n2;
        for (int i = 0; i < cnt; ++i) {
            float ms = 0.0f;
            if (hipEventSynchronize(ev[2 * i + 1]) != hipSuccess ||
                hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]) != hipSuccess) {
                rc = GMM_E_HIP;
                break;
            }
            t[pass] += ms;
        }
    }
    if (rc == GMM_OK) {
        if (ms1) *ms1 = t[0];
        if (n1) *n1 = g_prof.n1;
        if (ms2) *ms2 = t[1];
        if (n2) *n2 = g_prof.n2;
    }
    prof_release();
    return rc;
}

int32_t gmm_version(void) { return 100; }

}  // extern "C"
