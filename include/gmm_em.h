/*
 * gmm_em.h - C ABI of the fused diagonal-covariance GMM EM library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is one expectation-maximization (EM) iteration of a Gaussian
 * mixture with diagonal covariances, fused so that the N x K responsibility
 * matrix is never written to device memory: statistics are formed per data
 * tile and accumulated globally into O(K*D) buffers ("Flash-GMM: A
 * Memory-Efficient Kernel for Scalable Soft Clustering", section 1 for the
 * responsibility matrix, section 3 for the tiled EM with globally accumulated
 * per-tile statistics; the abstract for the use of responsibilities to assign
 * border vectors to several clusters).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Data X: device pointer, row-major, n rows of d values with a leading
 *   dimension ldx >= d (in elements, at most 2^24 - 1: GMM_E_UNSUPPORTED
 *   above), fp32 or bf16 (x_dtype). Values between d and ldx are never
 *   used (they may be read, never past the last row's d-th value).
 * Parameters: device pointers, fp32, row-major:
 *   weights[k] (mixture weights, >= 0, not all 0),
 *   means[k*d], variances[k*d] (> 0).
 * Workspace: a device buffer of at least gmm_workspace_bytes(d, k) bytes,
 *   owned by the caller. Its size does not depend on n. Calls that share a
 *   workspace must not overlap in time (use one stream, or separate
 *   workspaces).
 * Stream: a hipStream_t passed as void* (NULL = the null stream). All work is
 *   enqueued asynchronously on it; results are valid once the stream has
 *   reached them. Nothing synchronises except gmm_device_status and
 *   gmm_fit with tol > 0.
 * Errors: every function returns a gmm_status. Argument errors found on the
 *   host are returned before anything is enqueued (buffers are untouched).
 *   Invalid parameter values (non-finite, variance <= 0, negative weight,
 *   all weights zero) are detected on the device: the call still returns
 *   GMM_OK, outputs are NaN, and gmm_device_status reports GMM_E_PARAMS.
 *   No function throws or aborts.
 * Determinism: for a given device, inputs and (d, k) every output is
 *   bitwise reproducible; no floating-point atomics are used.
 * Ownership: the library allocates no device memory and keeps no state
 *   between calls besides cached device properties.
 */
#ifndef GMM_EM_H
#define GMM_EM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GMM_OK = 0,
    GMM_E_INVALID = 1,   /* bad size, pointer, stride or option */
    GMM_E_DTYPE = 2,     /* unsupported data type */
    GMM_E_WORKSPACE = 3, /* workspace missing or too small */
    GMM_E_PARAMS = 4,    /* invalid parameter values (reported by gmm_device_status) */
    GMM_E_HIP = 5,       /* a HIP runtime call failed */
    GMM_E_UNSUPPORTED = 6  /* shape outside what this build supports */
} gmm_status;

typedef enum { GMM_F32 = 0, GMM_BF16 = 1 } gmm_dtype;

/* Arithmetic of the E-step and M-step contractions (see gmm_estep_arithmetic). */
typedef enum {
    GMM_ESTEP_FP64 = 0,              /* both passes' E-step in fp64 */
    GMM_ESTEP_INT8_SLICES = 1,       /* normaliser pass on int8 slices, statistics pass fp64 */
    GMM_ESTEP_INT8_SLICES_BOTH = 2,  /* both passes' E-step on int8 slices, M-step fp64 */
    GMM_ESTEP_INT8_SLICES_MSTEP = 3, /* as 2, and the M-step on int8 slices too */
    GMM_ESTEP_BF16_SPLIT = 4         /* bf16 data: E-step and M-step on split bf16 */
} gmm_estep_kind;

/* Bytes of device workspace needed for data of dimension d and k components.
 * Independent of the number of rows. Returns 0 for unsupported shapes:
 * d <= 768 and k <= 2^22 are supported (d <= 128 uses register-tiled
 * kernels; wider rows use kernels that split the dimension over the waves of
 * a workgroup and process rows in chunks of 4096). */
size_t gmm_workspace_bytes(int32_t d, int32_t k);

/* One EM iteration (E-step, responsibilities, M-step) in place.
 *
 * Computes, for the input parameters theta = (weights, means, variances):
 *   l[n][k]  = log w[k] + log N(x_n | mu_k, diag(var_k))      (log-density)
 *   lse[n]   = log sum_k exp(l[n][k])                          (normaliser)
 *   r[n][k]  = exp(l[n][k] - lse[n])                          (responsibility)
 *   N[k] = sum_n r[n][k], S1[k] = sum_n r[n][k] x_n, S2 = sum_n r[n][k] x_n^2
 * and overwrites theta with the M-step update
 *   w'[k] = N[k]/n, mu'[k] = S1[k]/N[k], var'[k] = max(S2[k]/N[k] - mu'[k]^2, var_floor)
 * (a component with N[k] == 0 keeps its mean and variance and gets weight 0).
 * r is never stored: it lives in registers between the two contractions.
 * Schedule: two passes over the rows (normalisers, then statistics); the
 * second recomputes the log-densities instead of storing them.
 * Arithmetic: the E-step contraction sum_d (w b a - w a^2 / 2) (a = x - s,
 * b = mu - s, w = 1/var, s a per-dimension shift) runs either in fp64 or
 * exactly on int8 slices (the features and coefficients written as 7-bit
 * digits with power-of-two scales; integer products and sums are exact and
 * the digit levels are added in fp64), which differs from the fp64
 * contraction by at most 2^-20 nats per log-density plus fp64 rounding. The
 * call picks the int8 form on the device whenever its error bound holds for
 * the data and parameters at hand (always, for integer-valued data within
 * the supported range); gmm_estep_arithmetic reports which one ran. When
 * both passes use it they compute bitwise identical log-densities. The M-step
 * contraction is fp64, except where every feature is exact in its digits
 * (integer-valued data, or data on a grid of 2^-m, within the range): then
 * it runs on int8 slices as well, on responsibilities cut per 64-row block
 * and component to 42 bits below the block's largest one (fp32 precision
 * for every row within 2^-18 of it); N[k], S1[k] and S2[k] are then exact for
 * those weights up to fp64 rounding, so the variance keeps full accuracy.
 * Responsibilities keep the fp64 exponent range: a component whose
 * responsibilities are all below fp32's smallest value but above fp64's
 * still gets a nonzero N[k].
 * bf16 data (d <= 128) that the int8 form does not cover runs both passes on
 * the bf16 matrix units instead when its checks hold: a = x - s exact in
 * bf16, and 2^-23 * max_k sum_d (|w/2| amax_d^2 + |w b| amax_d) <= 2^-7
 * (amax_d the largest |a| in dimension d). Features [a^2 hi, a^2 lo, a] are
 * exact in bf16, coefficients are split in three bf16 parts, each 32-dim
 * slice accumulates in fp32 and the slices add in fp64: the log-densities
 * differ from the fp64 contraction by about 2^-24 of the slices' magnitude
 * (that estimate is what the check bounds). The M-step contracts fp32
 * responsibilities (exact as three bf16 parts; those below 2^-100 count as
 * 0) in fp32 per 32-row tile and fp64 across tiles.
 * loglik_dev (device, 1 double, may be NULL) receives sum_n lse[n] for the
 * INPUT parameters. var_floor must be finite and >= 0. n >= 1. */
int gmm_em_step(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                float* weights, float* means, float* variances, int32_t k, float var_floor,
                double* loglik_dev, void* workspace, size_t workspace_bytes, void* stream);

/* gmm_em_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same EM step with the same arguments and results, but no workspace
 * argument. It uses a device array of 128 MiB that the library holds in its
 * code object (one copy per GPU, kept until the process ends); the call
 * itself allocates nothing. The array is shared by every call on a GPU:
 * calls that overlap in time on one GPU (several streams or host threads)
 * race and give undefined results. It holds no state that a call depends on
 * (each call rewrites what it reads). Shapes whose workspace does not fit
 * 128 MiB (with its 262,144-row chunks and the statistics pass's row groups
 * reduced to fit) return GMM_E_UNSUPPORTED: d = 96 with k = 1024 fits, d = 768
 * with k = 16384 does not. The reduction order differs from gmm_em_step's,
 * so results agree to rounding, not bitwise. */
int gmm_em_step_noalloc(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                        float* weights, float* means, float* variances, int32_t k,
                        float var_floor, double* loglik_dev, void* stream);

/* max_iter EM iterations (gmm_em_step repeated). loglik_hist_dev (device,
 * max_iter doubles, may be NULL) receives L(theta_t) for t = 0, 1, ...
 * When tol > 0 the host reads each L after its step (one synchronisation per
 * iteration) and stops once L_t - L_{t-1} < tol * |L_t|. iters_done (host
 * pointer, may be NULL) receives the number of steps taken. */
int gmm_fit(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
            float* weights, float* means, float* variances, int32_t k, float var_floor,
            int32_t max_iter, double tol, double* loglik_hist_dev, int32_t* iters_done,
            void* workspace, size_t workspace_bytes, void* stream);

/* Log-likelihood of the data under the parameters (the E-step half only).
 * total_dev (device, 1 double) receives sum_n lse[n]; per_row_dev (device,
 * n doubles, may be NULL) receives lse[n]. n may be 0 (total = 0). */
int gmm_loglik(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
               const float* weights, const float* means, const float* variances, int32_t k,
               double* total_dev, double* per_row_dev, void* workspace, size_t workspace_bytes,
               void* stream);

/* Soft multi-assignment: the m components of highest responsibility for each
 * row, most responsible first (ties: smaller component index first), with
 * their responsibilities r[n][k]. idx_dev (device, n*m int32) and resp_dev
 * (device, n*m floats) are row-major n x m. 1 <= m <= min(k, 4). n may be 0.
 * The log-densities run on int8 slices for fp32 rows where gmm_em_step's
 * conditions for them hold, else in fp64 (bf16 rows: fp64).
 * Parameter errors are reported by gmm_device_status; the outputs are then
 * unspecified. */
int gmm_assign_topm(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                    const float* weights, const float* means, const float* variances, int32_t k,
                    int32_t m, int32_t* idx_dev, float* resp_dev, void* workspace,
                    size_t workspace_bytes, void* stream);

/* One Lloyd (k-means) step, the hard-assignment quantizer that the Flash-GMM
 * pages compare the GMM against in the IVF coarse quantizer ("Flash-GMM: A
 * Memory-Efficient Kernel for Scalable Soft Clustering", section 3). It is
 * the EM step's limit for equal weights and equal spherical variances
 * shrinking to zero, and runs on the same two passes:
 *   z[n]  = argmin_k |x_n - c_k|^2       (ties: smaller k)
 *   c'_k  = mean of the rows with z = k  (c_k kept when no row has z = k)
 * centroids (device, k x d floats, row-major) is read and overwritten with c'.
 * assign_dev (device, n int32, may be NULL) receives z. inertia_dev (device,
 * 1 double, may be NULL) receives sum_n |x_n - c_z[n]|^2 for the INPUT
 * centroids. The distances use the expanded form 2 a.b - a.a - b.b about a
 * per-dimension shift, in fp64 or, where the data and centroids allow it (as
 * for gmm_em_step: the int8 slices' error bound holds), on exact int8 slices
 * (exact up to fp64 rounding either way), so rows whose two nearest
 * centroids are within rounding of each other may be assigned either one.
 * The workspace is the one for (d, k). n >= 1; d <= 768 (GMM_E_UNSUPPORTED
 * otherwise). A non-finite centroid is reported by gmm_device_status and
 * turns the outputs into NaN. */
int gmm_kmeans_step(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                    float* centroids, int32_t k, int32_t* assign_dev, double* inertia_dev,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Inverted lists of an IVF coarse quantizer from top-m soft assignments: the
 * GMM responsibilities put border vectors in several lists ("Flash-GMM: A
 * Memory-Efficient Kernel for Scalable Soft Clustering", abstract; the
 * review page, section 1, for the IVF index). idx_dev and resp_dev (device,
 * n*m int32 and floats, row-major n x m, most responsible first, as
 * gmm_assign_topm writes them). Row r goes to list idx[r][0] and, for
 * j >= 1, to list idx[r][j] when resp[r][j] >= min_resp; ids outside [0, k)
 * are skipped. resp_dev may be NULL: then every entry is kept and the
 * stored values are 1. Output (device): offsets_dev (k+1 int64; list c is
 * entries offsets[c] .. offsets[c+1]-1, offsets[k] = entries stored),
 * rows_dev (int32 row ids, capacity n*m; each list in increasing row order)
 * and values_dev (the entries' responsibilities, capacity n*m, may be NULL).
 * The result does not depend on scheduling (a stable counting sort).
 * 1 <= k <= 16384 and n*m < 2^31 (GMM_E_UNSUPPORTED otherwise); min_resp
 * must not be NaN. The workspace (device, 256-byte aligned) has
 * gmm_ivf_workspace_bytes(n, m, k) bytes; it depends on n. */
size_t gmm_ivf_workspace_bytes(int64_t n, int32_t m, int32_t k);
int gmm_ivf_build(const int32_t* idx_dev, const float* resp_dev, int64_t n, int32_t m, int32_t k,
                  float min_resp, int64_t* offsets_dev, int32_t* rows_dev, float* values_dev,
                  void* workspace, size_t workspace_bytes, void* stream);

/* max_iter Lloyd steps (gmm_kmeans_step repeated) on the centroids in place.
 * inertia_hist_dev (device, max_iter doubles, may be NULL) receives the
 * inertia of the centroids entering step t, t = 0, 1, ... When tol > 0 the
 * host reads each inertia after its step (one synchronisation per step) and
 * stops once I_{t-1} - I_t < tol * I_t. iters_done (host pointer, may be
 * NULL) receives the number of steps taken. */
int gmm_kmeans_fit(const void* x, int64_t n, int32_t d, int64_t ldx, int32_t x_dtype,
                   float* centroids, int32_t k, int32_t max_iter, double tol,
                   double* inertia_hist_dev, int32_t* iters_done, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Synchronises the stream and returns GMM_E_PARAMS if the last call that used
 * this workspace found invalid parameter values, GMM_OK otherwise, or
 * GMM_E_HIP if the synchronisation failed. */
int gmm_device_status(const void* workspace, void* stream);

/* Synchronises the stream and returns the gmm_estep_kind of the last call
 * that used this workspace: of the E-step of gmm_em_step / gmm_fit /
 * gmm_loglik, of the distance pass of gmm_kmeans_step / gmm_kmeans_fit, or of
 * the log-densities of gmm_assign_topm (the last two report
 * GMM_ESTEP_INT8_SLICES when they ran on int8 slices, else GMM_ESTEP_FP64;
 * rows wider than 128 always run in fp64), or -1 if the workspace is NULL or
 * the synchronisation failed. */
int gmm_estep_arithmetic(const void* workspace, void* stream);

/* Static description of a status code. */
const char* gmm_status_string(int status);

/* Measurement hook (not part of the method). gmm_profile_begin(max_launches)
 * creates 4 * max_launches HIP events (host objects; no device memory) and
 * starts recording them on the calling entry point's stream around every
 * normaliser-pass (pass 1) and statistics-pass (pass 2) launch of the calls
 * that follow, up to max_launches of each. gmm_profile_end() synchronises
 * those events, returns the summed milliseconds and launch counts of each
 * pass, stops recording and destroys the events (GMM_E_INVALID if no
 * recording is active). This recording is the library's only process-wide
 * state: it is guarded by a mutex, but it is outside the re-entrancy promise
 * above (calls on several streams between begin and end are all recorded
 * into the same totals). Meant for benchmarks. */
int gmm_profile_begin(int32_t max_launches);
int gmm_profile_end(double* ms_pass1, int32_t* launches_pass1, double* ms_pass2,
                    int32_t* launches_pass2);

/* Library version as major*10000 + minor*100 + patch. */
int32_t gmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GMM_EM_H */
