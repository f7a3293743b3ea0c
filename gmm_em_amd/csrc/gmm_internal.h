// gmm_internal.h - host-side plan shared by the C ABI and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gmm {

// Largest padded dimension of the narrow kernels (features or coefficients of
// a K-tile in registers); wider data uses the D-sliced wide kernels, whose
// padded dimension is a multiple of 128 up to WIDE_MAX_DP (16 rows of fp64
// values in LDS).
constexpr int MAX_DP = 128;
constexpr int WIDE_MAX_DP = 768;
// Rows per chunk of the wide path (bounds its per-(row, K-tile) partials).
constexpr int64_t WIDE_CHUNK_ROWS = 4096;
// Top-m candidates kept per (row, K-tile) by the wide normaliser pass.
constexpr int WIDE_TM = 4;
// Rows per chunk: bounds the per-row normaliser scratch (lse) so that the
// workspace size does not depend on the number of rows.
constexpr int64_t CHUNK_ROWS = (int64_t)1 << 22;
// Largest leading dimension (elements): 32 rows of fp32 values must span
// fewer than 2^31 bytes (the statistics pass's per-tile buffer offsets).
constexpr int64_t MAX_LDX = ((int64_t)1 << 24) - 1;
// Rows per normaliser-pass block (one log-likelihood partial each).
constexpr int LL_ROWS = 64;

// Workspace layout and launch geometry for one (d, k).
struct Plan {
    int d = 0, dp = 0;         // data dimension and its padding to a multiple of 16
    int k = 0, kp = 0;         // components and their padding to a multiple of 128
    int ntiles = 0;            // 16-component K-tiles (kp / 16)
    int ngroups = 0;           // row groups of the statistics pass
    size_t bytes = 0;          // workspace bytes
    // device pointers (null when planning sizes only)
    int* status = nullptr;     // [0]: invalid-parameter flag, [1]: some weight > 0
    double* shift = nullptr;   // [dp] per-dim shift, permuted dim order
    double* Pg = nullptr;      // [kp][2*dp] coefficient rows, MFMA operand order
    double* cvec = nullptr;    // [kp] per-component constants
    double* lse = nullptr;     // [CHUNK_ROWS] per-row normaliser of the current chunk
    double* llpart = nullptr;  // [CHUNK_ROWS / LL_ROWS] log-likelihood partials
    double* npart = nullptr;   // [ngroups][kp] responsibility mass partials
    double* part = nullptr;    // [ngroups][kp][2*dp] first/second moment partials
    double* ll_tmp = nullptr;  // [1] scratch total
    int kgroups = 0;           // K-groups of the statistics pass (blocks per row group)
    bool wide = false;         // dp > MAX_DP: the D-sliced wide kernels
    int64_t chunk = 0;         // rows per chunk (CHUNK_ROWS or WIDE_CHUNK_ROWS)
    double2* wlpart = nullptr; // wide: [chunk][ntiles] per-(row, K-tile) (max, sum)
    double* wtval = nullptr;   // wide: [chunk][ntiles][WIDE_TM] top-m candidate values
    int32_t* wtidx = nullptr;  // wide: [chunk][ntiles][WIDE_TM] candidate components
};

bool make_plan(int d, int k, void* ws, Plan* pl);

hipError_t launch_prologue(const Plan& pl, const float* w, const float* mu, const float* var,
                           hipStream_t st);
// lse_out may be null (normalisers not kept); m > 0 also writes the top-m
// components (idx, resp, row-major n x m) of each row.
// km (k-means mode, with m = 1): the row value summed into the partials is
// the best log-density instead of the normaliser.
hipError_t launch_lse(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                      double* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                      hipStream_t st, int km = 0);
hipError_t launch_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                        const double* lse, int acc, hipStream_t st);
hipError_t launch_finalize(const Plan& pl, int groups, int64_t n, float var_floor, float* w,
                           float* mu, float* var, hipStream_t st);
// Wide path (pl.wide): normaliser partials + merge (writes lse_out, the
// log-likelihood partials and, with m > 0, the top-m outputs), and the
// statistics pass.
hipError_t launch_wide_lse(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                           double* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                           hipStream_t st, int km = 0);
hipError_t launch_wide_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                             const double* lse, int acc, hipStream_t st);
// k-means statistics of the wide path (one dim slice per wave)
hipError_t launch_wide_km_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                                const int32_t* z, int acc, hipStream_t st);
int waves_per_stats_block(int dp);
hipError_t launch_ll_final(const Plan& pl, int nparts, double* out, hipStream_t st,
                           double scale = 1.0);
// k-means statistics: per (row group, K-tile) sums of x - s and counts of the
// rows assigned (z) to each centroid, in the statistics partials' layout.
hipError_t launch_km_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                           const int32_t* z, int acc, hipStream_t st);
// k-means centroid update from the statistics partials.
hipError_t launch_kmfinal(const Plan& pl, float* c, hipStream_t st);

}  // namespace gmm
