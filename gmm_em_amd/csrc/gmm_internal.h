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
// Allocation-free EM step: bytes of its per-device scratch and the row chunk
// its plan uses.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)128 << 20;
constexpr int64_t NOALLOC_CHUNK_ROWS = (int64_t)1 << 18;
// Largest leading dimension (elements): 32 rows of fp32 values must span
// fewer than 2^31 bytes (the statistics pass's per-tile buffer offsets).
constexpr int64_t MAX_LDX = ((int64_t)1 << 24) - 1;
// Rows per normaliser-pass block (one log-likelihood partial each).
constexpr int LL_ROWS = 64;
// Rows per staged tile of the statistics passes (two 16-row MFMA blocks).
constexpr int STATS_ROWS = 32;

// E-step on exact int8 slices (gmm_i8.hip). Digits per feature column kind
// (a, a^2), coefficient digits (8 hold an fp64 value exactly), levels
// i + j = 2 .. I + J, 64-byte chunks per packed row, truncation bound (nats).
constexpr int I8_MAX_DIGITS = 3;
constexpr int I8_MAX_J = 8;
constexpr int I8_MAX_LEV = I8_MAX_DIGITS + I8_MAX_J - 1;
constexpr int I8_MAX_NC = 6;
constexpr double I8_DELTA = 9.5367431640625e-07;  // 2^-20
// per tile: the number of levels (a tile's operands are levels x chunks
// pieces of 1 KB)
constexpr int I8_TINFO = 1;
// plan[] indices: digit counts, truncation flags, per-dim scale exponents
constexpr int I8P_IA = 0, I8P_IB = 1, I8P_TRUNC_A = 2, I8P_TRUNC_B = 3, I8P_GA = 8,
              I8P_GB = 8 + MAX_DP, I8P_SIZE = 8 + 2 * MAX_DP;
// status word slots: [0] invalid parameters, [1] some weight > 0,
// [4] int8 path selected for this call, [5] int8 path not applicable,
// [6] non-finite data value seen by the data pass
constexpr int I8S_MODE = 4, I8S_FAIL = 5, I8S_NONFINITE = 6;
// [7] int8 statistics pass selected, [8] largest level count over the tiles
constexpr int I8S_MODE2 = 7, I8S_MAXLEV = 8;
// Mode values: status[I8S_MODE] 0 = fp64 pass 1, 1 = int8 slices, 2 = split
// bf16; status[I8S_MODE2] 0 = fp64 statistics, 1 = int8 E-step + fp64
// M-step, 2 = int8 E-step and M-step, 3 = split bf16 E-step and M-step.
constexpr int MODE1_B16 = 2, MODE2_B16 = 3;
// [9] split-bf16 path not applicable (data or coefficients out of range, or
// its rounding estimate above B16_DELTA)
constexpr int I8S_B16FAIL = 9;

// E-step and M-step on split bf16 (gmm_b16.hip), for bf16 data with d <= 128:
// 32-dim slices (d padded to DQ = 32 * dc), eight bf16 products per slice,
// one 1 KB MFMA operand piece per (slice, product) and K-tile.
constexpr int B16_MAX_DC = 4;
constexpr int B16_PROD = 8;
constexpr int B16_TILE_BYTES = B16_MAX_DC * B16_PROD * 1024;
// The statistics pass's operand pieces of one row: 12 dc pieces of 1 KB per
// 32-row tile (E and M layouts of the three feature kinds), written by the
// normaliser pass for chunks of B16_CHUNK_ROWS rows (the allocation-free
// entry point: NOALLOC_B16_CHUNK_ROWS).
constexpr int B16_PIECE_ROW_BYTES = 12 * 1024 / 32;  // per row and 32-dim slice
constexpr int64_t B16_CHUNK_ROWS = (int64_t)1 << 20;
constexpr int64_t NOALLOC_B16_CHUNK_ROWS = (int64_t)1 << 14;
// accepted estimate of the fp32 rounding of a log-density (nats): 2^-7
constexpr double B16_DELTA = 0.0078125;
// The statistics pass keeps a K-tile's digit levels in registers: at most
// S8_LV levels of S8_NC chunks; rows of packed digits are handed from the
// normaliser pass through the workspace with this stride (bytes), and the
// statistics pass runs for padded dimensions up to S8_MAX_DP (LDS).
constexpr int S8_NC = 5, S8_LV = 9;
constexpr int S8_FLG = S8_NC * 64 + 16;
constexpr int S8_MAX_DP = 112;

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
    // int8-slice E-step (narrow path only)
    unsigned long long* i8_amax = nullptr;  // [MAX_DP] largest |x - s| per dim (fp64 bits)
    int* i8_lsb = nullptr;     // [MAX_DP] lowest set bit exponent of x - s per dim
    int* i8_plan = nullptr;    // [I8P_SIZE] digit counts and scale exponents
    double* i8_dbl = nullptr;  // [1] sum of the largest scaled features
    int8_t* i8_coef = nullptr; // [ntiles][I8_MAX_LEV][chunks][1024] level digit pieces
    int* i8_ek = nullptr;      // [kp] per-component scale exponent
    int* i8_tinfo = nullptr;   // [ntiles][I8_TINFO] levels per tile
    int8_t* i8_rows = nullptr; // [CHUNK_ROWS][S8_FLG] packed digit rows of the current chunk
    // [b16_chunk / STATS_ROWS][12 dc][1024 B] the split-bf16 statistics pass's
    // operand pieces of the current chunk (the same memory as i8_rows: one
    // call uses one of them)
    uint32_t* b16_pieces = nullptr;
    int64_t b16_chunk = 0;     // rows per chunk of an EM step on bf16 data
    uint16_t* b16_coef = nullptr;  // [ntiles][B16_TILE_BYTES / 2] split-bf16 coefficient pieces
    double* b16_cvec = nullptr;    // [kp] per-component constants of the split-bf16 path (shift 0)
    unsigned long long* b16_amax = nullptr;  // [MAX_DP] largest |x| per dim (fp64 bits), bf16 data
    int* b16_lsb = nullptr;        // [MAX_DP] lowest set bit exponent of x per dim, bf16 data
    int i8_nc = 0;             // bit c set: the pass-1 kernel for c chunks per packed row may run
    bool i8_stats = false;     // the int8 statistics pass exists for this dp
    double2* wlpart = nullptr; // wide: [chunk][ntiles] per-(row, K-tile) (max, sum)
    double* wtval = nullptr;   // wide: [chunk][ntiles][WIDE_TM] top-m candidate values
    int32_t* wtidx = nullptr;  // wide: [chunk][ntiles][WIDE_TM] candidate components
};

// Workspace layout for (d, k). chunk_rows: rows per launch of the narrow
// passes (sizes the per-row scratch); max_groups: cap on the statistics
// pass's row groups (sizes the partials); b16_rows: rows per launch of an EM
// step on bf16 data (sizes the split-bf16 operand pieces; at most chunk_rows,
// a multiple of 256).
bool make_plan(int d, int k, void* ws, Plan* pl, int64_t chunk_rows = CHUNK_ROWS,
               int max_groups = 512, int64_t b16_rows = B16_CHUNK_ROWS);

hipError_t launch_prologue(const Plan& pl, const float* w, const float* mu, const float* var,
                           hipStream_t st);
// lse_out may be null (normalisers not kept); m > 0 also writes the top-m
// components (idx, resp, row-major n x m) of each row.
// km (k-means mode, with m = 1): the row value summed into the partials is
// the best log-density instead of the normaliser.
// skip (device, may be null): the kernel does nothing when *skip == 1 (the
// int8-slice pass runs instead).
hipError_t launch_lse(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                      double* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                      hipStream_t st, int km = 0, const int* skip = nullptr);
// int8-slice E-step: data pass, digit plan and coefficient digits, then the
// mode flag (status[I8S_MODE]) that selects the int8 or the fp64 pass 1.
// em_stats: the call is an EM step or log-likelihood (the int8 and split-bf16
// statistics / normaliser variants may be selected), not k-means or top-m.
hipError_t launch_i8_prologue(const Plan& pl, const float* w, const float* mu, const float* var,
                              const void* x, int64_t n, int64_t ldx, int dtype, hipStream_t st,
                              bool em_stats = true);
hipError_t launch_lse8(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                       double* lse_out, int ll_acc, hipStream_t st);
// k-means mode of the int8-slice pass 1 (after launch_i8_prologue with null
// weights and variances): each row's nearest centroid into z and its
// -|x - c_z|^2 into the partials, when status[I8S_MODE] == 1
hipError_t launch_lse8_km(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                          int32_t* z, int ll_acc, hipStream_t st);
// top-m mode of the int8-slice pass 1 for fp32 data (m <= 4): the normalisers
// and each row's m most responsible components (idx, resp), as launch_lse
hipError_t launch_lse8_topm(const Plan& pl, const void* x, int64_t n, int64_t ldx, double* lse_out,
                            int ll_acc, int m, int32_t* idx, float* resp, hipStream_t st);
// Split-bf16 path: coefficient pieces and the applicability check (run by
// launch_i8_prologue for bf16 data), the normaliser pass (status[I8S_MODE] ==
// MODE1_B16; with `pieces` it also writes the chunk's operand pieces for the
// statistics pass, n <= b16_chunk) and the statistics pass (status[I8S_MODE2]
// == MODE2_B16), which reads those pieces instead of the rows.
hipError_t launch_b16_coef(const Plan& pl, const float* w, const float* mu, const float* var,
                           hipStream_t st);
hipError_t launch_lse16(const Plan& pl, const void* x, int64_t n, int64_t ldx, double* lse_out,
                        int ll_acc, bool pieces, hipStream_t st);
hipError_t launch_stats16(const Plan& pl, int64_t n, const double* lse, int acc, hipStream_t st);
// int8-slice statistics passes (status[I8S_MODE2] == 1: int8 E-step with the
// fp64 M-step; == 2: the M-step on int8 slices too; the fp64 statistics
// kernel is told to skip through the same flag when it is nonzero)
hipError_t launch_stats8(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                         const double* lse, int acc, hipStream_t st);
hipError_t launch_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                        const double* lse, int acc, hipStream_t st, const int* skip = nullptr);
// bit mask of the chunk counts a packed row can have at dimension d
int i8_nc_for(int d);
bool i8_stats_for(int dp);
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
