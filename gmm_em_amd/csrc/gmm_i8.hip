// gmm_i8.hip - the E-step contraction on exact int8 slices (v_mfma_i32_16x16x64_i8).
//
// The E-step log-density of the fused EM step ("Flash-GMM: A Memory-Efficient
// Kernel for Scalable Soft Clustering", section 3: a tiled E-step whose
// responsibilities never reach HBM) is the contraction
//   l[n][k] = sum_f F[n][f] P[k][f] + c_k,   F = [a^2, a] (a = x - s),
//                                            P = [-w/2, w b] (w = 1/var, b = mu - s),
// whose terms cancel to a few nats while each is as large as w a^2 (up to
// ~1e10 for a component at the variance floor). fp32 cannot hold that; fp64
// MFMA can but runs at 1/64 of the int8 MFMA rate. Here the contraction is
// computed exactly on int8 MFMA (the Ozaki splitting of a floating-point
// product into exactly representable slices, Ozaki, Ogita, Oishi and Rump
// 2012; on integer matrix units, Ootomo, Ozaki and Yokota 2024):
//
//  * every feature column is scaled by a power of two 2^G (per dimension and
//    power, from the data's largest |a|) and written as digits of 7 bits:
//    F = 2^G sum_i phi_i 128^-i, phi_1 in [-127, 127], phi_i in [-64, 64];
//    integer data (the descriptor workload) needs 1 digit for a and 2 for a^2
//    and is represented exactly;
//  * every coefficient row, with the feature scales folded in, is scaled by a
//    power of two 2^E_k per component and written as J digits q_j in
//    [-64, 64]; 8 digits hold an fp64 coefficient exactly, and J is the
//    smallest count whose truncation error is below 2^-20 nats for every row;
//  * products of digits are exact, and so are their int32 sums (|sum| <
//    2^23), so level L = i + j contributes 2^(E_k - 7L) * sum_f phi_i q_j
//    exactly; the levels are added in fp64.
// The result equals the fp64 contraction up to the 2^-20 truncation bound and
// fp64 rounding of the level sum. Where the features are not exact in 3
// digits and the truncation of the data cannot be bounded below 2^-20 nats,
// the prologue selects the fp64 kernels instead (a flag in the workspace that
// both kernel variants read; no host synchronisation).
//
// MFMA layout (16x16x64 i8, wave64, measured on gfx950): lane l = 16h + i
// holds A[i][16h .. 16h+15] and B[16h .. 16h+15][i]; register q of the result
// is C[4h + q][i]. Here A = feature digits of 16 rows, B = coefficient digits
// of 16 components: lane (h, i) ends with l[row 4h + q][component i].
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gmm_device.h"
#include "gmm_internal.h"

namespace gmm {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Layout of the packed feature row (bytes): digit blocks i = 1 .. max(Ia, Ib),
// each [a^2 digit i (dq bytes) if i <= Ib][a digit i (dq bytes) if i <= Ia]
// with dq = d rounded up to 16 (dims d .. dq-1 hold 0, so every block starts
// on a 16-byte MFMA column tile), zero padding up to a multiple of 64 (one
// MFMA chunk).
struct I8Layout {
    int ia, ib, fl0, nc;  // digit counts, used bytes, 64-byte chunks
    int off_b[I8_MAX_DIGITS + 1], off_a[I8_MAX_DIGITS + 1];  // block offsets, -1 if absent
};

__device__ __forceinline__ int i8_dq(int d) { return (d + 15) / 16 * 16; }

__device__ __forceinline__ I8Layout i8_layout(const int* plan, int d) {
    I8Layout L;
    L.ia = plan[I8P_IA];
    L.ib = plan[I8P_IB];
    const int dq = i8_dq(d);
    int off = 0;
    const int im = L.ia > L.ib ? L.ia : L.ib;
    for (int i = 1; i <= I8_MAX_DIGITS; ++i) {
        L.off_b[i] = -1;
        L.off_a[i] = -1;
        if (i <= im) {
            if (i <= L.ib) { L.off_b[i] = off; off += dq; }
            if (i <= L.ia) { L.off_a[i] = off; off += dq; }
        }
    }
    L.fl0 = off;
    L.nc = (off + 63) / 64;
    return L;
}

// ---------------------------------------------------------------------------
// Data pass: per dimension, the largest |a| (a = x - s) and the lowest set bit
// over all rows. a is formed in fp64 exactly (fp32 data minus an integer).
// For bf16 data also the same two figures of x itself (the split-bf16 path
// works without the shift).
// ---------------------------------------------------------------------------
__global__ void k_i8_reset(unsigned long long* amax, int* lsb, unsigned long long* amax0,
                           int* lsb0, int dp) {
    for (int i = threadIdx.x; i < dp; i += blockDim.x) {
        amax[i] = 0ull;
        lsb[i] = 0x7fffffff;
        amax0[i] = 0ull;
        lsb0[i] = 0x7fffffff;
    }
}

__device__ __forceinline__ int lowest_bit_exponent(double a) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(a);
    const int be = (int)((u >> 52) & 0x7ff);
    const unsigned long long frac = u & ((1ull << 52) - 1);
    if (be == 0) return -1074 + __builtin_ctzll(frac);  // subnormal (a != 0)
    return be - 1075 + __builtin_ctzll(frac | (1ull << 52));
}

template <typename XT>
__global__ __launch_bounds__(256) void k_i8_xstats(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
                                                   int dp, const double* __restrict__ shift,
                                                   unsigned long long* __restrict__ amax,
                                                   int* __restrict__ lsb,
                                                   unsigned long long* __restrict__ amax0,
                                                   int* __restrict__ lsb0, int* __restrict__ status) {
    __shared__ unsigned long long sm[256], sm0[256];
    __shared__ int sl[256], sl0[256];
    const int dd = threadIdx.x & 127, r0 = threadIdx.x >> 7;  // two rows per sweep, 128 dims
    const bool live = dd < d;
    const double s = live ? shift[(dd & 1) * (dp >> 1) + (dd >> 1)] : 0.0;
    unsigned long long mx = 0ull, mx0 = 0ull;
    int lo = 0x7fffffff, lo0 = 0x7fffffff, bad = 0;
    if (live) {
        // 8 rows per thread and sweep, loaded together
        constexpr int U = 8;
        const int64_t stride = (int64_t)gridDim.x * 2 * U;
        for (int64_t base = (int64_t)blockIdx.x * 2 * U + r0; base < n; base += stride) {
            float xv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = base + 2 * u;
                xv[u] = row < n ? load_x(x + row * ldx + dd) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (base + 2 * u >= n) continue;
                const double a = (double)xv[u] - s;
                if (!isfinite(a)) { bad = 1; continue; }
                if (sizeof(XT) == 2 && xv[u] != 0.0f) {
                    const double x0 = (double)xv[u];
                    const unsigned long long b = (unsigned long long)__double_as_longlong(fabs(x0));
                    mx0 = b > mx0 ? b : mx0;
                    const int e = lowest_bit_exponent(x0);
                    lo0 = e < lo0 ? e : lo0;
                }
                if (a != 0.0) {
                    const unsigned long long b = (unsigned long long)__double_as_longlong(fabs(a));
                    mx = b > mx ? b : mx;
                    const int e = lowest_bit_exponent(a);
                    lo = e < lo ? e : lo;
                }
            }
        }
    }
    sm[threadIdx.x] = mx;
    sl[threadIdx.x] = lo;
    sm0[threadIdx.x] = mx0;
    sl0[threadIdx.x] = lo0;
    __syncthreads();
    if (threadIdx.x < 128 && live) {
        const unsigned long long m2 = sm[threadIdx.x + 128];
        const int l2 = sl[threadIdx.x + 128];
        mx = mx > m2 ? mx : m2;
        lo = lo < l2 ? lo : l2;
        if (mx) atomicMax(&amax[dd], mx);
        if (lo != 0x7fffffff) atomicMin(&lsb[dd], lo);
        if (sizeof(XT) == 2) {
            const unsigned long long n2 = sm0[threadIdx.x + 128];
            const int k2 = sl0[threadIdx.x + 128];
            mx0 = mx0 > n2 ? mx0 : n2;
            lo0 = lo0 < k2 ? lo0 : k2;
            if (mx0) atomicMax(&amax0[dd], mx0);
            if (lo0 != 0x7fffffff) atomicMin(&lsb0[dd], lo0);
        }
    }
    if (bad) atomicOr(&status[I8S_NONFINITE], 1);
}

// Smallest g with v <= 127/128 * 2^g (v >= 0; v = 0 gives 0).
__device__ __forceinline__ int scale_exp(double v) {
    if (!(v > 0.0)) return 0;
    int g = ilogb(v) + 1;  // v < 2^g
    if (ldexp(v, -g) > 127.0 / 128.0) ++g;
    return g;
}

// ---------------------------------------------------------------------------
// Plan: per-dimension scales, digit counts and the bound inputs (one block).
// plan[I8P_GA + d], plan[I8P_GB + d]: exponents G of the a and a^2 columns;
// plan[I8P_IA / I8P_IB]: digits per column kind; plan[I8P_TRUNC_A / _B]: 1 if
// that kind is not exact in its digits; dbl[0] = sum over columns of the
// largest scaled |feature| (bounds the coefficient truncation error).
// ---------------------------------------------------------------------------
__global__ void k_i8_plan(const unsigned long long* __restrict__ amax, const int* __restrict__ lsb,
                          int d, int* __restrict__ plan, double* __restrict__ dbl,
                          int* __restrict__ status) {
    __shared__ int s_ia[128], s_ib[128];
    __shared__ double s_sf[128];
    const int dd = threadIdx.x;
    int ia = 1, ib = 1;
    double sf = 0.0;
    if (dd < d) {
        const double am = __longlong_as_double((long long)amax[dd]);
        const double bm = am * am;
        const int ga = scale_exp(am), gb = scale_exp(bm);
        plan[I8P_GA + dd] = ga;
        plan[I8P_GB + dd] = gb;
        if (am > 0.0) {
            const int lo = lsb[dd];
            // digits i cover down to 2^(g - 7i): exact once g - 7i <= lowest bit
            ia = (ga - lo + 6) / 7;
            ib = (gb - 2 * lo + 6) / 7;
            ia = ia < 1 ? 1 : ia;
            ib = ib < 1 ? 1 : ib;
        }
        sf = ldexp(am, -ga) + ldexp(bm, -gb);
    }
    s_ia[dd] = ia;
    s_ib[dd] = ib;
    s_sf[dd] = sf;
    __syncthreads();
    if (dd == 0) {
        int ma = 1, mb = 1;
        double tot = 0.0;
        for (int j = 0; j < d; ++j) {
            ma = s_ia[j] > ma ? s_ia[j] : ma;
            mb = s_ib[j] > mb ? s_ib[j] : mb;
            tot += s_sf[j];
        }
        plan[I8P_TRUNC_A] = ma > I8_MAX_DIGITS;
        plan[I8P_TRUNC_B] = mb > I8_MAX_DIGITS;
        ma = ma > I8_MAX_DIGITS ? I8_MAX_DIGITS : ma;
        mb = mb > I8_MAX_DIGITS ? I8_MAX_DIGITS : mb;
        plan[I8P_IA] = ma;
        plan[I8P_IB] = mb;
        dbl[0] = tot;
        const int fl0 = i8_dq(d) * (ma + mb);
        if ((fl0 + 63) / 64 > I8_MAX_NC) atomicOr(&status[I8S_FAIL], 1);
    }
}

// ---------------------------------------------------------------------------
// Coefficient digits, one block per 16-component K-tile (256 threads: 16 per
// component). Writes, for each level L = 2 .. Imax + J_t (lev = L - 2), the
// digit vector matched position by position to the packed feature row
// (feature digit i meets coefficient digit L - i), in MFMA B-operand order,
// as consecutive 1 KB pieces (a tile is one contiguous copy). Also E_k and
// the tile's level count.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_i8_coef(const float* __restrict__ w, const float* __restrict__ mu,
                                                 const float* __restrict__ var, int k, int d, int dp,
                                                 const double* __restrict__ shift,
                                                 const int* __restrict__ plan,
                                                 const double* __restrict__ dbl,
                                                 int8_t* __restrict__ coef8, int* __restrict__ ek,
                                                 int* __restrict__ tinfo, int* __restrict__ status) {
    __shared__ int8_t dig[16][2 * MAX_DP][I8_MAX_J];  // [comp][column][digit]
    __shared__ double red[256];
    __shared__ int s_e[16], s_j[16];
    const int tile = blockIdx.x;
    const int c = threadIdx.x >> 4, sub = threadIdx.x & 15;
    const int slot = tile * 16 + c;
    const bool live = slot < k;
    const I8Layout L = i8_layout(plan, d);
    // a layout wider than the kernels' chunk budget: k_i8_plan has already
    // marked the int8 path inapplicable, and nothing is written
    if (L.nc > I8_MAX_NC) return;
    const int dph = dp >> 1;
    // k-means mode (no variances): w = 2, so l = 2 b a - a^2 - |b|^2 = -|x - c|^2
    const bool km = var == nullptr;
    // columns: 0 .. d-1 the a^2 coefficients (-w/2), d .. 2d-1 the a coefficients (w b)
    auto coef_u = [&](int col) -> double {
        const int dd = col < d ? col : col - d;
        const double s = shift[(dd & 1) * dph + (dd >> 1)];
        const double iw = km ? 2.0 : 1.0 / (double)var[(int64_t)slot * d + dd];
        if (col < d) return ldexp(-0.5 * iw, plan[I8P_GB + dd]);
        return ldexp(iw * ((double)mu[(int64_t)slot * d + dd] - s), plan[I8P_GA + dd]);
    };
    double um = 0.0;
    if (live)
        for (int col = sub; col < 2 * d; col += 16) um = fmax(um, fabs(coef_u(col)));
    red[threadIdx.x] = um;
    __syncthreads();
    if (sub == 0) {
        double m = 0.0;
        for (int j = 0; j < 16; ++j) m = fmax(m, red[threadIdx.x + j]);
        // |coefficient| * 2^-E <= 1/2, so the first digit lies in [-64, 64]
        const int e = m > 0.0 ? ilogb(m) + 2 : 0;
        // coefficient truncation after J digits: 2^E * 2^(-7J-1) * sum_f max|F_f|
        int J = 1;
        while (J < I8_MAX_J && ldexp(dbl[0], e - 7 * J - 1) > I8_DELTA) ++J;
        s_e[c] = e;
        s_j[c] = live ? J : 1;
        if (live) ek[slot] = e;
        else ek[slot] = 0;
    }
    __syncthreads();
    const int e = s_e[c];
    int jt = 1;
    for (int j = 0; j < 16; ++j) jt = s_j[j] > jt ? s_j[j] : jt;
    // digits (and the feature-truncation bound for inexact data)
    double tb = 0.0;
    for (int col = sub; col < 2 * MAX_DP; col += 16) {
        double r = (live && col < 2 * d) ? ldexp(coef_u(col), -e) : 0.0;
        if (live && col < 2 * d) {
            const bool trunc = col < d ? plan[I8P_TRUNC_B] : plan[I8P_TRUNC_A];
            const int id = col < d ? L.ib : L.ia;
            if (trunc) tb += fabs(r) * ldexp(1.0, e - 7 * id - 1);
        }
        for (int j = 0; j < I8_MAX_J; ++j) {
            const double t = r * 128.0;
            const double q = rint(t);
            dig[c][col][j] = (int8_t)q;
            r = t - q;
        }
    }
    red[threadIdx.x] = tb;
    __syncthreads();
    if (sub == 0 && live) {
        double t = 0.0;
        for (int j = 0; j < 16; ++j) t += red[threadIdx.x + j];
        if (t > I8_DELTA) atomicOr(&status[I8S_FAIL], 1);
    }
    const int im = L.ia > L.ib ? L.ia : L.ib;
    const int nlev = im + jt - 1;
    if (threadIdx.x == 0) {
        tinfo[tile * I8_TINFO] = nlev;
        atomicMax(&status[I8S_MAXLEV], nlev);
    }
    // level vectors in B-operand order, every chunk of the packed row (zero
    // where the level pairs no digits, and for every level past the tile's
    // count, so that kernels may contract a fixed number of levels): piece
    // (lev * nc + chunk) holds, at [lane 16h + c][16 bytes], positions
    // 64 chunk + 16h .. +15 of component c
    const int nc = L.nc;
    int8_t* dst = coef8 + (int64_t)tile * I8_MAX_LEV * I8_MAX_NC * 1024;
    for (int lev = 0; lev < I8_MAX_LEV; ++lev) {
        const int Lv = lev + 2;
        for (int pos = sub; pos < nc * 64; pos += 16) {
            int v = 0;
            for (int i = 1; i <= im; ++i) {
                const int j = Lv - i;
                if (j < 1 || j > jt) continue;
                if (L.off_b[i] >= 0 && pos >= L.off_b[i] && pos < L.off_b[i] + d) v = dig[c][pos - L.off_b[i]][j - 1];
                if (L.off_a[i] >= 0 && pos >= L.off_a[i] && pos < L.off_a[i] + d) v = dig[c][d + pos - L.off_a[i]][j - 1];
            }
            const int ch = pos >> 6, h = (pos >> 4) & 3, u = pos & 15;
            dst[(int64_t)(lev * nc + ch) * 1024 + (16 * h + c) * 16 + u] = (int8_t)v;
        }
    }
}

// Digit counts (Ia, Ib) an exact layout can have: a^2 carries about twice
// the bits of a, so Ib >= Ia, and with at most three digits each only these
// three pairs occur (the mode kernel below checks it, and the int8
// statistics pass with the int8 M-step is built for exactly these).
__host__ __device__ constexpr bool x8_counts_ok(int ia, int ib) {
    return (ia == 1 && (ib == 1 || ib == 2)) || (ia == 2 && ib == 3);
}

// Mode: the int8 normaliser pass runs when no check failed and the data is
// finite; the int8 statistics pass as well when a tile's digit levels fit
// its registers (stats_ok: the kernel exists for this dimension): with the
// M-step on int8 slices too (mode 2) when every feature is exact in its
// digits, else with the fp64 M-step (mode 1). Otherwise, for bf16 data
// (b16_ok: the split-bf16 kernels were launched for this call) whose checks
// passed, both passes run on split bf16 (else on fp64); that path works on x
// itself, so the shift is set to 0 for the finalisation.
__global__ void k_i8_mode(int* status, const int* plan, int d, int dp, int stats_ok, int b16_ok,
                          double* shift) {
    __shared__ int sel_b16;
    if (threadIdx.x == 0) {
        const int m1 = (status[I8S_FAIL] == 0 && status[I8S_NONFINITE] == 0) ? 1 : 0;
        const I8Layout L = i8_layout(plan, d);
        int m2 = (m1 && stats_ok && L.nc <= S8_NC && status[I8S_MAXLEV] <= S8_LV) ? 1 : 0;
        if (m2 && plan[I8P_TRUNC_A] == 0 && plan[I8P_TRUNC_B] == 0 &&
            x8_counts_ok(plan[I8P_IA], plan[I8P_IB]))
            m2 = 2;
        const int b16 = (!m1 && b16_ok && status[I8S_B16FAIL] == 0 && status[I8S_NONFINITE] == 0) ? 1 : 0;
        status[I8S_MODE] = b16 ? MODE1_B16 : m1;
        status[I8S_MODE2] = b16 ? MODE2_B16 : m2;
        sel_b16 = b16;
    }
    __syncthreads();
    if (sel_b16)
        for (int i = threadIdx.x; i < dp; i += blockDim.x) shift[i] = 0.0;
}

// One fold of the level sums: a pair of consecutive levels L, L+1 is first
// combined exactly in int32 (128 acc_L + acc_{L+1}: |acc| < 2^22, so no
// overflow), then added in fp64 with its power-of-two scale (a lone last
// level comes with acc_{L+1} = 0). Both passes fold in the same order, so
// they produce bitwise identical log-densities.
__device__ __forceinline__ void fold_pair(double& l, int a, int b, double sc) {
    l = fma((double)(a * 128 + b), sc, l);
}

// ---------------------------------------------------------------------------
// Pass 1 on int8 slices: per-row logsumexp over all components.
// Block = 8 waves, 64 rows per wave (four 16-row MFMA tiles), 512 rows. Each
// wave packs the digit rows of its 64 rows once (through LDS) and keeps them
// in registers as A operands; the K-tiles' level vectors stream through two
// LDS buffers (tile t+1 is copied while tile t is contracted). The kernel is
// built for an exact chunk count NC and at most LV levels (the variants
// whose NC or LV do not match the plan return at once): per level pair of
// the tile (its count is loaded one tile ahead), all NC chunks into one
// int32 accumulator per row tile, folded into fp64 (l += acc * 2^(E_k - 7L));
// the finished tile's values go into the online logsumexp (fp64 running
// maximum, fp32 scaled sum). Levels past a tile's count have zero digits.
// MODE selects what the kernel keeps per row: 0 the normaliser; 1 (k-means)
// the best value and its component instead; 2 or 4 the normaliser and the
// top-2 or top-4 components (soft assignment), with 32 rows per wave (two
// row tiles) so that the candidate lists fit the registers of two waves per
// SIMD.
// ---------------------------------------------------------------------------
constexpr int L8_WAVES = 8;
constexpr int L8_RT = 4;  // 16-row tiles per wave

template <int NC, int LV, typename XT, int MODE = 0>
__global__ __launch_bounds__(L8_WAVES * 64, 1)
void k_lse8(const XT* __restrict__ x, int64_t n, int d, int64_t ldx, int dp,
            const double* __restrict__ shift, const int* __restrict__ plan,
            const int8_t* __restrict__ coef8, const int* __restrict__ ek,
            const int* __restrict__ tinfo, const double* __restrict__ cvec, int ntiles,
            double* __restrict__ lse_out, double* __restrict__ llpart, int ll_accumulate,
            int8_t* __restrict__ drows, const int* __restrict__ status,
            int32_t* __restrict__ z_out = nullptr, int k = 0, int m_out = 0,
            float* __restrict__ resp_out = nullptr) {
    constexpr bool KM = MODE == 1;
    constexpr int TM = MODE >= 2 ? MODE : 0;  // candidates kept per row
    constexpr int TMA = TM > 0 ? TM : 1;
    constexpr int RT = TM > 0 ? 2 : L8_RT;   // 16-row tiles per wave
    constexpr int ROWS = L8_WAVES * RT * 16;
    static_assert(ROWS % LL_ROWS == 0, "whole log-likelihood partials per block");
    constexpr int FLS = NC * 64 + 16;            // LDS stride of a packed row (conflict-free b128 reads)
    constexpr int TBL = LV * NC * 1024;          // bytes of one tile's level vectors
    constexpr int STG = L8_WAVES * 16 * FLS;     // staging of 16 rows per wave
    constexpr int TB = TBL > STG ? TBL : STG;
    __shared__ __attribute__((aligned(16))) int8_t cbuf[2][TB];
    __shared__ double rowll[ROWS];
    if (status[I8S_MODE] != 1) return;  // the fp64 kernels run instead
    const I8Layout LY = i8_layout(plan, d);
    const int maxlev = status[I8S_MAXLEV];
    if (LY.nc != NC || maxlev > LV || (LV > S8_LV && maxlev <= S8_LV)) return;  // another variant runs

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = lane & 15, h = lane >> 4;
    const int64_t wrow = (int64_t)blockIdx.x * ROWS + wave * (RT * 16);
    const int dph = dp >> 1;
    const bool hand_off = MODE == 0 && status[I8S_MODE2] != 0;

    // ---- pack the wave's rows: digits of a^2 and a, through LDS. Lane l
    // handles dims l and l + 64 (d <= 128) of 16 rows at a time, with the
    // per-dimension shift and scales loaded once and the 32 values of a
    // 16-row tile loaded together.
    v4i A[RT][NC];
    {
        int8_t* stg = &cbuf[1][wave * 16 * FLS];
        double sh[2], ga[2], gb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int dd = lane + 64 * u;
            const bool live = dd < d;
            sh[u] = live ? shift[(dd & 1) * dph + (dd >> 1)] : 0.0;
            ga[u] = live ? ldexp(1.0, -plan[I8P_GA + dd]) : 0.0;
            gb[u] = live ? ldexp(1.0, -plan[I8P_GB + dd]) : 0.0;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {  // unrolled: A stays in registers
            float xv[16][2];
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int64_t row = wrow + rt * 16 + r;
                    const int dd = lane + 64 * u;
                    xv[r][u] = (row < n && dd < d) ? load_x(x + row * ldx + dd) : 0.0f;
                }
            for (int e = lane; e < 16 * FLS / 16; e += 64) ((v4i*)stg)[e] = v4i{0, 0, 0, 0};
            __syncthreads();
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int8_t* pr = stg + r * FLS;
                const bool rv = wrow + rt * 16 + r < n;  // rows past n pack as zeros
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int dd = lane + 64 * u;
                    if (dd >= d) continue;
                    const double a = rv ? (double)xv[r][u] - sh[u] : 0.0;
                    double va = a * ga[u], vb = (a * a) * gb[u];
#pragma unroll
                    for (int i = 1; i <= I8_MAX_DIGITS; ++i) {
                        const double ta = va * 128.0, tb = vb * 128.0;
                        const double qa = rint(ta), qb = rint(tb);
                        va = ta - qa;
                        vb = tb - qb;
                        if (LY.off_a[i] >= 0) pr[LY.off_a[i] + dd] = (int8_t)qa;
                        if (LY.off_b[i] >= 0) pr[LY.off_b[i] + dd] = (int8_t)qb;
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int c = 0; c < NC; ++c) A[rt][c] = *(const v4i*)(stg + ci * FLS + 64 * c + 16 * h);
            // hand the packed rows to the statistics pass (row stride S8_FLG)
            if (hand_off) {
                const int per_row = LY.nc * 4;  // 16-byte pieces
                for (int e = lane; e < 16 * per_row; e += 64) {
                    const int r = e / per_row, u = e - r * per_row;
                    const int64_t row = wrow + rt * 16 + r;
                    if (row < n)
                        *(v4i*)(drows + row * S8_FLG + u * 16) = *(const v4i*)(stg + r * FLS + u * 16);
                }
            }
            __syncthreads();
        }
    }

    // ---- stream the K-tiles: tile t+1's level vectors are copied into the
    // other buffer by buffer-to-LDS loads (one 1 KB operand piece per wave
    // instruction, no registers held) while tile t is contracted
    constexpr int TSTRIDE = I8_MAX_LEV * I8_MAX_NC * 1024;
    auto issue_tile = [&](int t, int buf) {
        const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(coef8 + (int64_t)t * TSTRIDE), (short)0, TSTRIDE, BUF_RSRC_WORD3);
        for (int p = wave; p < LV * NC; p += L8_WAVES)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                cr, (__attribute__((address_space(3))) void*)(cbuf[buf] + p * 1024), 16, lane * 16,
                p * 1024, 0, 0);
    };
    // normaliser mode: online logsumexp (m, s); k-means mode: the best value
    // and its component (m, bi; the first in component order on ties)
    double m[RT][4];
    float s[RT][4];
    int bi[RT][4];
    double tv[RT][4][TMA];  // top-m candidates (value, component), best first
    int ti[RT][4][TMA];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            m[rt][q] = KM ? -INFINITY : -1.0e300;
            s[rt][q] = 0.0f;
            bi[rt][q] = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < TMA; ++j) {
                tv[rt][q][j] = -INFINITY;
                ti[rt][q][j] = 0x7fffffff;
            }
        }
    issue_tile(0, 0);
    // per-component scale exponent and constant of the next tile, loaded one
    // tile ahead (their latency would otherwise stall the first fold)
    int ekn = ek[ci];
    double ccn = cvec[ci];
    int nln = tinfo[0];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
        const double scale = ldexp(1.0, ekn - 14);  // level 2
        const double cc = ccn;
        const int nl = nln;  // this tile's digit levels (those past it are zero)
        if (t + 1 < ntiles) {
            ekn = ek[(t + 1) * 16 + ci];
            ccn = cvec[(t + 1) * 16 + ci];
            nln = tinfo[(t + 1) * I8_TINFO];
        }
        double l[RT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) l[rt][q] = 0.0;
        const int8_t* cb = cbuf[buf] + lane * 16;
        double sc = scale * (1.0 / 128.0);  // a pair starting at level 2
        // the wave issuing its matrix block goes first on the SIMD; its
        // logsumexp below runs at normal priority under the other wave's
        // matrix block
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int lev = 0; lev < LV; lev += 2) {
            if (lev >= nl) break;  // the tile's remaining levels are zero
            v4i acc0[RT], acc1[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                acc0[rt] = v4i{0, 0, 0, 0};
                acc1[rt] = v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const v4i b0 = *(const v4i*)(cb + (lev * NC + c) * 1024);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) acc0[rt] = mfma_i8(A[rt][c], b0, acc0[rt]);
                if (lev + 1 < LV) {
                    const v4i b1 = *(const v4i*)(cb + ((lev + 1 < LV ? lev + 1 : lev) * NC + c) * 1024);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) acc1[rt] = mfma_i8(A[rt][c], b1, acc1[rt]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int q = 0; q < 4; ++q) fold_pair(l[rt][q], acc0[rt][q], acc1[rt][q], sc);
            sc *= 1.0 / 16384.0;
            // keep each pair's products and fold together: bounds the live
            // accumulators (the register budget of two waves per SIMD)
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (KM) {
                    const double v = l[rt][q] + cc;
                    const bool up = v > m[rt][q];
                    m[rt][q] = up ? v : m[rt][q];
                    bi[rt][q] = up ? t * 16 + ci : bi[rt][q];
                } else {
                    lse_push(m[rt][q], s[rt][q], l[rt][q] + cc);
                    // components arrive in increasing order along the lane
                    if constexpr (TM > 0) top_push_inc<TM>(tv[rt][q], ti[rt][q], l[rt][q] + cc, t * 16 + ci);
                }
            }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile t+1 have landed
        __syncthreads();                // ... and every wave's; tile t's buffer is free
    }

    // ---- merge the 16 lanes holding the same rows (fixed butterfly order)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll 1
            for (int off = 1; off < 16; off <<= 1) {
                const double m2 = shfl_xor_d(m[rt][q], off);
                if constexpr (KM) {
                    const int i2 = __shfl_xor(bi[rt][q], off);
                    const bool take = m2 > m[rt][q] || (m2 == m[rt][q] && i2 < bi[rt][q]);
                    m[rt][q] = take ? m2 : m[rt][q];
                    bi[rt][q] = take ? i2 : bi[rt][q];
                } else {
                    const float s2 = __shfl_xor(s[rt][q], off);
                    lse_merge(m[rt][q], s[rt][q], m2, s2);
                    if constexpr (TM > 0) top_merge<TM>(tv[rt][q], ti[rt][q], off);
                }
            }
        }
    if (ci == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int lr = wave * (RT * 16) + rt * 16 + 4 * h + q;
                const int64_t row = (int64_t)blockIdx.x * ROWS + lr;
                double v = 0.0;
                if (row < n) {
                    if constexpr (KM) {
                        // the row's best value -|x - c_z|^2 (its share of -inertia)
                        v = m[rt][q];
                        z_out[row] = bi[rt][q] < k ? bi[rt][q] : -1;
                    } else {
                        v = m[rt][q] + log((double)s[rt][q]);
                        if (lse_out) lse_out[row] = v;
                        if constexpr (TM > 0) {
#pragma unroll
                            for (int j = 0; j < TM; ++j) {  // (static indices: the lists stay in registers)
                                if (j >= m_out) continue;
                                const int sl = ti[rt][q][j];
                                z_out[row * m_out + j] = sl < k ? sl : -1;
                                if (resp_out) resp_out[row * m_out + j] = __expf((float)(tv[rt][q][j] - v));
                            }
                        }
                    }
                }
                rowll[lr] = v;
            }
    }
    __syncthreads();
    // one partial per 64 rows: wave w < ROWS / 64 sums rows 64w .. 64w + 63
    // (its own rows at 64 rows per wave; fixed order)
    if (wave < ROWS / LL_ROWS) {
        double tot = rowll[wave * LL_ROWS + lane];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) tot += shfl_xor_d(tot, off);
        const int64_t pi = (int64_t)blockIdx.x * (ROWS / LL_ROWS) + wave;
        if (lane == 0 && pi * LL_ROWS < n) llpart[pi] = (ll_accumulate ? llpart[pi] : 0.0) + tot;
    }
}

// ---------------------------------------------------------------------------
// Pass 2 on int8 slices: statistics. Same organisation as the fp64
// statistics pass (a block of 4 waves, wave w owning K-tile kg*4 + w, the
// block walking its row group in 32-row tiles): the wave's coefficient digit
// levels stay in registers, the row tiles' packed digit rows (written by the
// normaliser pass) arrive by buffer-to-LDS copies, and the E-step is the int8
// contraction with the normaliser pass's fold, so both passes see the same
// log-densities bit for bit. The M-step is unchanged: fp64 MFMA of
// r = exp(l - lse) against the rows' fp64 [a, a^2] (staged in LDS), with
// register statistics over the row group. The int8 result layout gives lane
// (h, i) rows 4h + q of a 16-row tile; the M-step takes its 4-row groups in
// that order (row 16 rb + 4h + q for step (rb, q)), so responsibilities
// still go from the E-step accumulators to the M-step operand in registers.
// ---------------------------------------------------------------------------
template <int DP, typename XT>
__global__ __launch_bounds__(256, 1)
void k_stats8(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
              const int8_t* __restrict__ drows, const int8_t* __restrict__ coef8,
              const int* __restrict__ ek, const int* __restrict__ tinfo,
              const double* __restrict__ cvec, const double* __restrict__ shift,
              const int* __restrict__ plan, int ntiles, const double* __restrict__ lse,
              int64_t rows_per_group, double* __restrict__ part, double* __restrict__ npart,
              int accumulate, const int* __restrict__ status) {
    constexpr int WV = 4, NT = 256;
    constexpr int DPH = DP / 2, HS = DPH + 4, S = 4 * HS + 2;  // fp64 feature tile layout
    constexpr int PER = STATS_ROWS * DP / NT;
    constexpr int NJ = DP / 16;
    constexpr int DGB = STATS_ROWS * S8_FLG;      // digit bytes of a 32-row tile
    constexpr int DGP = (DGB + 1023) / 1024;      // 1 KB copy pieces
    static_assert(PER * NT == STATS_ROWS * DP, "every thread stages the same number of values");
    __shared__ __attribute__((aligned(16))) double fs[2][STATS_ROWS * S];
    __shared__ double ls[2][STATS_ROWS];
    __shared__ __attribute__((aligned(16))) int8_t dg[2][DGP * 1024];
    if (status[I8S_MODE2] != 1) return;  // the fp64 statistics pass runs instead

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = lane & 15, h = lane >> 4;
    const int kgroups = ntiles / WV;
    const int nb = gridDim.x;
    const int o = (nb % 8 == 0) ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
    const int g = o / kgroups;
    const int tile = (o % kgroups) * WV + wave;
    const int slot = tile * 16 + ci;
    const I8Layout LY = i8_layout(plan, d);
    const int nc = LY.nc;
    const int nl = tinfo[tile * I8_TINFO];

    // the K-tile's digit levels (B operands), resident for the whole pass
    v4i qd[S8_LV][S8_NC];
    {
        const int8_t* cp = coef8 + (int64_t)tile * (I8_MAX_LEV * I8_MAX_NC * 1024) + lane * 16;
#pragma unroll
        for (int lev = 0; lev < S8_LV; ++lev)
#pragma unroll
            for (int c = 0; c < S8_NC; ++c)
                qd[lev][c] = (lev < nl && c < nc) ? *(const v4i*)(cp + (lev * nc + c) * 1024)
                                                  : v4i{0, 0, 0, 0};
    }
    const double scale = ldexp(1.0, ek[slot] - 14);
    const double cc = cvec[slot];

    f64x4 acc[2 * NJ];
#pragma unroll
    for (int j = 0; j < 2 * NJ; ++j) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
    double n64 = 0.0;

    const int64_t gr0 = (int64_t)g * rows_per_group;
    int64_t gr1 = gr0 + rows_per_group;
    if (gr1 > n) gr1 = n;
    const int64_t ntile_rows = gr1 > gr0 ? (gr1 - gr0 + STATS_ROWS - 1) / STATS_ROWS : 0;

    // fp64 features for the M-step, staged as in the fp64 statistics pass
    float xv[PER];
    double lv = 0.0;
    double shv[PER];
    uint32_t xoff[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid + NT * i;
        const int r = e / DP, dd = e % DP;
        shv[i] = shift[(dd & 1) * DPH + (dd >> 1)];
        xoff[i] = dd < d ? (uint32_t)(((int64_t)r * ldx + dd) * (int64_t)sizeof(XT)) : 0xFFFFFFF0u;
    }
    auto load = [&](int64_t it) {
        const int64_t rbase = gr0 + it * STATS_ROWS;
        int64_t nv = gr1 - rbase;
        nv = nv < 0 ? 0 : (nv > STATS_ROWS ? STATS_ROWS : nv);
        const int xbytes = nv > 0 ? (int)(((nv - 1) * ldx + d) * (int64_t)sizeof(XT)) : 0;
        const __amdgpu_buffer_rsrc_t xr =
            __builtin_amdgcn_make_buffer_rsrc((void*)(x + rbase * ldx), (short)0, xbytes, BUF_RSRC_WORD3);
#pragma unroll
        for (int i = 0; i < PER; ++i) xv[i] = buf_load_x<XT>(xr, xoff[i]);
        const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(lse + rbase), (short)0, (int)(nv * (int64_t)sizeof(double)), BUF_RSRC_WORD3);
        const int lrow = tid & (STATS_ROWS - 1);
        const double v = buf_load_f64(lr, (uint32_t)lrow * 8u);
        lv = lrow < nv ? v : INFINITY;  // rows past the row group: responsibility 0
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + NT * i;
            const int r = e / DP, dd = e % DP;
            const int pp = 2 * (dd & 1), t = dd >> 1;
            const double a = (double)xv[i] - shv[i];
            fs[buf][r * S + pp * HS + t] = a;
            fs[buf][r * S + (pp + 1) * HS + t] = a * a;
        }
        ls[buf][tid & (STATS_ROWS - 1)] = lv;
    };
    // digit rows of tile it: contiguous in the workspace (stride S8_FLG), so
    // the copy is DGP pieces of 1 KB; rows past the row group read as 0
    auto issue_dg = [&](int64_t it, int buf) {
        const int64_t rbase = gr0 + it * STATS_ROWS;
        int64_t nv = gr1 - rbase;
        nv = nv < 0 ? 0 : (nv > STATS_ROWS ? STATS_ROWS : nv);
        const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(drows + rbase * S8_FLG), (short)0, (int)(nv * S8_FLG), BUF_RSRC_WORD3);
        for (int p = wave; p < DGP; p += WV)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                dr, (__attribute__((address_space(3))) void*)(dg[buf] + p * 1024), 16, lane * 16,
                p * 1024, 0, 0);
    };

    if (ntile_rows > 0) {
        load(0);
        issue_dg(0, 0);
        store(0);
        if (ntile_rows > 1) load(1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int64_t it = 0; it < ntile_rows; ++it) {
        const int buf = (int)(it & 1);
        // next tile's digit rows (its buffer was last read before the
        // previous iteration's closing barrier)
        if (it + 1 < ntile_rows) issue_dg(it + 1, buf ^ 1);
        // E-step: two 16-row tiles, all levels, the normaliser pass's fold.
        // Every chunk is contracted: a chunk past the rows' digits has zero
        // coefficients (its digit bytes are not written and read as anything),
        // and a missing second level of the last pair has zero coefficients.
        const int8_t* db = dg[buf];
        v4i A[2][S8_NC];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int c = 0; c < S8_NC; ++c)
                A[rb][c] = *(const v4i*)(db + (16 * rb + ci) * S8_FLG + 64 * c + 16 * h);
        double l[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q) l[rb][q] = 0.0;
        double sc = scale * (1.0 / 128.0);
#pragma unroll
        for (int lev = 0; lev < S8_LV; lev += 2) {
            if (lev < nl) {
                v4i a0[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
                v4i a1[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
#pragma unroll
                for (int c = 0; c < S8_NC; ++c) {
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) a0[rb] = mfma_i8(A[rb][c], qd[lev][c], a0[rb]);
                    if (lev + 1 < S8_LV) {
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb)
                            a1[rb] = mfma_i8(A[rb][c], qd[lev + 1 < S8_LV ? lev + 1 : lev][c], a1[rb]);
                    }
                }
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) fold_pair(l[rb][q], a0[rb][q], a1[rb][q], sc);
                sc *= 1.0 / 16384.0;
            }
        }
        // responsibilities of rows 16 rb + 4h + q
        double r[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                r[rb][q] = exp_f64range(l[rb][q] + cc - ls[buf][16 * rb + 4 * h + q]);
                n64 += r[rb][q];
            }
        // stage the next tile's fp64 features (buffer buf^1 was last read
        // before the previous iteration's closing barrier)
        if (it + 1 < ntile_rows) {
            store(buf ^ 1);
            if (it + 2 < ntile_rows) load(it + 2);
        }
        // M-step: step (rb, q) contracts r[row 16 rb + 4h + q][comp ci] with
        // feature column 16j + ci of that row; a step whose 64
        // responsibilities are all exactly zero adds nothing and is skipped
        const double* fb = fs[buf];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double rv = r[rb][q];
                if (__builtin_amdgcn_ballot_w64(rv != 0.0) == 0) continue;
                const double* fm = fb + (16 * rb + 4 * h + q) * S;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int dd = 16 * j + ci;
                    acc[j] = mfma4d(rv, fm[2 * (dd & 1) * HS + (dd >> 1)], acc[j]);
                    acc[NJ + j] = mfma4d(rv, fm[(2 * (dd & 1) + 1) * HS + (dd >> 1)], acc[NJ + j]);
                }
            }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's digit copies of the next tile have landed
        __syncthreads();
    }

    // responsibility mass: lanes ci, ci+16, ci+32, ci+48 hold disjoint rows
    n64 += shfl_xor_d(n64, 16);
    n64 += shfl_xor_d(n64, 32);
    const int64_t gbase = (int64_t)g * ntiles * 16;
    if (h == 0) {
        double* np = npart + gbase + slot;
        *np = (accumulate ? *np : 0.0) + n64;
    }
#pragma unroll
    for (int j = 0; j < 2 * NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int comp = tile * 16 + 4 * q + h;
            double* p2 = part + (gbase + comp) * (2 * DP) + 16 * j + ci;
            *p2 = (accumulate ? *p2 : 0.0) + acc[j][q];
        }
}

// ---------------------------------------------------------------------------
// Pass 2 with the M-step on int8 slices as well (mode 2: every feature is
// exact in its digits). The statistics [sum r, sum r a, sum r a^2] are the
// contraction over rows of the responsibilities with the rows' features, and
// the features' digits are already in the packed rows. Per 64-row block and
// component, the responsibilities are put on a block exponent e (every r of
// the block is below 2^e) and cut to r' = u 2^(e - 41), u an integer of at
// most 42 bits written as six 7-bit digits: r' is r to fp32 precision for
// every row within 2^-18 of the block's largest responsibility and below it
// by less than 2^(e - 41) for the others (six digits rather than four: where
// a component's main rows agree in a dimension, its variance there comes from
// rows of small responsibility, which need their own relative precision).
// Sums of digit products are exact in int32, so the kernel
// computes the statistics of the weights r' exactly (up to the fp64 rounding
// of the block sums), and the mass sum r' is taken from the same integers:
// mean and variance are those of one consistent set of weights, so the
// variance's cancellation (E[a^2] - mean^2) does not magnify the rounding.
//
// Block = 4 waves, wave w owns K-tile kg*4 + w as in the other statistics
// passes; the block walks its row group in 64-row blocks. Per block:
//  * the packed digit rows arrive by buffer-to-LDS copies (one block ahead);
//  * the E-step's int8 result leaves lane (h, i) with rows 16s + 4h + q
//    (tile s, register q) of component i: these 16 rows become the lane's
//    16 positions of the M-step contraction, so the responsibilities turn
//    into MFMA operands without leaving the lane, and the feature digit
//    columns are read in the same row order by transposed LDS reads
//    (ds_read_b64_tr_b8) straight from the packed rows;
//  * the E-step as in the pass above (same fold, same bits), then the
//    digits of r', and the M-step: A = feature digit columns (16 dims),
//    B = responsibility digits (16 components), one int32 accumulator per
//    level (feature digit i + responsibility digit j), levels folded in
//    pairs into fp64 with the block's scale 2^(e - 20 - 7 level).
// The feature scale 2^G of each dimension multiplies the sums once at the end.
// ---------------------------------------------------------------------------
constexpr int X8_ROWS = 64;  // rows per block: the int8 MFMA's contraction length
constexpr int X8_RD = 6;     // responsibility digits

// Transposed LDS read (ds_read_b64_tr_b8, measured on gfx950): within each
// group of 16 lanes, lane 8u + b receives byte b of the 8 bytes read by
// lanes 2k + u, k = 0 .. 7 (its byte k), whatever the addresses.
typedef int v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2i lds_read_tr8(const int8_t* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)p);
}

// One 16-dimension tile of one feature kind: its NI digit columns against
// the responsibility digits, one int32 accumulator per level i + j, levels
// folded in pairs into the fp64 sums of dims 16 j + 4 h + q of component ci.
// The digit columns come straight from the block's packed rows: column
// 16 j + ci of lane (h, ci) at position 8 t + k is row 16 (2t + k/4) + 4h +
// k%4, the row the responsibility digits hold at that position; lane
// (h, m) reads 8 bytes of row 16 (2t + m/8) + 4h + (m/2)%4 at column
// 16 j + 8 (m%2) (rofs[t] is that row's offset plus 8 (m%2)).
template <int NI>
__device__ __forceinline__ void x8_mstep_tile(const int8_t* db, const int (&rofs)[2], const int (&coff)[NI],
                                              int j, const v4i (&R)[X8_RD], double sp0,
                                              double (&acc)[4]) {
    constexpr int NLV = NI + X8_RD - 1;
    v4i B[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const v2i lo = lds_read_tr8(db + rofs[0] + coff[i] + 16 * j);
        const v2i hi = lds_read_tr8(db + rofs[1] + coff[i] + 16 * j);
        B[i] = v4i{lo[0], lo[1], hi[0], hi[1]};
    }
    v4i S[NLV];
#pragma unroll
    for (int lv = 0; lv < NLV; ++lv) S[lv] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int jr = 0; jr < X8_RD; ++jr) S[i + jr] = mfma_i8(B[i], R[jr], S[i + jr]);
    double sp = sp0;
#pragma unroll
    for (int lv = 0; lv < NLV; lv += 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) fold_pair(acc[q], S[lv][q], lv + 1 < NLV ? S[lv + 1][q] : 0, sp);
        sp *= 1.0 / 16384.0;
    }
}

template <int DP, int IA, int IB>
__global__ __launch_bounds__(256, 1)
void k_stats8x(const int8_t* __restrict__ drows, int64_t n, int d,
               const int8_t* __restrict__ coef8, const int* __restrict__ ek,
               const int* __restrict__ tinfo, const double* __restrict__ cvec,
               const int* __restrict__ plan, int ntiles, const double* __restrict__ lse,
               int64_t rows_per_group, double* __restrict__ part, double* __restrict__ npart,
               int accumulate, const int* __restrict__ status) {
    constexpr int WV = 4, NT = 256;
    constexpr int NJ = DP / 16;
    constexpr int DGB = X8_ROWS * S8_FLG;         // packed digit rows of one block
    constexpr int DGP = (DGB + 1023) / 1024;      // 1 KB copy pieces
    constexpr double LOG2E = 1.4426950408889634074;
    __shared__ __attribute__((aligned(16))) int8_t dg[2][DGP * 1024];
    __shared__ double ls[2][X8_ROWS];
    if (status[I8S_MODE2] != 2) return;  // another statistics pass runs instead
    if (plan[I8P_IA] != IA || plan[I8P_IB] != IB) return;  // the variant for these counts runs

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = lane & 15, h = lane >> 4;
    const int kgroups = ntiles / WV;
    const int nb = gridDim.x;
    const int o = (nb % 8 == 0) ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
    const int g = o / kgroups;
    const int tile = (o % kgroups) * WV + wave;
    const int slot = tile * 16 + ci;
    const int nl = tinfo[tile * I8_TINFO];
    const int dq = i8_dq(d);

    // the K-tile's E-step digit levels (B operands), resident for the pass
    v4i qd[S8_LV][S8_NC];
    {
        const int nc = i8_layout(plan, d).nc;
        const int8_t* cp = coef8 + (int64_t)tile * (I8_MAX_LEV * I8_MAX_NC * 1024) + lane * 16;
#pragma unroll
        for (int lev = 0; lev < S8_LV; ++lev)
#pragma unroll
            for (int c = 0; c < S8_NC; ++c)
                qd[lev][c] = (lev < nl && c < nc) ? *(const v4i*)(cp + (lev * nc + c) * 1024)
                                                  : v4i{0, 0, 0, 0};
    }
    const double scale = ldexp(1.0, ek[slot] - 14);
    const double cc = cvec[slot];

    double acc[2][NJ][4];  // [a^2, a][dim tile][dim 16 j + 4 h + q], component ci
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[k2][j][q] = 0.0;
    double n64 = 0.0;

    const int64_t gr0 = (int64_t)g * rows_per_group;
    int64_t gr1 = gr0 + rows_per_group;
    if (gr1 > n) gr1 = n;
    const int64_t nblk = gr1 > gr0 ? (gr1 - gr0 + X8_ROWS - 1) / X8_ROWS : 0;

    auto rows_in = [&](int64_t it) -> int {
        const int64_t nv = gr1 - (gr0 + it * X8_ROWS);
        return nv < 0 ? 0 : (nv > X8_ROWS ? X8_ROWS : (int)nv);
    };
    // packed digit rows of block it (rows past the group read as 0)
    auto issue_dg = [&](int64_t it, int buf) {
        const int64_t rbase = gr0 + it * X8_ROWS;
        const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(drows + rbase * S8_FLG), (short)0, rows_in(it) * S8_FLG, BUF_RSRC_WORD3);
        for (int p = wave; p < DGP; p += WV)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                dr, (__attribute__((address_space(3))) void*)(dg[buf] + p * 1024), 16, lane * 16,
                p * 1024, 0, 0);
    };
    // normaliser of row tid of block it (+inf past the group: r = 0)
    auto load_ls = [&](int64_t it) -> double {
        const int nv = rows_in(it);
        return tid < nv ? lse[gr0 + it * X8_ROWS + tid] : INFINITY;
    };

    if (nblk > 0) {
        issue_dg(0, 0);
        if (tid < X8_ROWS) ls[0][tid] = load_ls(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // M-step operand addresses: digit block offsets in the packed row (a^2
    // digit i at dq (min(i-1, Ib) + min(i-1, Ia)), a digit i after it) and
    // this lane's two row offsets for the transposed reads
    int cb[IB], ca[IA];
#pragma unroll
    for (int i = 0; i < IB; ++i) cb[i] = dq * ((i < IB ? i : IB) + (i < IA ? i : IA));
#pragma unroll
    for (int i = 0; i < IA; ++i) ca[i] = dq * ((i < IB ? i : IB) + (i < IA ? i : IA) + (i < IB ? 1 : 0));
    int rofs[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        rofs[t] = (16 * (2 * t + (ci >> 3)) + 4 * h + ((ci >> 1) & 3)) * S8_FLG + 8 * (ci & 1);

    for (int64_t it = 0; it < nblk; ++it) {
        const int buf = (int)(it & 1);
        double lsn = INFINITY;
        if (it + 1 < nblk) {
            issue_dg(it + 1, buf ^ 1);
            if (tid < X8_ROWS) lsn = load_ls(it + 1);
        }
        const int8_t* db = dg[buf];

        // ---- E-step: four 16-row tiles, the normaliser pass's fold
        double l[4][4];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            v4i A[2][S8_NC];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int c = 0; c < S8_NC; ++c)
                    A[rb][c] = *(const v4i*)(db + (16 * (2 * hf + rb) + ci) * S8_FLG + 64 * c + 16 * h);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int q = 0; q < 4; ++q) l[2 * hf + rb][q] = 0.0;
            // every level (a tile's levels past its count have zero digits):
            // one branch-free block the scheduler can interleave, measured
            // faster here than stopping at the tile's count
            double sc = scale * (1.0 / 128.0);
#pragma unroll
            for (int lev = 0; lev < S8_LV; lev += 2) {
                v4i a0[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
                v4i a1[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
#pragma unroll
                for (int c = 0; c < S8_NC; ++c) {
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) a0[rb] = mfma_i8(A[rb][c], qd[lev][c], a0[rb]);
                    if (lev + 1 < S8_LV) {
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb)
                            a1[rb] = mfma_i8(A[rb][c], qd[lev + 1 < S8_LV ? lev + 1 : lev][c], a1[rb]);
                    }
                }
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        fold_pair(l[2 * hf + rb][q], a0[rb][q], a1[rb][q], sc);
                sc *= 1.0 / 16384.0;
            }
        }

        // ---- responsibilities on the block exponent, as four 7-bit digits
        double t[4][4];
        double tm = -INFINITY;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                t[s][q] = l[s][q] + cc - ls[buf][16 * s + 4 * h + q];
                tm = fmax(tm, t[s][q]);
            }
        tm = fmax(tm, shfl_xor_d(tm, 16));
        tm = fmax(tm, shfl_xor_d(tm, 32));
        const double z = tm * LOG2E;
        const int e = z > -1000.0 ? (int)floor(z) + 1 : -1000;  // every r of the block < 2^e
        const double yb = (double)(6 - e);
        const double snh = ldexp(1.0, e - 20), snl = ldexp(1.0, e - 41);
        v4i R[X8_RD];
        bool any = false;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t uh[4], ul[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double y = fmax(fma(t[s][q], LOG2E, yb), -64.0);  // log2(r 2^(6 - e)) < 6
                const float v = __builtin_amdgcn_exp2f((float)y);
                // v = hi 2^-14 + lo 2^-35 (+ less than 2^-35): hi < 2^20 + 1, lo < 2^21
                const float hf = floorf(v * 16384.0f);
                const float vl = fmaf(hf, -1.0f / 16384.0f, v);  // exact
                uh[q] = (uint32_t)hf;
                ul[q] = (uint32_t)(vl * 34359738368.0f);
                n64 = fma((double)(int)uh[q], snh, fma((double)(int)ul[q], snl, n64));
                any |= (uh[q] | ul[q]) != 0u;
            }
#pragma unroll
            for (int jr = 0; jr < X8_RD; ++jr) {
                const uint32_t* u = jr < 3 ? uh : ul;
                const int sh = 7 * (2 - jr % 3);
                R[jr][s] = (int)(((u[0] >> sh) & 127u) | (((u[1] >> sh) & 127u) << 8) |
                                 (((u[2] >> sh) & 127u) << 16) | (((u[3] >> sh) & 127u) << 24));
            }
        }

        // ---- M-step: feature digit columns x responsibility digits (a
        // block whose responsibilities are all exactly zero adds nothing)
        if (__builtin_amdgcn_ballot_w64(any) != 0) {
            const double sp0 = ldexp(1.0, e - 20);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                x8_mstep_tile<IB>(db, rofs, cb, j, R, sp0, acc[0][j]);
                x8_mstep_tile<IA>(db, rofs, ca, j, R, sp0, acc[1][j]);
            }
        }
        if (it + 1 < nblk && tid < X8_ROWS) ls[buf ^ 1][tid] = lsn;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's digit copies of the next block have landed
        __syncthreads();
    }

    // responsibility mass: lanes ci, ci+16, ci+32, ci+48 hold disjoint rows
    n64 += shfl_xor_d(n64, 16);
    n64 += shfl_xor_d(n64, 32);
    const int64_t gbase = (int64_t)g * ntiles * 16;
    if (h == 0) {
        double* np = npart + gbase + slot;
        *np = (accumulate ? *np : 0.0) + n64;
    }
    double* pc = part + (gbase + slot) * (2 * DP);
#pragma unroll
    for (int kind = 0; kind < 2; ++kind)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int dd = 16 * j + 4 * h + q;
                const int gexp = dd < d ? plan[(kind == 0 ? I8P_GB : I8P_GA) + dd] : 0;
                double* p2 = pc + (kind == 0 ? DP : 0) + dd;
                *p2 = (accumulate ? *p2 : 0.0) + ldexp(acc[kind][j][q], gexp);
            }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
hipError_t launch_i8_prologue(const Plan& pl, const float* w, const float* mu, const float* var,
                              const void* x, int64_t n, int64_t ldx, int dtype, hipStream_t st,
                              bool em_stats) {
    hipLaunchKernelGGL(k_i8_reset, dim3(1), dim3(128), 0, st, pl.i8_amax, pl.i8_lsb, pl.b16_amax,
                       pl.b16_lsb, pl.dp);
    if (n > 0) {
        int64_t b = (n + 2047) / 2048;
        const unsigned blocks = (unsigned)(b > 8192 ? 8192 : (b < 1 ? 1 : b));
        if (dtype == 0)
            hipLaunchKernelGGL(k_i8_xstats<float>, dim3(blocks), dim3(256), 0, st, (const float*)x, n,
                               pl.d, ldx, pl.dp, pl.shift, pl.i8_amax, pl.i8_lsb, pl.b16_amax,
                               pl.b16_lsb, pl.status);
        else
            hipLaunchKernelGGL(k_i8_xstats<uint16_t>, dim3(blocks), dim3(256), 0, st, (const uint16_t*)x,
                               n, pl.d, ldx, pl.dp, pl.shift, pl.i8_amax, pl.i8_lsb, pl.b16_amax,
                               pl.b16_lsb, pl.status);
    }
    hipLaunchKernelGGL(k_i8_plan, dim3(1), dim3(128), 0, st, pl.i8_amax, pl.i8_lsb, pl.d, pl.i8_plan,
                       pl.i8_dbl, pl.status);
    hipLaunchKernelGGL(k_i8_coef, dim3(pl.ntiles), dim3(256), 0, st, w, mu, var, pl.k, pl.d, pl.dp,
                       pl.shift, pl.i8_plan, pl.i8_dbl, pl.i8_coef, pl.i8_ek, pl.i8_tinfo, pl.status);
    const bool b16 = dtype != 0 && pl.b16_coef != nullptr && var != nullptr && em_stats;
    if (b16) {
        const hipError_t e = launch_b16_coef(pl, w, mu, var, st);
        if (e != hipSuccess) return e;
    }
    // (only an EM step runs a statistics pass on these kernels: k-means has its
    // own, the top-m assignment none)
    hipLaunchKernelGGL(k_i8_mode, dim3(1), dim3(64), 0, st, pl.status, pl.i8_plan, pl.d, pl.dp,
                       pl.i8_stats && em_stats ? 1 : 0, b16 ? 1 : 0, pl.shift);
    return hipGetLastError();
}

template <int NC, int LV, typename XT, int MODE>
static void launch_lse8_t(const Plan& pl, const void* x, int64_t n, int64_t ldx, double* lse_out,
                          int ll_acc, int32_t* z, int m, float* resp, hipStream_t st) {
    const int rows = L8_WAVES * (MODE >= 2 ? 2 : L8_RT) * 16;
    const int64_t blocks = (n + rows - 1) / rows;
    hipLaunchKernelGGL((k_lse8<NC, LV, XT, MODE>), dim3((unsigned)blocks), dim3(L8_WAVES * 64), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.dp, pl.shift, pl.i8_plan, pl.i8_coef, pl.i8_ek,
                       pl.i8_tinfo, pl.cvec, pl.ntiles, lse_out, pl.llpart, ll_acc, pl.i8_rows,
                       pl.status, z, pl.k, m, resp);
}

// Chunk counts a packed row can have at this dimension: ceil(dq t / 64) for
// t = Ia + Ib = 2 .. 2 * I8_MAX_DIGITS feature blocks, at most I8_MAX_NC
// (wider layouts fail the plan). Bit c of the result marks chunk count c.
int i8_nc_for(int d) {
    const int dq = (d + 15) / 16 * 16;
    int mask = 0;
    for (int t = 2; t <= 2 * I8_MAX_DIGITS; ++t) {
        const int nc = (dq * t + 63) / 64;
        if (nc <= I8_MAX_NC) mask |= 1 << nc;
    }
    return mask;
}

// Every variant whose chunk count the plan can produce, for both level
// counts; the plan's digit counts (on the device) let exactly one work.
template <typename XT, int MODE>
static hipError_t launch_lse8_all(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                  double* lse_out, int ll_acc, int32_t* z, int m, float* resp,
                                  hipStream_t st) {
#define VAR(NCV)                                                                                  \
    if (pl.i8_nc & (1 << NCV)) {                                                                  \
        launch_lse8_t<NCV, S8_LV, XT, MODE>(pl, x, n, ldx, lse_out, ll_acc, z, m, resp, st);      \
        launch_lse8_t<NCV, I8_MAX_LEV, XT, MODE>(pl, x, n, ldx, lse_out, ll_acc, z, m, resp, st); \
    }
    VAR(1) VAR(2) VAR(3) VAR(4) VAR(5) VAR(6)
#undef VAR
    return hipGetLastError();
}

hipError_t launch_lse8(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                       double* lse_out, int ll_acc, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    return dtype == 0 ? launch_lse8_all<float, 0>(pl, x, n, ldx, lse_out, ll_acc, nullptr, 0, nullptr, st)
                      : launch_lse8_all<uint16_t, 0>(pl, x, n, ldx, lse_out, ll_acc, nullptr, 0, nullptr, st);
}

hipError_t launch_lse8_km(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                          int32_t* z, int ll_acc, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    return dtype == 0 ? launch_lse8_all<float, 1>(pl, x, n, ldx, nullptr, ll_acc, z, 0, nullptr, st)
                      : launch_lse8_all<uint16_t, 1>(pl, x, n, ldx, nullptr, ll_acc, z, 0, nullptr, st);
}

// top-m mode (m <= 4): fp32 data only (the caller runs the fp64 pass for bf16)
hipError_t launch_lse8_topm(const Plan& pl, const void* x, int64_t n, int64_t ldx, double* lse_out,
                            int ll_acc, int m, int32_t* idx, float* resp, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    return m <= 2 ? launch_lse8_all<float, 2>(pl, x, n, ldx, lse_out, ll_acc, idx, m, resp, st)
                  : launch_lse8_all<float, 4>(pl, x, n, ldx, lse_out, ll_acc, idx, m, resp, st);
}

template <int DP, typename XT>
static hipError_t launch_stats8_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                  const double* lse, int acc, hipStream_t st) {
    int64_t rpg = ((n + pl.ngroups - 1) / pl.ngroups + STATS_ROWS - 1) / STATS_ROWS * STATS_ROWS;
    if (rpg < STATS_ROWS) rpg = STATS_ROWS;
    hipLaunchKernelGGL((k_stats8<DP, XT>), dim3(pl.ngroups * (pl.ntiles / 4)), dim3(256), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.i8_rows, pl.i8_coef, pl.i8_ek, pl.i8_tinfo,
                       pl.cvec, pl.shift, pl.i8_plan, pl.ntiles, lse, rpg, pl.part, pl.npart, acc,
                       pl.status);
    return hipGetLastError();
}

// The three digit-count variants of the int8 M-step pass (each returns at
// once unless the mode flag and the plan's digit counts select it).
template <int DP>
static hipError_t launch_stats8x_t(const Plan& pl, int64_t n, const double* lse, int acc,
                                   hipStream_t st) {
    int64_t rpg = ((n + pl.ngroups - 1) / pl.ngroups + X8_ROWS - 1) / X8_ROWS * X8_ROWS;
    if (rpg < X8_ROWS) rpg = X8_ROWS;
    const dim3 grid(pl.ngroups * (pl.ntiles / 4)), block(256);
#define VAR(IAV, IBV)                                                                          \
    hipLaunchKernelGGL((k_stats8x<DP, IAV, IBV>), grid, block, 0, st, pl.i8_rows, n, pl.d,     \
                       pl.i8_coef, pl.i8_ek, pl.i8_tinfo, pl.cvec, pl.i8_plan, pl.ntiles, lse, \
                       rpg, pl.part, pl.npart, acc, pl.status);
    static_assert(x8_counts_ok(1, 1) && x8_counts_ok(1, 2) && x8_counts_ok(2, 3), "variants");
    VAR(1, 1) VAR(1, 2) VAR(2, 3)
#undef VAR
    return hipGetLastError();
}

bool i8_stats_for(int dp) { return dp <= S8_MAX_DP; }

hipError_t launch_stats8(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                         const double* lse, int acc, hipStream_t st) {
    hipError_t e = hipErrorInvalidValue;
    switch (pl.dp) {
#define CASE(DPV)                                                                          \
    case DPV:                                                                              \
        e = dtype == 0 ? launch_stats8_t<DPV, float>(pl, x, n, ldx, lse, acc, st)         \
                       : launch_stats8_t<DPV, uint16_t>(pl, x, n, ldx, lse, acc, st);     \
        if (e == hipSuccess) e = launch_stats8x_t<DPV>(pl, n, lse, acc, st);              \
        break;
        CASE(16) CASE(32) CASE(48) CASE(64) CASE(80) CASE(96) CASE(112)
#undef CASE
    }
    return e;
}

}  // namespace gmm
