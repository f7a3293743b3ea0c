// gmm_kernels.hip - device kernels of the fused diagonal-GMM EM step (gfx950).
//
// One EM iteration is computed without ever writing the N x K responsibility
// matrix: the E-step log-densities of a tile of rows against a tile of
// components are formed in MFMA accumulators, turned into responsibilities in
// registers and immediately contracted against the same rows for the M-step
// statistics ("Flash-GMM: A Memory-Efficient Kernel for Scalable Soft
// Clustering", section 3: per-tile statistics accumulated globally in O(K*D)
// buffers; section 1: the responsibility matrix is what must not be
// materialised).
//
// Arithmetic
// ----------
// With a per-dimension shift s, a = x - s, w = 1/var, b = mu - s:
//   l[n][k] = sum_d ( w b a - w a^2 / 2 ) + c_k,
//   c_k     = log pi_k - 1/2 sum_d ( w b^2 + log var ) - D/2 log 2 pi.
// The sum over d is a dense contraction of feature rows [a, a^2] with
// coefficient rows [w b, -w/2] (the X^2 (1/var)^T and X (mu/var)^T products
// of the expanded Gaussian exponent). Both contractions of the step run on
// v_mfma_f64_16x16x4_f64: the expanded form cancels terms of size w a^2
// against each other, which fp32 cannot resolve for narrow components far
// from the shift (a component at the variance floor has w = 1e6), while in
// fp64 the features a, a^2 and all products and sums stay exact to ~1e-16.
//
// MFMA operand layout (16x16x4 f64, wave64): lane l = 16*h + i.
//   A operand: A[i][h]; B operand: B[h][i]; C: register q holds C[4q + h][i].
// E-step: A = feature (row i of a 16-row block), B = coefficient (component i
//   of a 16-wide K-tile); step t uses feature (dim 2t + (h>>1), power
//   1 + (h&1)); register q of lane (h, i) ends with l[row 4q+h][comp i].
// M-step: those registers, as r = exp(l - lse), are the A operand as they
//   stand: step q contracts A[comp i][h] = r[row 4q+h][comp i] with
//   B[h][j] = feature column 16J + j of row 4q + h; register q of lane (h, i)
//   accumulates S[comp 4q+h][feature 16J+i] = sum_n r[n][comp] f[n]. The
//   responsibilities never leave registers.
//
// Two passes per row chunk (the M-step of a component needs each row's
// normaliser over ALL components before any of its responsibilities exist):
//   pass 1 (k_lse):   row-stationary: every K-tile streams through LDS; per-row
//                     online logsumexp; writes lse per row and fp64
//                     log-likelihood partials (and the top-m components).
//   pass 2 (k_stats): K-tile-stationary: coefficients and statistics stay in
//                     registers; recomputes l with the same instruction
//                     sequence as pass 1, so both passes see bitwise identical
//                     log-densities.
// Partials are summed in a fixed order in fp64 by k_finalize: no atomics on
// floating-point data, bitwise reproducible results.
//
// k-means (Lloyd) step, the quantizer the pages' GMM replaces (same source,
// section 3): k_params without weights or variances gives coefficients with
// l = -|x - c|^2; k_lse with a top-1 list yields the assignment and sums the
// best l (minus the inertia); k_km_stats adds each row, one-hot, into its
// centroid's sums (no MFMA needed); k_kmfinal divides.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "gmm_device.h"
#include "gmm_internal.h"

namespace gmm {

// ---------------------------------------------------------------------------
// Prologue: parameter checks, shift, coefficient rows and constants.
// ---------------------------------------------------------------------------
__global__ void k_status_reset(int* status) {
    if (threadIdx.x < 16) status[threadIdx.x] = 0;
}

// (w and var null: k-means mode, centroids only; every weight counts as 1)
__global__ void k_validate(const float* __restrict__ w, const float* __restrict__ mu,
                           const float* __restrict__ var, int k, int d, int* status) {
    const int64_t total = (int64_t)k * d;
    int bad = 0, anypos = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float m = mu[i], v = var ? var[i] : 1.0f;
        if (!isfinite(m) || !isfinite(v) || !(v > 0.0f)) bad = 1;
        if (i < k) {
            const float wi = w ? w[i] : 1.0f;
            if (!isfinite(wi) || wi < 0.0f) bad = 1;
            if (wi > 0.0f) anypos = 1;
        }
    }
    if (bad) atomicOr(&status[0], 1);
    if (anypos) atomicOr(&status[1], 1);
}

// Shift s_d = rint(mean_k mu[k][d]) (one block per dim, fixed-order fp64
// sum), stored in the permuted dim order used by the kernels:
// pos(d) = (d & 1) * DP/2 + d / 2 (even dims, then odd dims).
__global__ void k_shift(const float* __restrict__ mu, int k, int d, int dp,
                        double* __restrict__ shift) {
    __shared__ double red[256];
    const int dd = blockIdx.x;
    double acc = 0.0;
    if (dd < d)
        for (int j = threadIdx.x; j < k; j += 256) acc += (double)mu[(int64_t)j * d + dd];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int sft = 128; sft > 0; sft >>= 1) {
        if (threadIdx.x < sft) red[threadIdx.x] += red[threadIdx.x + sft];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        double sv = dd < d ? rint(red[0] / (double)k) : 0.0;
        if (!isfinite(sv)) sv = 0.0;
        shift[(dd & 1) * (dp >> 1) + (dd >> 1)] = sv;
    }
}

// Coefficients of slot `blockIdx.x` (component = slot when slot < k, else
// padding with coefficient 0 and constant -inf), in operand order:
//   Pg[slot][h][t]: h&1 = 0 -> w*b of dim 2t+(h>>1), h&1 = 1 -> -w/2.
//   cvec[slot] = log pi - 1/2 sum_d (w b^2 + log var) - D/2 log 2pi.
// k-means mode (w and var null): w = 2 and no log terms, so that
//   l = sum_d (2 b a - a^2) - sum_d b^2 = -|x - c|^2 exactly.
__global__ void k_params(const float* __restrict__ w, const float* __restrict__ mu,
                         const float* __restrict__ var, int k, int d, int dp,
                         const double* __restrict__ shift, double* __restrict__ Pg,
                         double* __restrict__ cvec) {
    __shared__ double red[128];
    const int slot = blockIdx.x;
    const bool live = slot < k;
    const bool km = w == nullptr;
    const int dph = dp >> 1;
    double part = 0.0;
    double* row = Pg + (int64_t)slot * 2 * dp;
    for (int dd = threadIdx.x; dd < dp; dd += blockDim.x) {
        double cb = 0.0, cq = 0.0;
        if (live && dd < d) {
            const double s = shift[(dd & 1) * dph + (dd >> 1)];
            const double b = (double)mu[(int64_t)slot * d + dd] - s;
            if (km) {
                cb = 2.0 * b;
                cq = -1.0;
                part += 2.0 * b * b;
            } else {
                const double v = (double)var[(int64_t)slot * d + dd];
                const double iw = 1.0 / v;
                cb = iw * b;
                cq = -0.5 * iw;
                part += iw * b * b + log(v);
            }
        }
        const int t = dd >> 1, hh = (dd & 1) << 1;
        row[(hh + 0) * dph + t] = cb;
        row[(hh + 1) * dph + t] = cq;
    }
    red[threadIdx.x] = part;
    __syncthreads();
    for (int sft = blockDim.x >> 1; sft > 0; sft >>= 1) {
        if (threadIdx.x < sft) red[threadIdx.x] += red[threadIdx.x + sft];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double LOG_2PI = 1.8378770664093454835606594728112;
        cvec[slot] = !live ? -INFINITY
                     : km  ? -0.5 * red[0]
                           : log((double)w[slot]) - 0.5 * (red[0] + (double)d * LOG_2PI);
    }
}

// ---------------------------------------------------------------------------
// Pass 1: per-row logsumexp over all components.
// Block: 8 waves x 16 rows. Each lane holds the fp64 features of its row in
// E-operand order (feature (dim 2t + (h>>1), power 1 + (h&1)) for t = 0..
// DP/2-1), computed once; the K-tiles' coefficient rows and constants stream
// through three LDS buffers shared by the block's waves. Up to D = 96 a block
// has 4 waves (64 rows) and two blocks share a CU, so one block's prologue
// and epilogue overlap the other's MFMAs; above, 8 waves (128 rows; three
// buffers of 128-dim tiles leave LDS for one block). In k-means mode (km,
// with the k-means coefficients) the row's value is its best log-density.
// ---------------------------------------------------------------------------
template <int DP>
struct LseGeom {
    static constexpr int WAVES = DP <= 96 ? 4 : 8;
    static constexpr int ROWS = WAVES * 16;
    static constexpr int NT = WAVES * 64;
    static_assert(ROWS % LL_ROWS == 0 && LL_ROWS == 64, "one partial per 64 rows");
};

template <int DP, typename XT, int TM>
__global__ __launch_bounds__(LseGeom<DP>::NT, 8 / LseGeom<DP>::WAVES)
void k_lse(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
           const double* __restrict__ Pg, const double* __restrict__ cvec,
           const double* __restrict__ shift, int ntiles, double* __restrict__ lse_out,
           double* __restrict__ llpart, int ll_accumulate, int k, int m_out,
           int32_t* __restrict__ idx_out, float* __restrict__ resp_out, int km,
           const int* __restrict__ skip) {
    if (skip && *skip != 0) return;  // the int8-slice pass runs instead
    constexpr int DPH = DP / 2;
    constexpr int PSTR = 2 * DP + 2;  // LDS stride of one component (doubles)
    constexpr int TMA = TM > 0 ? TM : 1;
    constexpr int NT = LseGeom<DP>::NT;
    constexpr int LSE_ROWS = LseGeom<DP>::ROWS;
    __shared__ __attribute__((aligned(16))) double Pt[3][16 * PSTR];
    __shared__ double Ct[3][16];
    __shared__ double rowll[LSE_ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ci = lane & 15, h = lane >> 4, half = h >> 1;
    const bool sq = h & 1;
    const int64_t rowb = (int64_t)blockIdx.x * LSE_ROWS + wave * 16;

    double fe[DPH];
    {
        const int64_t row = rowb + ci;
        const bool ok = row < n;
        const XT* xp = x + (ok ? row : 0) * ldx;
#pragma unroll
        for (int t = 0; t < DPH; ++t) {
            const int dd = 2 * t + half;
            const float xv = (ok && dd < d) ? load_x(xp + dd) : 0.0f;
            fe[t] = feat(xv, shift[half * DPH + t], sq);
        }
    }

    // K-tiles stream through three LDS buffers: in iteration t the waves
    // read tile t from buffer t%3 while tile t+2 is written to buffer
    // (t+2)%3 (last read in iteration t-1). So the one barrier per tile never
    // separates a buffer's writes from its reads by less than a full
    // iteration, and the first coefficients of tile t+1 (written in iteration
    // t-1) are read before the barrier that ends iteration t: a wave starts
    // its next MFMA chain as soon as it leaves the barrier. Up to D = 96 the
    // global loads of a tile are also issued one iteration ahead of its LDS
    // stores, so no wave waits on an L2 round trip inside the loop.
    constexpr int NBUF = 3;
    constexpr int SPT = (16 * DP + NT - 1) / NT;  // coefficient pairs per thread
    double pvx[2 * SPT];
    double cv = 0.0;
    auto gload = [&](int tile) {
        const double* src = Pg + (int64_t)tile * 16 * 2 * DP;
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int i = tid + NT * u;
            if (SPT * NT == 16 * DP || i < 16 * DP) { const double2 v = *(const double2*)(src + 2 * i); pvx[2 * u] = v.x; pvx[2 * u + 1] = v.y; }
        }
        if (tid < 16) cv = cvec[tile * 16 + tid];
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int i = tid + NT * u;
            if (SPT * NT == 16 * DP || i < 16 * DP) {
                const int e = 2 * i;
                const int comp = e / (2 * DP), off = e % (2 * DP);
                *(double2*)&Pt[buf][comp * PSTR + off] = double2{pvx[2 * u], pvx[2 * u + 1]};
            }
        }
        if (tid < 16) Ct[buf][tid] = cv;
    };

    double m[4];
    float s[4];
    double tv[4][TMA];
    int ti[4][TMA];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        m[q] = -1.0e300;
        s[q] = 0.0f;
#pragma unroll
        for (int j = 0; j < TMA; ++j) { tv[q][j] = -INFINITY; ti[q][j] = 0x7fffffff; }
    }

    // Above D = 96 (or with the longer top-m lists) the register budget is
    // spent: tile t+2 is loaded and stored at the top of iteration t.
    constexpr bool AHEAD = DP <= 128 && TM <= 2;
    auto stage_now = [&](int tile, int buf) {
        const double* src = Pg + (int64_t)tile * 16 * 2 * DP;
        for (int i = tid; i < 16 * DP; i += NT) {  // pairs of doubles
            const int e = 2 * i;
            const int comp = e / (2 * DP), off = e % (2 * DP);
            *(double2*)&Pt[buf][comp * PSTR + off] = *(const double2*)(src + e);
        }
        if (tid < 16) Ct[buf][tid] = cvec[tile * 16 + tid];
    };
    if constexpr (AHEAD) {
        gload(0);
        lstore(0);
        gload(ntiles > 1 ? 1 : 0);
        lstore(1);
        gload(ntiles > 2 ? 2 : ntiles - 1);
    } else {
        stage_now(0, 0);
        if (ntiles > 1) stage_now(1, 1);
    }
    __syncthreads();

    // coefficients stream from LDS through a two-batch register ring
    // (shorter batches where the features or top-m lists fill the registers)
    constexpr int EB = (DP >= 128 || TM > 2) ? 4 : 8;
    constexpr int NBT = DPH / EB;
    double2 ring[2][EB / 2];
    {
        const double* pp = &Pt[0][ci * PSTR + h * DPH];
#pragma unroll
        for (int u = 0; u < EB / 2; ++u) ring[0][u] = *(const double2*)(pp + 2 * u);
    }
    // The finished tile's values are folded into the running normaliser
    // (and top-m list) while the next tile's MFMAs run: lp/cp/pidx hold the
    // previous tile (none before tile 0: -inf values with an index that
    // never enters a top-m list).
    f64x4 lp = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    double cp = 0.0;
    int pidx = 0x7fffffff;
    double cc = Ct[0][ci];
    auto fold = [&]() {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double l = lp[q] + cp;
            lse_push(m[q], s[q], l);
            if constexpr (TM > 0) top_push_inc<TM>(tv[q], ti[q], l, pidx);
        }
    };
    // pins the fold's results at this point of the instruction stream (the
    // compiler would otherwise sink the arithmetic into a later tile)
    auto pin_fold = [&]() {
#pragma unroll
        for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(m[q]), "+v"(s[q]));
    };
    // One tile; its buffer index is a compile-time constant so that every
    // LDS address is one base register plus an immediate offset.
    auto tile_step = [&](int tile, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        constexpr int bnext = (buf + 1) % NBUF;
        constexpr int bstore = (buf + 2) % NBUF;
        // nothing moves between tiles (the fold of tile t-1 stays in tile t)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (AHEAD) {
            // unconditional: past the last tile these write a buffer that is
            // never read again (the loads are clamped to the last tile)
            lstore(bstore);
            gload(tile + 3 < ntiles ? tile + 3 : ntiles - 1);
        } else if (tile + 2 < ntiles) {
            stage_now(tile + 2, bstore);
        }
        const double* pp = &Pt[buf][ci * PSTR + h * DPH];
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) {
            const int cur = bt & 1;
            if (bt + 1 < NBT) {
#pragma unroll
                for (int u = 0; u < EB / 2; ++u)
                    ring[cur ^ 1][u] = *(const double2*)(pp + (bt + 1) * EB + 2 * u);
            }
#pragma unroll
            for (int u = 0; u < EB / 2; ++u) {
                const int t = bt * EB + 2 * u;
                acc = mfma4d(fe[t + 0], ring[cur][u].x, acc);
                acc = mfma4d(fe[t + 1], ring[cur][u].y, acc);
            }
            if (bt == 0) fold();
            if (bt + 1 < NBT) __builtin_amdgcn_sched_group_barrier(0x100, EB / 2, 0);
            if (bt == 0) {
                // the previous tile's fold spread over this batch's MFMAs
#pragma unroll
                for (int u = 0; u < EB; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, TM > 0 ? 12 : 6, 0);
                }
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, EB, 0);
            }
        }
        // the next tile's first batch and constant (written one iteration
        // earlier), then this tile's result becomes the one to fold
        {
            const double* pn = &Pt[bnext][ci * PSTR + h * DPH];
#pragma unroll
            for (int u = 0; u < EB / 2; ++u) ring[0][u] = *(const double2*)(pn + 2 * u);
        }
        lp = acc;
        cp = cc;
        cc = Ct[bnext][ci];
        pidx = tile * 16 + ci;
        pin_fold();
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    int tile = 0;
    for (; tile + 3 <= ntiles; tile += 3) {
        tile_step(tile, B0{});
        tile_step(tile + 1, B1{});
        tile_step(tile + 2, B2{});
    }
    if (tile < ntiles) tile_step(tile, B0{});
    if (tile + 1 < ntiles) tile_step(tile + 1, B1{});
    fold();

    // Merge the 16 lanes that hold the same rows (fixed butterfly order).
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll 1
        for (int off = 1; off < 16; off <<= 1) {
            const double m2 = shfl_xor_d(m[q], off);
            const float s2 = __shfl_xor(s[q], off);
            lse_merge(m[q], s[q], m2, s2);
            if constexpr (TM > 0) top_merge<TM>(tv[q], ti[q], off);
        }
    }
    if (ci == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int lr = wave * 16 + 4 * q + h;
            const int64_t row = (int64_t)blockIdx.x * LSE_ROWS + lr;
            double v = 0.0;
            if (row < n) {
                // k-means mode: the row's value is its best log-density,
                // -|x - c_z|^2 (the row's contribution to -inertia)
                if constexpr (TM > 0) v = km ? tv[q][0] : m[q] + log((double)s[q]);
                else v = m[q] + log((double)s[q]);
                if (lse_out) lse_out[row] = v;
                if constexpr (TM > 0) {
                    for (int j = 0; j < m_out; ++j) {
                        const int sl = ti[q][j];
                        idx_out[row * m_out + j] = sl < k ? sl : -1;
                        if (resp_out) resp_out[row * m_out + j] = __expf((float)(tv[q][j] - v));
                    }
                }
            }
            rowll[lr] = v;
        }
    }
    __syncthreads();
    // Fixed-order sums of the block's rows, one partial per 64 rows: wave w
    // (w < rows / 64) takes rows 64w + lane, then a butterfly over the lanes.
    if (wave < LSE_ROWS / LL_ROWS) {
        double tot = rowll[wave * 64 + lane];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) tot += shfl_xor_d(tot, off);
        const int64_t pi = (int64_t)blockIdx.x * (LSE_ROWS / LL_ROWS) + wave;
        if (lane == 0) llpart[pi] = (ll_accumulate ? llpart[pi] : 0.0) + tot;
    }
}

// ---------------------------------------------------------------------------
// Pass 2: statistics. Block = WV waves; wave w owns K-tile kg*WV + w (16
// components): its coefficient rows stay in registers and its statistics in
// fp64 MFMA accumulators. The block walks the rows of its row group in
// 32-row tiles whose fp64 features are staged (double-buffered) in LDS as
// feats[row][p][t] = power (1 + (p&1)) of dim 2t + (p>>1), the E-operand order,
// so the E-step reads its A operand directly and the M-step reads a single
// feature per MFMA.
//
// Schedule of one tile (one wave has a SIMD to itself, so nothing else hides
// its non-MFMA work): the E-step MFMAs of tile it are interleaved with the
// staging of tile it+1 (LDS stores of values loaded one iteration earlier)
// and the global loads of tile it+2; then the responsibilities; then the
// M-step, whose feature reads run one 4-row group ahead of its MFMAs. Row
// indices are clamped instead of branched on so that the staging stays in
// the E-step's basic block; values of rows outside the row group are zeroed.
// ---------------------------------------------------------------------------

template <int DP>
struct StatsGeom {
    static constexpr int DPH = DP / 2;
    // LDS strides (doubles) chosen so that neither pass's reads conflict on
    // the 32 four-byte banks:
    // * HS, one (parity, power) section, is 4 mod 8: an M-step read (16
    //   lanes: dims 16J + ci of one row, even ci in section 0 and odd ci in
    //   section 2, 8 doubles each) covers banks 2k and 2k + 4*HS = 2k + 16;
    // * S, one row, is 2 mod 4: an E-step 16-byte read (8 lanes: rows ci of
    //   one section) starts at bank 2*S*ci = 4*ci mod 32.
    static constexpr int HS = DPH + 4;
    static constexpr int S = 4 * HS + 2;
    static constexpr int WV = DP <= 64 ? 8 : 4;  // 8 waves fit 256 registers each only up to 64
    static constexpr int NT = WV * 64;
    static constexpr int PER = (STATS_ROWS * DP + NT - 1) / NT;  // x values per thread
    static_assert(PER * NT == STATS_ROWS * DP, "every thread stages the same number of values");
};

template <int DP, typename XT>
__global__ __launch_bounds__(StatsGeom<DP>::NT, 1)
void k_stats(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
             const double* __restrict__ Pg, const double* __restrict__ cvec,
             const double* __restrict__ shift, int ntiles, const double* __restrict__ lse,
             int64_t rows_per_group, double* __restrict__ part, double* __restrict__ npart,
             int accumulate, const int* __restrict__ skip) {
    if (skip && *skip != 0) return;  // the int8-slice statistics pass runs instead
    using G = StatsGeom<DP>;
    constexpr int DPH = G::DPH, HS = G::HS, S = G::S, WV = G::WV, NT = G::NT, PER = G::PER;
    constexpr int NJ = DP / 16;  // 16-dim column blocks per power
    constexpr int EB = DPH % 8 == 0 ? 8 : DPH;  // E-step t-steps per batch
    constexpr int NB = DPH / EB;                // E-step batches
    static_assert(PER % NB == 0, "staging slices must split evenly over the E batches");
    constexpr int SL = PER / NB;                // staged values per batch
    __shared__ __attribute__((aligned(16))) double fs[2][STATS_ROWS * S];
    __shared__ double ls[2][STATS_ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ci = lane & 15, h = lane >> 4;
    const int kgroups = ntiles / WV;
    // Workgroups are dispatched to the 8 XCDs round-robin by index. Remap so
    // that the blocks of one XCD take consecutive (row group, K-group) pairs:
    // all K-groups of a row group then run on one XCD and share its L2 copy
    // of each row tile instead of fetching it from HBM once per XCD.
    const int nb = gridDim.x;
    const int o = (nb % 8 == 0) ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
    const int g = o / kgroups;
    const int tile = (o % kgroups) * WV + wave;
    const int slot = tile * 16 + ci;

    // Stationary coefficients: P[slot][h][t], t = 0..DPH-1.
    double pr[DPH];
    {
        const double* src = Pg + (int64_t)slot * 2 * DP + h * DPH;
#pragma unroll
        for (int t = 0; t < DPH; t += 2) {
            const double2 v = *(const double2*)(src + t);
            pr[t] = v.x;
            pr[t + 1] = v.y;
        }
    }
    const double cc = cvec[slot];

    f64x4 acc[2 * NJ];
#pragma unroll
    for (int j = 0; j < 2 * NJ; ++j) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
    double n64 = 0.0;

    const int64_t gr0 = (int64_t)g * rows_per_group;
    int64_t gr1 = gr0 + rows_per_group;
    if (gr1 > n) gr1 = n;
    const int64_t ntile_rows = gr1 > gr0 ? (gr1 - gr0 + STATS_ROWS - 1) / STATS_ROWS : 0;

    // Staging: thread tid handles elements tid + NT*i of the tile's
    // STATS_ROWS x DP values (row-major, coalesced global reads). Loads go
    // through a buffer resource built per tile (scalar instructions only):
    // its range ends after the last valid value of the tile's last row in
    // the row group, and the buffer unit returns 0 for offsets past it, so
    // rows past the row group need no clamping or select. Padding dims use
    // an offset past every range and read as 0 too. The per-element offsets
    // are loop-invariant: no vector instruction is spent on addressing.
    float xv[PER];
    double lv = 0.0;
    double shv[PER];     // shift of the dims this thread stages
    uint32_t xoff[PER];  // byte offset of the element within its tile
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
        // normalisers: rows past the row group get +inf (responsibility 0)
        const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(lse + rbase), (short)0, (int)(nv * (int64_t)sizeof(double)), BUF_RSRC_WORD3);
        const int lrow = tid & (STATS_ROWS - 1);
        const double v = buf_load_f64(lr, (uint32_t)lrow * 8u);
        lv = lrow < nv ? v : INFINITY;
    };
    // (several threads write the same normaliser: same value, same slot)
    auto storel = [&](double* lsb) { lsb[tid & (STATS_ROWS - 1)] = lv; };
    auto store1 = [&](double* fsb, int i) {
        const int e = tid + NT * i;
        const int r = e / DP, dd = e % DP;
        const int pp = 2 * (dd & 1), t = dd >> 1;
        const double a = (double)xv[i] - shv[i];
        fsb[r * S + pp * HS + t] = a;
        fsb[r * S + (pp + 1) * HS + t] = a * a;
    };

    if (ntile_rows > 0) {
        load(0);
#pragma unroll
        for (int i = 0; i < PER; ++i) store1(fs[0], i);
        storel(ls[0]);
        load(1);
    }
    __syncthreads();

    // One tile; BUF (the LDS buffer holding tile it) is a compile-time
    // constant so every LDS address is a register plus an immediate offset.
    auto tile_step = [&](int64_t it, auto bufc) {
        constexpr int BUF = decltype(bufc)::value;
        const double* fb = fs[BUF];
        // E-step for both 16-row blocks as two independent MFMA chains:
        // register q of lane (h, ci) of chain rb -> l[row 16rb + 4q + h][slot].
        // Interleaved: LDS stores of tile it+1 (its values arrived during the
        // previous iteration) and the global loads of tile it+2. Buffer BUF^1
        // was last read before the previous iteration's closing barrier.
        const double* fa0 = fb + ci * S + h * HS;
        const double* fa1 = fa0 + 16 * S;
        f64x4 e0 = {0.0, 0.0, 0.0, 0.0}, e1 = {0.0, 0.0, 0.0, 0.0};
        // Features stream from LDS through a two-batch register ring, so each
        // batch's reads are in flight during the previous batch's MFMAs.
        double2 ring0[2][EB / 2], ring1[2][EB / 2];
#pragma unroll
        for (int u = 0; u < EB / 2; ++u) {
            ring0[0][u] = *(const double2*)(fa0 + 2 * u);
            ring1[0][u] = *(const double2*)(fa1 + 2 * u);
        }
        double lsr[2][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            lsr[0][q] = ls[BUF][4 * q + h];
            lsr[1][q] = ls[BUF][16 + 4 * q + h];
        }
        storel(ls[BUF ^ 1]);
        __builtin_amdgcn_sched_group_barrier(0x100, EB + 8, 0);
#pragma unroll
        for (int bt = 0; bt < NB; ++bt) {
            const int cur = bt & 1;
            if (bt + 1 < NB) {
#pragma unroll
                for (int u = 0; u < EB / 2; ++u) {
                    ring0[cur ^ 1][u] = *(const double2*)(fa0 + (bt + 1) * EB + 2 * u);
                    ring1[cur ^ 1][u] = *(const double2*)(fa1 + (bt + 1) * EB + 2 * u);
                }
            }
#pragma unroll
            for (int u = 0; u < EB / 2; ++u) {
                const int t = bt * EB + 2 * u;
                e0 = mfma4d(ring0[cur][u].x, pr[t + 0], e0);
                e1 = mfma4d(ring1[cur][u].x, pr[t + 0], e1);
                e0 = mfma4d(ring0[cur][u].y, pr[t + 1], e0);
                e1 = mfma4d(ring1[cur][u].y, pr[t + 1], e1);
            }
#pragma unroll
            for (int i = bt * SL; i < (bt + 1) * SL; ++i) store1(fs[BUF ^ 1], i);
            // order: next batch's LDS reads, then this batch's MFMAs with the
            // staging stores spread between them
            if (bt + 1 < NB) __builtin_amdgcn_sched_group_barrier(0x100, EB, 0);
#pragma unroll
            for (int u = 0; u < 2 * EB; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                if (u % 8 == 0) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            }
        }
        // the next-but-one tile's values are loaded once this tile's staging
        // registers have been written to LDS
        load(it + 2);
        __builtin_amdgcn_sched_barrier(0);
        double r[2][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            r[0][q] = exp_f64range(e0[q] + cc - lsr[0][q]);
            r[1][q] = exp_f64range(e1[q] + cc - lsr[1][q]);
            n64 += r[0][q];
            n64 += r[1][q];
        }
        // M-step: A = r (component ci, row 16rb + 4q + h), B = feature
        // column 16j + ci of that row (a, then a^2, both read from LDS). The
        // features of the next 4-row group are read while this group's
        // MFMAs run. A group whose 64 responsibilities are all exactly zero
        // (fp64 exp underflow) is skipped: its MFMAs would add exact zeros.
        double fc[NJ], qc[NJ], fn[NJ], qn[NJ];
        auto mread = [&](int grp, double (&f)[NJ], double (&fq)[NJ]) {
            const double* fm = fb + ((grp >> 2) * 16 + 4 * (grp & 3) + h) * S;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int dd = 16 * j + ci;
                f[j] = fm[2 * (dd & 1) * HS + (dd >> 1)];
                fq[j] = fm[(2 * (dd & 1) + 1) * HS + (dd >> 1)];
            }
        };
        mread(0, fc, qc);
#pragma unroll
        for (int grp = 0; grp < 8; ++grp) {
            if (grp + 1 < 8) mread(grp + 1, fn, qn);
            const double rv = r[grp >> 2][grp & 3];
            if (__builtin_amdgcn_ballot_w64(rv != 0.0) != 0) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[j] = mfma4d(rv, fc[j], acc[j]);
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[NJ + j] = mfma4d(rv, qc[j], acc[NJ + j]);
            }
            if (grp + 1 < 8) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    fc[j] = fn[j];
                    qc[j] = qn[j];
                }
            }
        }
        __syncthreads();
    };
    for (int64_t it = 0; it < ntile_rows; it += 2) {
        tile_step(it, std::integral_constant<int, 0>());
        if (it + 1 < ntile_rows) tile_step(it + 1, std::integral_constant<int, 1>());
    }

    // Responsibility mass: lanes ci, ci+16, ci+32, ci+48 hold disjoint rows.
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
            double* p = part + (gbase + comp) * (2 * DP) + 16 * j + ci;
            *p = (accumulate ? *p : 0.0) + acc[j][q];
        }
}

// ---------------------------------------------------------------------------
// Finalize: fixed-order fp64 sum over row groups, then the M-step update.
// ---------------------------------------------------------------------------
__global__ void k_finalize(const double* __restrict__ part, const double* __restrict__ npart,
                           int ngroups, int kp, int dp, int d, int k,
                           const double* __restrict__ shift, int64_t n, float var_floor,
                           float* __restrict__ w, float* __restrict__ mu, float* __restrict__ var,
                           const int* __restrict__ status) {
    const int comp = blockIdx.x;
    if (comp >= k) return;
    const bool bad = status[0] != 0 || status[1] == 0;
    double N = 0.0;
    for (int gg = 0; gg < ngroups; ++gg) N += npart[(int64_t)gg * kp + comp];
    const int dph = dp >> 1;
    for (int dd = threadIdx.x; dd < d; dd += blockDim.x) {
        double s1 = 0.0, s2 = 0.0;
        for (int gg = 0; gg < ngroups; ++gg) {
            const double* p = part + ((int64_t)gg * kp + comp) * 2 * dp;
            s1 += p[dd];
            s2 += p[dp + dd];
        }
        const int64_t e = (int64_t)comp * d + dd;
        if (bad) {
            mu[e] = NAN;
            var[e] = NAN;
        } else if (N > 0.0) {
            const double sh = shift[(dd & 1) * dph + (dd >> 1)];
            const double m1 = s1 / N;
            const double v = s2 / N - m1 * m1;
            mu[e] = (float)(sh + m1);
            var[e] = (float)(v > (double)var_floor ? v : (double)var_floor);
        }
    }
    // A component with positive mass keeps a positive fp32 weight: below the
    // smallest fp32 value its weight is stored as that value instead of 0,
    // which would remove it for good (log 0). While a weight is that small its
    // mean and variance do not depend on it (the weight cancels from their
    // weighted averages).
    if (threadIdx.x == 0) {
        float wf = (float)(N / (double)n);
        if (N > 0.0 && wf == 0.0f) wf = __int_as_float(1);  // smallest positive fp32
        w[comp] = bad ? NAN : (N > 0.0 ? wf : 0.0f);
    }
}

// Fixed-order fp64 sum of the per-block log-likelihood partials, times
// `scale` (1 for the log-likelihood; -1 turns the k-means mode's summed best
// log-densities -|x - c_z|^2 into the inertia).
__global__ void k_ll_final(const double* __restrict__ llpart, int nparts, double* __restrict__ out,
                           const int* __restrict__ status, double scale) {
    __shared__ double red[256];
    double acc = 0.0;
    const int per = (nparts + 255) / 256;
    const int lo = threadIdx.x * per;
    for (int i = lo; i < lo + per && i < nparts; ++i) acc += llpart[i];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int sft = 128; sft > 0; sft >>= 1) {
        if (threadIdx.x < sft) red[threadIdx.x] += red[threadIdx.x + sft];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        *out = (status[0] != 0 || status[1] == 0) ? NAN : scale * red[0];
}

// k-means statistics (one-hot responsibilities from the assignment z): for
// row group g and K-tile t (16 centroids), the sum of a = x - s over the rows
// assigned to each centroid of the tile, and their count, in the layout of
// the statistics pass's partials. The 8 waves of a block take consecutive
// eighths of the row group; a wave reads the assignments of 64 * KMS_ZB
// rows at a time, writes the rows assigned to the tile (row offset and
// centroid, in row order) to a list of its own in LDS, then loads the
// listed rows KMS_BATCH at a time and adds them, in row order, into its own
// LDS accumulator (each lane owns two dims, so no two lanes touch one
// element). With 16 of K centroids a tile matches about 16/K of the rows:
// the list keeps the load batches full. The eight accumulators are summed
// in a fixed order at the end. Every row is read by exactly one block; no
// MFMA work is needed.
constexpr int KMS_WAVES = 8;
constexpr int KMS_BATCH = 16;  // matched rows loaded at once
constexpr int KMS_ZB = 8;      // 64-row chunks of assignments listed at once

template <int DP, typename XT>
__global__ __launch_bounds__(KMS_WAVES * 64)
void k_km_stats(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
                const double* __restrict__ shift, const int32_t* __restrict__ z, int ntiles,
                int64_t rows_per_group, double* __restrict__ part, double* __restrict__ npart,
                int accumulate) {
    static_assert(DP <= 128, "two dims per lane");
    constexpr int KS = 128;  // accumulator row stride: every lane's two dims fit
    __shared__ double kacc[KMS_WAVES][16 * KS];
    __shared__ int kcnt[KMS_WAVES][16];
    // per wave: the matched rows of 64 * KMS_ZB rows, (offset << 4) | centroid
    __shared__ int klist[KMS_WAVES][64 * KMS_ZB];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x / ntiles, tile = blockIdx.x - g * ntiles;
    const int kp = ntiles * 16, c0 = tile * 16;
    double* my = kacc[wave];
    int* lst = klist[wave];
    for (int i = lane; i < 16 * KS; i += 64) my[i] = 0.0;
    if (lane < 16) kcnt[wave][lane] = 0;
    constexpr int DPH = DP / 2;
    const int dA = lane, dB = lane + 64;
    const double sA = dA < d ? shift[(dA & 1) * DPH + (dA >> 1)] : 0.0;
    const double sB = dB < d ? shift[(dB & 1) * DPH + (dB >> 1)] : 0.0;
    // a row is read through a buffer resource that ends after its d values:
    // lanes past d read 0 (and add 0 to accumulator padding), no branches
    const uint32_t oA = (uint32_t)(dA * sizeof(XT)), oB = (uint32_t)(dB * sizeof(XT));
    const int rbytes = (int)(d * sizeof(XT));
    const int64_t r0 = (int64_t)g * rows_per_group;
    const int64_t r1 = r0 + rows_per_group < n ? r0 + rows_per_group : n;
    const int64_t span = r1 > r0 ? r1 - r0 : 0;
    const int64_t per = (span + KMS_WAVES - 1) / KMS_WAVES;
    const int64_t wa = per * wave < span ? per * wave : span;
    const int64_t wb = per * (wave + 1) < span ? per * (wave + 1) : span;
    const int64_t w0 = r0 + wa, w1 = r0 + wb;
    for (int64_t rz = w0; rz < w1; rz += 64 * KMS_ZB) {
        int zc[KMS_ZB];
#pragma unroll
        for (int u = 0; u < KMS_ZB; ++u) {
            const int64_t r = rz + 64 * u + lane;
            zc[u] = (r < w1 ? z[r] : -1) - c0;
        }
        // list the matched rows in row order (chunk u, then lane)
        int nl = 0;  // uniform
#pragma unroll
        for (int u = 0; u < KMS_ZB; ++u) {
            const bool hit = (unsigned)zc[u] < 16u;
            const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
            const int pos = nl + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (hit) lst[pos] = ((64 * u + lane) << 4) | zc[u];
            nl += __builtin_popcountll(m);
        }
        __builtin_amdgcn_wave_barrier();
        for (int b0 = 0; b0 < nl; b0 += KMS_BATCH) {
            int cb[KMS_BATCH];
            float xa[KMS_BATCH], xb[KMS_BATCH];
#pragma unroll
            for (int i = 0; i < KMS_BATCH; ++i) {
                // past the list's end: its first entry of the batch again
                // (loaded but not added)
                const int e = __builtin_amdgcn_readfirstlane(lst[b0 + i < nl ? b0 + i : b0]);
                cb[i] = e & 15;
                const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(x + (rz + (e >> 4)) * ldx), (short)0, rbytes, BUF_RSRC_WORD3);
                xa[i] = buf_load_x<XT>(xr, oA);
                xb[i] = buf_load_x<XT>(xr, oB);
            }
#pragma unroll
            for (int i = 0; i < KMS_BATCH; ++i) {
                if (b0 + i < nl) {
                    double* ar = my + cb[i] * KS;
                    ar[dA] += (double)xa[i] - sA;
                    ar[dB] += (double)xb[i] - sB;
                    if (lane == 0) kcnt[wave][cb[i]] += 1;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    for (int i = tid; i < 16 * KS; i += KMS_WAVES * 64) {
        const int cc = i / KS, dd = i - cc * KS;
        if (dd < d) {
            double sum = 0.0;
#pragma unroll
            for (int w = 0; w < KMS_WAVES; ++w) sum += kacc[w][i];
            double* p = part + ((int64_t)g * kp + c0 + cc) * 2 * DP + dd;
            *p = (accumulate ? *p : 0.0) + sum;
        }
    }
    if (tid < 16) {
        int cnt = 0;
#pragma unroll
        for (int w = 0; w < KMS_WAVES; ++w) cnt += kcnt[w][tid];
        double* np = npart + (int64_t)g * kp + c0 + tid;
        *np = (accumulate ? *np : 0.0) + (double)cnt;
    }
}

// k-means update: c'[k] = s + S1[k] / N[k] for a non-empty cluster (fixed-
// order fp64 sums over the row groups), the input centroid otherwise.
__global__ void k_kmfinal(const double* __restrict__ part, const double* __restrict__ npart,
                          int ngroups, int kp, int dp, int d, int k,
                          const double* __restrict__ shift, float* __restrict__ c,
                          const int* __restrict__ status) {
    const int comp = blockIdx.x;
    if (comp >= k) return;
    const bool bad = status[0] != 0;
    double N = 0.0;
    for (int gg = 0; gg < ngroups; ++gg) N += npart[(int64_t)gg * kp + comp];
    const int dph = dp >> 1;
    for (int dd = threadIdx.x; dd < d; dd += blockDim.x) {
        double s1 = 0.0;
        for (int gg = 0; gg < ngroups; ++gg) s1 += part[((int64_t)gg * kp + comp) * 2 * dp + dd];
        const int64_t e = (int64_t)comp * d + dd;
        if (bad) c[e] = NAN;
        else if (N > 0.0) c[e] = (float)(shift[(dd & 1) * dph + (dd >> 1)] + s1 / N);
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI in gmm_api.hip).
// ---------------------------------------------------------------------------
template <int DP, typename XT, int TM>
static hipError_t launch_lse_tm(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                double* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                                int km, hipStream_t st, const int* skip) {
    using G = LseGeom<DP>;
    const int64_t blocks = (n + G::ROWS - 1) / G::ROWS;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_lse<DP, XT, TM>), dim3((unsigned)blocks), dim3(G::NT), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.Pg, pl.cvec, pl.shift, pl.ntiles, lse_out,
                       pl.llpart, ll_acc, pl.k, m, idx, resp, km, skip);
    return hipGetLastError();
}

template <int DP, typename XT>
static hipError_t launch_lse_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                               double* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                               int km, hipStream_t st, const int* skip) {
    if (m <= 0) return launch_lse_tm<DP, XT, 0>(pl, x, n, ldx, lse_out, ll_acc, 0, idx, resp, 0, st, skip);
    if (m == 1) return launch_lse_tm<DP, XT, 1>(pl, x, n, ldx, lse_out, ll_acc, m, idx, resp, km, st, skip);
    if (m == 2) return launch_lse_tm<DP, XT, 2>(pl, x, n, ldx, lse_out, ll_acc, m, idx, resp, km, st, skip);
    return launch_lse_tm<DP, XT, 4>(pl, x, n, ldx, lse_out, ll_acc, m, idx, resp, km, st, skip);
}

template <int DP, typename XT>
static hipError_t launch_stats_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                 const double* lse, int acc, hipStream_t st, const int* skip) {
    using G = StatsGeom<DP>;
    int64_t rpg = ((n + pl.ngroups - 1) / pl.ngroups + STATS_ROWS - 1) / STATS_ROWS * STATS_ROWS;
    if (rpg < STATS_ROWS) rpg = STATS_ROWS;
    hipLaunchKernelGGL((k_stats<DP, XT>), dim3(pl.ngroups * (pl.ntiles / G::WV)), dim3(G::NT), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.Pg, pl.cvec, pl.shift, pl.ntiles, lse, rpg,
                       pl.part, pl.npart, acc, skip);
    return hipGetLastError();
}

#define GMM_DP_CASES(M) M(16) M(32) M(48) M(64) M(80) M(96) M(112) M(128)

hipError_t launch_lse(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                      double* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                      hipStream_t st, int km, const int* skip) {
    switch (pl.dp) {
#define CASE(DPV)                                                                          \
    case DPV:                                                                              \
        return dtype == 0 ? launch_lse_t<DPV, float>(pl, x, n, ldx, lse_out, ll_acc, m, idx, \
                                                     resp, km, st, skip)                    \
                          : launch_lse_t<DPV, uint16_t>(pl, x, n, ldx, lse_out, ll_acc, m,   \
                                                        idx, resp, km, st, skip);
        GMM_DP_CASES(CASE)
#undef CASE
    }
    return hipErrorInvalidValue;
}

template <int DP, typename XT>
static hipError_t launch_km_stats_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                    const int32_t* z, int acc, hipStream_t st) {
    int64_t rpg = (n + pl.ngroups - 1) / pl.ngroups;
    if (rpg < 1) rpg = 1;
    hipLaunchKernelGGL((k_km_stats<DP, XT>), dim3(pl.ngroups * pl.ntiles), dim3(KMS_WAVES * 64), 0,
                       st, (const XT*)x, n, pl.d, ldx, pl.shift, z, pl.ntiles, rpg, pl.part,
                       pl.npart, acc);
    return hipGetLastError();
}

hipError_t launch_km_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                           const int32_t* z, int acc, hipStream_t st) {
    switch (pl.dp) {
#define CASE(DPV)                                                                      \
    case DPV:                                                                          \
        return dtype == 0 ? launch_km_stats_t<DPV, float>(pl, x, n, ldx, z, acc, st) \
                          : launch_km_stats_t<DPV, uint16_t>(pl, x, n, ldx, z, acc, st);
        GMM_DP_CASES(CASE)
#undef CASE
    }
    return hipErrorInvalidValue;
}

hipError_t launch_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                        const double* lse, int acc, hipStream_t st, const int* skip) {
    switch (pl.dp) {
#define CASE(DPV)                                                                          \
    case DPV:                                                                              \
        return dtype == 0 ? launch_stats_t<DPV, float>(pl, x, n, ldx, lse, acc, st, skip) \
                          : launch_stats_t<DPV, uint16_t>(pl, x, n, ldx, lse, acc, st, skip);
        GMM_DP_CASES(CASE)
#undef CASE
    }
    return hipErrorInvalidValue;
}


int waves_per_stats_block(int dp) { return dp <= 64 ? StatsGeom<64>::WV : StatsGeom<128>::WV; }

hipError_t launch_prologue(const Plan& pl, const float* w, const float* mu, const float* var,
                           hipStream_t st) {
    hipLaunchKernelGGL(k_status_reset, dim3(1), dim3(64), 0, st, pl.status);
    const int64_t total = (int64_t)pl.k * pl.d;
    int vb = (int)((total + 255) / 256);
    if (vb > 1024) vb = 1024;
    hipLaunchKernelGGL(k_validate, dim3(vb), dim3(256), 0, st, w, mu, var, pl.k, pl.d, pl.status);
    hipLaunchKernelGGL(k_shift, dim3(pl.dp), dim3(256), 0, st, mu, pl.k, pl.d, pl.dp, pl.shift);
    hipLaunchKernelGGL(k_params, dim3(pl.kp), dim3(128), 0, st, w, mu, var, pl.k, pl.d, pl.dp,
                       pl.shift, pl.Pg, pl.cvec);
    return hipGetLastError();
}

hipError_t launch_finalize(const Plan& pl, int groups, int64_t n, float var_floor, float* w,
                           float* mu, float* var, hipStream_t st) {
    hipLaunchKernelGGL(k_finalize, dim3(pl.k), dim3(128), 0, st, pl.part, pl.npart, groups,
                       pl.kp, pl.dp, pl.d, pl.k, pl.shift, n, var_floor, w, mu, var, pl.status);
    return hipGetLastError();
}

hipError_t launch_ll_final(const Plan& pl, int nparts, double* out, hipStream_t st, double scale) {
    hipLaunchKernelGGL(k_ll_final, dim3(1), dim3(256), 0, st, pl.llpart, nparts, out, pl.status,
                       scale);
    return hipGetLastError();
}

hipError_t launch_kmfinal(const Plan& pl, float* c, hipStream_t st) {
    hipLaunchKernelGGL(k_kmfinal, dim3(pl.k), dim3(128), 0, st, pl.part, pl.npart, pl.ngroups,
                       pl.kp, pl.dp, pl.d, pl.k, pl.shift, c, pl.status);
    return hipGetLastError();
}

}  // namespace gmm
