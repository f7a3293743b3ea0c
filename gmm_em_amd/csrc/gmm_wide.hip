// gmm_wide.hip - kernels of the fused diagonal-GMM EM step for data wider than
// 128 dims (padded dimension 256..768), gfx950.
//
// Same method and arithmetic as the narrow kernels (fp64 MFMA contractions of
// the expanded Gaussian exponent, "Flash-GMM: A Memory-Efficient Kernel for
// Scalable Soft Clustering", section 3; the N x K responsibility matrix is
// never stored, section 1), with a decomposition that fits wide rows:
//
// * A block owns one 16-component K-tile. Its waves (8, or 4 in the
//   statistics pass from 512 padded dims on) split the padded dimension
//   into slices: wave w keeps the K-tile's coefficients of slice w in
//   registers and, in the statistics pass, the slice's first and second
//   moments in MFMA accumulators.
// * Rows are processed in 16-row tiles. The tile's shifted values a = x - s
//   are staged once in LDS in fp64, natural dim order (a^2 is formed by one
//   multiply where an operand needs it: 16 rows of both powers would not
//   fit in LDS).
// * Each wave contracts its slice; the partial log-densities are summed
//   through LDS in a fixed order, so every wave sees the same l.
// * Normaliser pass: per (row, K-tile) a (max, scaled sum) partial and the
//   tile's top-m candidates go to a chunk buffer; k_wmerge then merges the
//   K-tiles of each row in a fixed order into lse, log-likelihood partials
//   and the row's top-m components.
// * Statistics pass: responsibilities r = exp(l - lse) of the tile, then
//   each wave accumulates r^T [a, a^2] of its slice. Per-row-group partials
//   are reduced by the narrow path's k_finalize.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gmm_device.h"
#include "gmm_internal.h"

namespace gmm {

constexpr int WROWS = 16;       // rows per tile (one MFMA row block)

// NW waves per block; wave w owns dims [w*DS, (w+1)*DS) of the padded row.
template <int DP, int NW>
struct WideGeom {
    static_assert(DP % 128 == 0 && DP > 128 && DP <= WIDE_MAX_DP, "wide padded dimension");
    static constexpr int NT = NW * 64;
    static constexpr int DPH = DP / 2;
    static constexpr int DS = DP / NW;   // dims per wave slice
    static constexpr int T1 = DS / 4;    // E-step t-steps per power (4 dims per t-step)
    static constexpr int TS = 2 * T1;    // E-step t-steps per slice
    static constexpr int NJ = DS / 16;   // 16-dim column blocks per slice
    static constexpr int RS = DP + 4;    // LDS row stride in doubles
    static constexpr int TPR = NT / WROWS;  // staging threads per row
    static constexpr int PR = DP / TPR;     // values staged per thread
    // E-step t-steps per batch (a shorter ring where a wave holds 1/4 of the row)
    static constexpr int EB = (T1 % 8 == 0 && NW == 8) ? 8 : 4;
    static_assert(T1 % EB == 0, "each power's t-steps are whole E batches");
};

// Waves per block of each pass: the statistics pass keeps a slice's
// coefficients and moment accumulators in registers, which past 384 padded
// dims only fit one wave per SIMD (512 registers).
template <int DP, int MODE>
struct WideWaves {
    static constexpr int NW = (MODE == 1 && DP >= 512) ? 4 : 8;
};

// A value of the LDS copy of a tile, which holds the source type's bytes.
template <typename XT>
__device__ __forceinline__ float load_raw_value(const float* base, int i);
template <>
__device__ __forceinline__ float load_raw_value<float>(const float* base, int i) {
    return base[i];
}
template <>
__device__ __forceinline__ float load_raw_value<uint16_t>(const float* base, int i) {
    return __uint_as_float(((uint32_t)((const uint16_t*)base)[i]) << 16);
}

// Blocks of one row group take consecutive K-tiles and land on one XCD
// (workgroups are dispatched to the 8 XCDs round-robin by index).
__device__ __forceinline__ int wide_block_order() {
    const int nb = gridDim.x;
    return (nb % 8 == 0) ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
}

// MODE 0: normaliser partials (+ top TM candidates). MODE 1: statistics.
//
// E-step order of wave w: t-step j < T1 contracts dims w*DS + 4j + h (lane
// group h) at power 1, t-step T1 + j the same dims at power 2, so the A
// operand is a value of the natural-order tile (squared in the second half)
// and the B operand the matching coefficient w*b or -w/2.
template <int DP, typename XT, int MODE, int TM>
__global__ __launch_bounds__((WideGeom<DP, WideWaves<DP, MODE>::NW>::NT), 1)
void k_wide(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
            const double* __restrict__ Pg, const double* __restrict__ cvec,
            const double* __restrict__ shift, int ntiles, int64_t rows_per_group,
            const double* __restrict__ lse,          // MODE 1: chunk normalisers
            double2* __restrict__ lpart,             // MODE 0: [rows][ntiles] (max, sum)
            double* __restrict__ tval, int32_t* __restrict__ tidx,  // MODE 0, TM > 0
            double* __restrict__ part, double* __restrict__ npart, int accumulate) {
    constexpr int NW = WideWaves<DP, MODE>::NW;
    using G = WideGeom<DP, NW>;
    constexpr int NT = G::NT, DPH = G::DPH, DS = G::DS, T1 = G::T1, TS = G::TS, NJ = G::NJ,
                  RS = G::RS, TPR = G::TPR, PR = G::PR, EB = G::EB;
    constexpr int TMA = TM > 0 ? TM : 1;
    // With 4 waves a wave's registers are full: the next tile's raw values
    // are then copied by the buffer unit straight into LDS (no registers).
    // (fp32 data only: one dword per lane, so the LDS layout is the rows'
    // own layout; bf16 data keeps the register path)
    constexpr bool RAWLDS = NW == 4 && sizeof(XT) == 4;
    __shared__ __attribute__((aligned(16))) float xraw[RAWLDS ? WROWS * DP : 1];
    __shared__ __attribute__((aligned(16))) double fa[WROWS * RS];  // a of the tile
    __shared__ double shl[DP];                                     // shift, natural order
    __shared__ __attribute__((aligned(16))) f64x4 xb[NW][64];      // partial l per wave
    __shared__ double ls[WROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int ci = lane & 15, h = lane >> 4;
    const int o = wide_block_order();
    const int g = o / ntiles;
    const int kt = o % ntiles;
    const int slot = kt * 16 + ci;

    // Coefficients: pr[j] = coefficient of (dim, power) of t-step j, read
    // from the operand rows P[slot][2*(dim&1) + power-1][dim>>1].
    double pr[TS];
    {
        const double* src = Pg + (int64_t)slot * 2 * DP;
#pragma unroll
        for (int j = 0; j < TS; ++j) {
            const int dim = w * DS + 4 * (j % T1) + h;
            const int pw = j < T1 ? 0 : 1;
            pr[j] = src[((dim & 1) * 2 + pw) * DPH + (dim >> 1)];
        }
    }
    const double cc = cvec[slot];
    for (int i = tid; i < DP; i += NT) shl[i] = shift[(i & 1) * DPH + (i >> 1)];

    f64x4 acc[MODE == 1 ? 2 * NJ : 1];
#pragma unroll
    for (int j = 0; j < (MODE == 1 ? 2 * NJ : 1); ++j) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
    double n64 = 0.0;

    const int64_t gr0 = (int64_t)g * rows_per_group;
    int64_t gr1 = gr0 + rows_per_group;
    if (gr1 > n) gr1 = n;
    const int64_t ntr = gr1 > gr0 ? (gr1 - gr0 + WROWS - 1) / WROWS : 0;

    // Staging: thread (sr, sl) = (tid / TPR, tid % TPR) loads dims sl + TPR*u
    // of row sr of the tile through a per-tile buffer resource whose range
    // ends after the tile's last valid value (rows past the group read as 0;
    // padding dims are zeroed by a select on a loop-invariant count).
    const int sr = tid / TPR, sl = tid % TPR;
    const int nvalid = d > sl ? (d - sl + TPR - 1) / TPR : 0;  // u < nvalid: dim < d
    const uint32_t xoff = (uint32_t)(((int64_t)sr * ldx + sl) * (int64_t)sizeof(XT));
    float xv[RAWLDS ? 1 : PR];
    (void)xv;
    // buffer resource of tile `it`: range ends after its last valid value
    auto tile_rsrc = [&](int64_t it) {
        const int64_t rbase = gr0 + it * WROWS;
        int64_t nv = gr1 - rbase;
        nv = nv < 0 ? 0 : (nv > WROWS ? WROWS : nv);
        const int xbytes = nv > 0 ? (int)(((nv - 1) * ldx + d) * (int64_t)sizeof(XT)) : 0;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(x + rbase * ldx), (short)0, xbytes,
                                                 BUF_RSRC_WORD3);
    };
    // LDS copy of tile `it`: each instruction moves 64 consecutive values of
    // one row (lane i -> value col + i); rows are whole multiples of 64.
    auto load_raw = [&](int64_t it) {
        if constexpr (RAWLDS) {
            static_assert(DP % 64 == 0, "a row is whole 64-value segments");
            const __amdgpu_buffer_rsrc_t xr = tile_rsrc(it);
            constexpr int SEG = WROWS * DP / 64;  // segments per tile
            static_assert(SEG % NW == 0, "segments split evenly over the waves");
#pragma unroll
            for (int k = 0; k < SEG / NW; ++k) {
                const int sg = w * (SEG / NW) + k;
                const int row = sg / (DP / 64), col = (sg % (DP / 64)) * 64;
                const int soff = (int)(((int64_t)row * ldx + col) * (int64_t)sizeof(XT));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (__attribute__((address_space(3))) void*)(xraw + sg * 64), 4, lane * 4,
                    soff, 0, 0);
            }
        }
    };
    auto load = [&](int64_t it) {
        const int64_t rbase = gr0 + it * WROWS;
        int64_t nv = gr1 - rbase;
        nv = nv < 0 ? 0 : (nv > WROWS ? WROWS : nv);
        const int xbytes = nv > 0 ? (int)(((nv - 1) * ldx + d) * (int64_t)sizeof(XT)) : 0;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(x + rbase * ldx), (short)0, xbytes, BUF_RSRC_WORD3);
#pragma unroll
        for (int u = 0; u < PR; ++u) {
            const float v = buf_load_x<XT>(xr, xoff + (uint32_t)(TPR * u * (int)sizeof(XT)));
            xv[u] = u < nvalid ? v : 0.0f;
        }
    };
    auto store = [&]() {
        double* dst = fa + sr * RS + sl;
        if constexpr (RAWLDS) {
            const float* src = xraw + sr * DP + sl;
#pragma unroll
            for (int u = 0; u < PR; ++u) {
                const float v = u < nvalid ? load_raw_value<XT>(src, TPR * u) : 0.0f;
                dst[TPR * u] = (double)v - shl[sl + TPR * u];
                if (u % 8 == 7) __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < PR; ++u) dst[TPR * u] = (double)xv[u] - shl[sl + TPR * u];
        }
    };
    auto stage_ls = [&](int64_t it) {
        if constexpr (MODE == 1) {
            if (tid < WROWS) {
                const int64_t row = gr0 + it * WROWS + tid;
                ls[tid] = row < gr1 ? lse[row] : INFINITY;
            }
        }
    };

    // E-step operand: lane (h, i) reads a of row i, dim w*DS + 4j + h.
    const double* pa = fa + ci * RS + w * DS + h;

    if (ntr > 0) {
        if constexpr (RAWLDS) load_raw(0);
        else load(0);
    }
    for (int64_t it = 0; it < ntr; ++it) {
        if constexpr (RAWLDS) __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS copies landed
        __syncthreads();  // every wave is done with the previous tile's LDS
        store();
        stage_ls(it);
        __syncthreads();
        // the next tile's values are loaded during this tile's E-step (8 waves)
        // or, where a wave's registers are full (4 waves), during its M-step
        constexpr bool EARLY = NW == 8;
        if (EARLY && it + 1 < ntr) load(it + 1);
        if (RAWLDS && it + 1 < ntr) load_raw(it + 1);  // xraw was consumed before the barrier

        // partial l over slice w: one chain of TS MFMAs, operands streamed
        // from LDS through a two-batch register ring
        f64x4 e = {0.0, 0.0, 0.0, 0.0};
        double ra[2][EB];
#pragma unroll
        for (int u = 0; u < EB; ++u) ra[0][u] = pa[4 * u];
#pragma unroll
        for (int bt = 0; bt < TS / EB; ++bt) {
            const int cur = bt & 1;
            if (bt + 1 < TS / EB) {
#pragma unroll
                for (int u = 0; u < EB; ++u) ra[cur ^ 1][u] = pa[4 * (((bt + 1) * EB + u) % T1)];
            }
#pragma unroll
            for (int u = 0; u < EB; ++u) {
                const int j = bt * EB + u;
                const double v = ra[cur][u];
                e = mfma4d(j < T1 ? v : v * v, pr[j], e);
            }
        }
        xb[w][lane] = e;
        __syncthreads();
        if (!EARLY && !RAWLDS && it + 1 < ntr) load(it + 1);

        if constexpr (MODE == 0) {
            // wave q (< 4) finishes rows 4q + h: fixed-order sum over the
            // slices, then (max, sum) and top-m over the tile's 16 components
            if (w < 4) {
                const int q = w;
                double l = xb[0][lane][q];
#pragma unroll
                for (int v = 1; v < NW; ++v) l += xb[v][lane][q];
                l += cc;
                double m = l > -1.0e300 ? l : -1.0e300;
                double s = l > -1.0e300 ? 1.0 : 0.0;
                double tv[TMA];
                int ti[TMA];
#pragma unroll
                for (int j = 0; j < TMA; ++j) { tv[j] = -INFINITY; ti[j] = 0x7fffffff; }
                if constexpr (TM > 0) top_push<TM>(tv, ti, l, slot);
#pragma unroll 1
                for (int off = 1; off < 16; off <<= 1) {
                    const double m2 = shfl_xor_d(m, off);
                    const double s2 = shfl_xor_d(s, off);
                    const double mn = fmax(m, m2);
                    s = s * (double)__expf((float)(m - mn)) + s2 * (double)__expf((float)(m2 - mn));
                    m = mn;
                    if constexpr (TM > 0) top_merge<TM>(tv, ti, off);
                }
                const int64_t row = gr0 + it * WROWS + 4 * q + h;
                if (ci == 0 && row < gr1) {
                    lpart[row * ntiles + kt] = double2{m, s};
                    if constexpr (TM > 0) {
#pragma unroll
                        for (int j = 0; j < TM; ++j) {
                            tval[(row * ntiles + kt) * TM + j] = tv[j];
                            tidx[(row * ntiles + kt) * TM + j] = ti[j];
                        }
                    }
                }
            }
        } else {
            // every wave forms the same l and r for all 16 rows
            double r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                double l = xb[0][lane][q];
#pragma unroll
                for (int v = 1; v < NW; ++v) l += xb[v][lane][q];
                r[q] = (double)__expf((float)(l + cc - ls[4 * q + h]));
                n64 += r[q];
            }
            const bool nz[4] = {__builtin_amdgcn_ballot_w64(r[0] != 0.0) != 0,
                                __builtin_amdgcn_ballot_w64(r[1] != 0.0) != 0,
                                __builtin_amdgcn_ballot_w64(r[2] != 0.0) != 0,
                                __builtin_amdgcn_ballot_w64(r[3] != 0.0) != 0};
            // M-step over slice w: B = a (then a^2) of row 4q + h, dim
            // w*DS + 16J + ci; 4-row groups with all-zero r are skipped
            // (their MFMAs would add exact zeros)
            // (the reads of block J+1 are issued with block J's MFMAs; the
            // scheduling barrier keeps the compiler from hoisting more)
            const double* pm = fa + h * RS + w * DS + ci;
            double av[2][4];
#pragma unroll
            for (int q = 0; q < 4; ++q) av[0][q] = pm[4 * q * RS];
#pragma unroll
            for (int J = 0; J < NJ; ++J) {
                const int cur = J & 1;
                if (J + 1 < NJ) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) av[cur ^ 1][q] = pm[4 * q * RS + 16 * (J + 1)];
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (nz[q]) acc[J] = mfma4d(r[q], av[cur][q], acc[J]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (nz[q]) acc[NJ + J] = mfma4d(r[q], av[cur][q] * av[cur][q], acc[NJ + J]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    if constexpr (MODE == 1) {
        const int64_t gbase = (int64_t)g * ntiles * 16;
        if (w == 0) {
            n64 += shfl_xor_d(n64, 16);
            n64 += shfl_xor_d(n64, 32);
            if (h == 0) {
                double* np = npart + gbase + slot;
                *np = (accumulate ? *np : 0.0) + n64;
            }
        }
        // register q of lane (h, ci) of block J: component 4q + h, column
        // w*DS + 16J + ci (first moment) or DP + that (second moment)
#pragma unroll
        for (int J = 0; J < 2 * NJ; ++J)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int comp = kt * 16 + 4 * q + h;
                const int col = (J < NJ ? 0 : DP) + w * DS + 16 * (J % NJ) + ci;
                double* p = part + (gbase + comp) * (2 * DP) + col;
                *p = (accumulate ? *p : 0.0) + acc[J][q];
            }
    }
}

// Merge of the normaliser partials of each row over its K-tiles (fixed
// order: lane l takes tiles l, l+64, ..., then a butterfly over the wave),
// giving lse, the block's log-likelihood partial and the top-m components.
// Block: 4 waves x 32 rows each = 128 rows (one log-likelihood partial).
template <int TM>
__global__ __launch_bounds__(256)
void k_wmerge(const double2* __restrict__ lpart, const double* __restrict__ tval,
              const int32_t* __restrict__ tidx, int ntiles, int64_t n, int k,
              double* __restrict__ lse_out, double* __restrict__ llpart, int ll_accumulate,
              int m_out, int32_t* __restrict__ idx_out, float* __restrict__ resp_out) {
    constexpr int TMA = TM > 0 ? TM : 1;
    __shared__ double rowll[LL_ROWS];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int j = 0; j < LL_ROWS / 4; ++j) {
        const int lr = w * (LL_ROWS / 4) + j;
        const int64_t row = (int64_t)blockIdx.x * LL_ROWS + lr;
        double v = 0.0;
        if (row < n) {
            double m = -1.0e300, s = 0.0;
            double tv[TMA];
            int ti[TMA];
#pragma unroll
            for (int q = 0; q < TMA; ++q) { tv[q] = -INFINITY; ti[q] = 0x7fffffff; }
            for (int t = lane; t < ntiles; t += 64) {
                const double2 p = lpart[row * ntiles + t];
                const double mn = fmax(m, p.x);
                s = s * (double)__expf((float)(m - mn)) + p.y * (double)__expf((float)(p.x - mn));
                m = mn;
                if constexpr (TM > 0)
                    for (int q = 0; q < TM; ++q)
                        top_push<TM>(tv, ti, tval[(row * ntiles + t) * TM + q],
                                     tidx[(row * ntiles + t) * TM + q]);
            }
#pragma unroll 1
            for (int off = 1; off < 64; off <<= 1) {
                const double m2 = shfl_xor_d(m, off);
                const double s2 = shfl_xor_d(s, off);
                const double mn = fmax(m, m2);
                s = s * (double)__expf((float)(m - mn)) + s2 * (double)__expf((float)(m2 - mn));
                m = mn;
                if constexpr (TM > 0) top_merge<TM>(tv, ti, off);
            }
            v = m + log(s);
            if (lane == 0) {
                if (lse_out) lse_out[row] = v;
                if constexpr (TM > 0) {
                    for (int q = 0; q < m_out; ++q) {
                        const int sl = ti[q];
                        idx_out[row * m_out + q] = sl < k ? sl : -1;
                        resp_out[row * m_out + q] = __expf((float)(tv[q] - v));
                    }
                }
            }
        }
        if (lane == 0) rowll[lr] = v;
    }
    __syncthreads();
    if (w == 0) {
        double tot = rowll[lane] + rowll[lane + 64];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) tot += shfl_xor_d(tot, off);
        if (lane == 0) llpart[blockIdx.x] = (ll_accumulate ? llpart[blockIdx.x] : 0.0) + tot;
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
static int64_t wide_rows_per_group(const Plan& pl, int64_t n) {
    int64_t rpg = ((n + pl.ngroups - 1) / pl.ngroups + WROWS - 1) / WROWS * WROWS;
    return rpg < WROWS ? WROWS : rpg;
}

template <int DP, typename XT, int TM>
static hipError_t launch_wlse_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                hipStream_t st) {
    const int64_t rpg = wide_rows_per_group(pl, n);
    const int groups = (int)((n + rpg - 1) / rpg);
    constexpr int NT = WideGeom<DP, WideWaves<DP, 0>::NW>::NT;
    hipLaunchKernelGGL((k_wide<DP, XT, 0, TM>), dim3(groups * pl.ntiles), dim3(NT), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.Pg, pl.cvec, pl.shift, pl.ntiles, rpg,
                       (const double*)nullptr, pl.wlpart, pl.wtval, pl.wtidx, (double*)nullptr,
                       (double*)nullptr, 0);
    return hipGetLastError();
}

template <int TM>
static hipError_t launch_wmerge_t(const Plan& pl, int64_t n, double* lse_out, int ll_acc, int m,
                                  int32_t* idx, float* resp, hipStream_t st) {
    const int64_t blocks = (n + LL_ROWS - 1) / LL_ROWS;
    hipLaunchKernelGGL((k_wmerge<TM>), dim3((unsigned)blocks), dim3(256), 0, st, pl.wlpart,
                       pl.wtval, pl.wtidx, pl.ntiles, n, pl.k, lse_out, pl.llpart, ll_acc, m, idx,
                       resp);
    return hipGetLastError();
}

template <int DP, typename XT>
static hipError_t launch_wstats_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                  const double* lse, int acc, hipStream_t st) {
    const int64_t rpg = wide_rows_per_group(pl, n);
    // every row group gets a block per K-tile (empty groups write zeros)
    constexpr int NT = WideGeom<DP, WideWaves<DP, 1>::NW>::NT;
    hipLaunchKernelGGL((k_wide<DP, XT, 1, 0>), dim3(pl.ngroups * pl.ntiles), dim3(NT), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.Pg, pl.cvec, pl.shift, pl.ntiles, rpg, lse,
                       (double2*)nullptr, (double*)nullptr, (int32_t*)nullptr, pl.part, pl.npart,
                       acc);
    return hipGetLastError();
}

#define GMM_WIDE_CASES(M) M(256) M(384) M(512) M(640) M(768)

hipError_t launch_wide_lse(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                           double* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                           hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipError_t e = hipErrorInvalidValue;
    const int tm = m <= 0 ? 0 : (m <= 2 ? 2 : 4);
    switch (pl.dp) {
#define CASE(DPV)                                                                             \
    case DPV:                                                                                 \
        if (tm == 0)                                                                          \
            e = dtype == 0 ? launch_wlse_t<DPV, float, 0>(pl, x, n, ldx, st)                 \
                           : launch_wlse_t<DPV, uint16_t, 0>(pl, x, n, ldx, st);             \
        else if (tm == 2)                                                                     \
            e = dtype == 0 ? launch_wlse_t<DPV, float, 2>(pl, x, n, ldx, st)                 \
                           : launch_wlse_t<DPV, uint16_t, 2>(pl, x, n, ldx, st);             \
        else                                                                                  \
            e = dtype == 0 ? launch_wlse_t<DPV, float, 4>(pl, x, n, ldx, st)                 \
                           : launch_wlse_t<DPV, uint16_t, 4>(pl, x, n, ldx, st);             \
        break;
        GMM_WIDE_CASES(CASE)
#undef CASE
    }
    if (e != hipSuccess) return e;
    if (tm == 0) return launch_wmerge_t<0>(pl, n, lse_out, ll_acc, 0, nullptr, nullptr, st);
    if (tm == 2) return launch_wmerge_t<2>(pl, n, lse_out, ll_acc, m, idx, resp, st);
    return launch_wmerge_t<4>(pl, n, lse_out, ll_acc, m, idx, resp, st);
}

hipError_t launch_wide_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                             const double* lse, int acc, hipStream_t st) {
    switch (pl.dp) {
#define CASE(DPV)                                                                        \
    case DPV:                                                                            \
        return dtype == 0 ? launch_wstats_t<DPV, float>(pl, x, n, ldx, lse, acc, st)    \
                          : launch_wstats_t<DPV, uint16_t>(pl, x, n, ldx, lse, acc, st);
        GMM_WIDE_CASES(CASE)
#undef CASE
    }
    return hipErrorInvalidValue;
}

}  // namespace gmm
