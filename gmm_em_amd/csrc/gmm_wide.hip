// gmm_wide.hip - kernels of the fused diagonal-GMM EM step for data wider than
// 128 dims (padded dimension 256..768), gfx950.
//
// Same method and arithmetic as the narrow kernels (fp64 MFMA contractions of
// the expanded Gaussian exponent, "Flash-GMM: A Memory-Efficient Kernel for
// Scalable Soft Clustering", section 3; the N x K responsibility matrix is
// never stored, section 1), with a decomposition that fits wide rows:
//
// * A block owns one 16-component K-tile and has 8 waves that split the
//   padded dimension into slices. In the normaliser pass wave w keeps the
//   K-tile's coefficients of slice w (of 8) in registers; in the statistics
//   pass 4 waves keep the coefficients of 4 slices and the other 4 the
//   slices' first and second moment accumulators.
// * Rows are processed in 16-row tiles. The tile's shifted values a = x - s
//   are staged once in LDS in fp64, natural dim order (a^2 is formed by one
//   multiply where an operand needs it: 16 rows of both powers would not
//   fit in LDS). The statistics pass for fp32 rows (k_wstats_p) instead
//   keeps three fp32 tiles in LDS and forms a where it is read, so that its
//   two wave roles can work on consecutive tiles at once.
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

#include <type_traits>

#include "gmm_device.h"
#include "gmm_internal.h"

namespace gmm {

constexpr int WROWS = 16;       // rows per tile (one MFMA row block)

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

// Tile staging shared by both wide kernels (NT threads): thread (sr, sl) =
// (tid / TPR, tid % TPR) handles dims sl + TPR*u of row sr. Loads go through
// a per-tile buffer resource whose range ends after the tile's last valid
// value (rows past the group read as 0); padding dims are zeroed by a select
// on a loop-invariant count. The stored value is a = x - s in fp64.
template <int DP, int NT, typename XT>
struct WideStage {
    static constexpr int TPR = NT / WROWS;  // threads per row
    static constexpr int PR = DP / TPR;     // values per thread
    const XT* x;
    int64_t ldx, gr0, gr1;
    int d, sl, nvalid;
    uint32_t xoff;
    float xv[PR];

    __device__ WideStage(const XT* x_, int64_t ldx_, int d_, int64_t gr0_, int64_t gr1_, int tid)
        : x(x_), ldx(ldx_), gr0(gr0_), gr1(gr1_), d(d_) {
        const int sr = tid / TPR;
        sl = tid % TPR;
        nvalid = d > sl ? (d - sl + TPR - 1) / TPR : 0;  // u < nvalid: dim < d
        xoff = (uint32_t)(((int64_t)sr * ldx + sl) * (int64_t)sizeof(XT));
    }
    __device__ __forceinline__ void load(int64_t it) {
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
    }
    // load() without the padding select, for d == DP (every dim is data)
    __device__ __forceinline__ void load_full(int64_t it) {
        const int64_t rbase = gr0 + it * WROWS;
        int64_t nv = gr1 - rbase;
        nv = nv < 0 ? 0 : (nv > WROWS ? WROWS : nv);
        const int xbytes = nv > 0 ? (int)(((nv - 1) * ldx + d) * (int64_t)sizeof(XT)) : 0;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(x + rbase * ldx), (short)0, xbytes, BUF_RSRC_WORD3);
#pragma unroll
        for (int u = 0; u < PR; ++u)
            xv[u] = buf_load_x<XT>(xr, xoff + (uint32_t)(TPR * u * (int)sizeof(XT)));
    }
    // store() with this thread's shifts in registers (shr[u]: dim sl + TPR*u)
    template <int RS>
    __device__ __forceinline__ void store_r(double* fa, const double (&shr)[PR], int tid) const {
        double* dst = fa + (tid / TPR) * RS + sl;
#pragma unroll
        for (int u = 0; u < PR; ++u) {
            dst[TPR * u] = (double)xv[u] - shr[u];
            if (u % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }
    // fa: the tile in LDS (row stride RS, natural dim order); shl: shifts
    template <int RS>
    __device__ __forceinline__ void store(double* fa, const double* shl, int tid) const {
        double* dst = fa + (tid / TPR) * RS + sl;
#pragma unroll
        for (int u = 0; u < PR; ++u) {
            dst[TPR * u] = (double)xv[u] - shl[sl + TPR * u];
            if (u % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// Coefficients of slice `s` of K-tile row `slot`, in the E-step order below:
// pr[2j + p] = coefficient of (dim s*DS + 4j + h, power p+1), read from the
// operand rows P[slot][2*(dim&1) + p][dim>>1].
//
// E-step order of a slice of DS dims: dim group j (dims s*DS + 4j + h, lane
// group h) is contracted at power 1 and then at power 2, so each A value is
// read from the natural-order tile once and used as a, then a*a; the B
// operand is the matching coefficient w*b, then -w/2.
template <int DP, int DS>
__device__ __forceinline__ void wide_coefs(double (&pr)[DS / 2], const double* Pg, int slot,
                                           int s, int h) {
    constexpr int DPH = DP / 2;
    const double* src = Pg + (int64_t)slot * 2 * DP;
#pragma unroll
    for (int j = 0; j < DS / 4; ++j) {
        const int dim = s * DS + 4 * j + h;
#pragma unroll
        for (int p = 0; p < 2; ++p) pr[2 * j + p] = src[((dim & 1) * 2 + p) * DPH + (dim >> 1)];
    }
}

// Partial l of a slice for the 16 rows of the tile (register q of lane
// (h, ci) -> row 4q + h, component ci): one chain of DS/2 MFMAs; the A
// values stream from LDS through a two-batch register ring of EB dim groups
// (the scheduling barrier keeps the compiler from hoisting further reads).
// hook(bt) runs after batch bt's MFMAs are issued: independent work placed
// there overlaps the MFMA chain.
struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};
template <int DS, typename Hook = NoHook>
__device__ __forceinline__ f64x4 wide_estep(const double* pa, const double (&pr)[DS / 2],
                                            Hook&& hook = Hook()) {
    constexpr int T1 = DS / 4, EB = 4;
    static_assert(T1 % EB == 0, "whole E batches");
    f64x4 e = {0.0, 0.0, 0.0, 0.0};
    double ra[2][EB];
#pragma unroll
    for (int u = 0; u < EB; ++u) ra[0][u] = pa[4 * u];
#pragma unroll
    for (int bt = 0; bt < T1 / EB; ++bt) {
        const int cur = bt & 1;
        if (bt + 1 < T1 / EB) {
#pragma unroll
            for (int u = 0; u < EB; ++u) ra[cur ^ 1][u] = pa[4 * ((bt + 1) * EB + u)];
        }
#pragma unroll
        for (int u = 0; u < EB; ++u) {
            const int j = bt * EB + u;
            const double v = ra[cur][u];
            e = mfma4d(v, pr[2 * j], e);
            e = mfma4d(v * v, pr[2 * j + 1], e);
        }
        hook(bt);
        __builtin_amdgcn_sched_barrier(0);
    }
    return e;
}

// ---------------------------------------------------------------------------
// Normaliser pass (wide). 8 waves; wave w contracts slice w (DP/8 dims).
// Per 16-row tile: stage, partial l per wave, fixed-order sum over the waves
// (waves 0-3 finish rows 4q + h, q = wave), then per (row, K-tile) the
// (max, scaled sum) over the tile's 16 components and its top TM candidates.
// ---------------------------------------------------------------------------
template <int DP, typename XT, int TM>
__global__ __launch_bounds__(512, 1)
void k_wlse(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
            const double* __restrict__ Pg, const double* __restrict__ cvec,
            const double* __restrict__ shift, int ntiles, int64_t rows_per_group,
            double2* __restrict__ lpart, double* __restrict__ tval, int32_t* __restrict__ tidx) {
    // RS (tile row stride, doubles) is odd: the 16 lanes of an E-step read
    // (16 rows, one dim) then hit 16 distinct pairs of the 32 LDS banks
    constexpr int NW = 8, NT = 512, DS = DP / NW, RS = DP + 1;
    constexpr int TMA = TM > 0 ? TM : 1;
    __shared__ __attribute__((aligned(16))) double fa[WROWS * RS];
    __shared__ __attribute__((aligned(16))) f64x4 xb[2][NW][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int ci = lane & 15, h = lane >> 4;
    const int o = wide_block_order();
    const int g = o / ntiles;
    const int kt = o % ntiles;
    const int slot = kt * 16 + ci;

    double pr[DS / 2];
    wide_coefs<DP, DS>(pr, Pg, slot, w, h);
    const double cc = cvec[slot];

    const int64_t gr0 = (int64_t)g * rows_per_group;
    int64_t gr1 = gr0 + rows_per_group;
    if (gr1 > n) gr1 = n;
    const int64_t ntr = gr1 > gr0 ? (gr1 - gr0 + WROWS - 1) / WROWS : 0;
    WideStage<DP, NT, XT> stg(x, ldx, d, gr0, gr1, tid);
    const double* pa = fa + ci * RS + w * DS + h;

    // Waves 0-3 fold tile it's partials (row 4q + h, q = wave) into per
    // (row, K-tile) results while tile it+1's E-step runs: the reduction is
    // split into steps placed after the E-step's MFMA batches. The partials
    // alternate between two buffers, so a tile's are read one iteration
    // after they were written, with the tile's barriers in between.
    const int wq = __builtin_amdgcn_readfirstlane(w);
    double rl = 0.0, rm = -1.0e300, rs = 0.0;
    double tv[TMA];
    int ti[TMA];
    auto red_start = [&](int buf) {
        const int q = wq;
        double l = xb[buf][0][lane][q];
#pragma unroll
        for (int v = 1; v < NW; ++v) l += xb[buf][v][lane][q];
        rl = l + cc;
        rm = rl > -1.0e300 ? rl : -1.0e300;
#pragma unroll
        for (int j = 0; j < TMA; ++j) { tv[j] = -INFINITY; ti[j] = 0x7fffffff; }
        if constexpr (TM > 0) top_push<TM>(tv, ti, rl, slot);
    };
    // the tile's 16 components: max over the 16 lanes, then one exponential
    // per lane and a sum over the 16 lanes (fixed butterfly orders)
    auto red_max = [&](int off) {
        rm = fmax(rm, shfl_xor_d(rm, off));
        if constexpr (TM > 0) top_merge<TM>(tv, ti, off);
    };
    auto red_exp = [&]() { rs = (double)__expf((float)(rl - rm)); };
    auto red_sum = [&](int off) { rs += shfl_xor_d(rs, off); };
    auto red_store = [&](int64_t rt) {
        const int64_t row = gr0 + rt * WROWS + 4 * wq + h;
        if (ci == 0 && row < gr1) {
            lpart[row * ntiles + kt] = double2{rm, rs};
            if constexpr (TM > 0) {
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    tval[(row * ntiles + kt) * TM + j] = tv[j];
                    tidx[(row * ntiles + kt) * TM + j] = ti[j];
                }
            }
        }
    };
    // the reduction's eleven steps (start, four max rounds, exponential, four
    // sum rounds, store) spread evenly over the E-step's NB batches
    constexpr int NB = DS / 16;
    constexpr int NSTEP = 11;
    auto red_step = [&](int k, int buf, int64_t rt) {
        if (k == 0) red_start(buf);
        else if (k <= 4) red_max(1 << (k - 1));
        else if (k == 5) red_exp();
        else if (k <= 9) red_sum(1 << (k - 6));
        else red_store(rt);
    };

    // the shifts of the dims this thread stages, in registers; rows without
    // padding dims skip the padding select
    using Stage = WideStage<DP, NT, XT>;
    double shr[Stage::PR];
#pragma unroll
    for (int u = 0; u < Stage::PR; ++u) {
        const int dim = stg.sl + Stage::TPR * u;
        shr[u] = shift[(dim & 1) * (DP / 2) + (dim >> 1)];
    }
    const bool full = d == DP;
    auto load = [&](int64_t it) {
        if (full) stg.load_full(it);
        else stg.load(it);
    };
    if (ntr > 0) load(0);
    for (int64_t it = 0; it < ntr; ++it) {
        __syncthreads();  // every wave is done with the previous tile's LDS
        stg.template store_r<RS>(fa, shr, tid);
        __syncthreads();
        if (it + 1 < ntr) load(it + 1);
        const int cur = (int)(it & 1);
        const bool red = wq < 4 && it > 0;  // wave-uniform
        auto hook = [&](int bt) {
            if (!red) return;
#pragma unroll
            for (int k = 0; k < NSTEP; ++k)
                if (k * NB / NSTEP == bt) red_step(k, cur ^ 1, it - 1);
        };
        xb[cur][w][lane] = wide_estep<DS>(pa, pr, hook);
    }
    if (ntr > 0) {
        __syncthreads();
        if (wq < 4) {
#pragma unroll
            for (int k = 0; k < NSTEP; ++k) red_step(k, (int)((ntr - 1) & 1), ntr - 1);
        }
    }
}

// ---------------------------------------------------------------------------
// Statistics pass (wide). 8 waves in two roles over 4 slices of DP/4 dims:
// waves 0-3 ("E") hold slice w's coefficients and contract it; waves 4-7
// ("M") hold slice w-4's first and second moment accumulators. One wave of
// each role per SIMD, so each keeps at most 256 registers; a role's loop
// runs the same barriers as the other's. Per 16-row tile:
//   stage (all) | E: partial l -> LDS; M: load the next tile | M: fixed-order
//   sum of the 4 partials, r = exp(l - lse), M-step over its slice
// Tiles whose responsibilities are all exactly zero are skipped (their
// MFMAs would add exact zeros).
// ---------------------------------------------------------------------------
template <int DP, typename XT>
__global__ __launch_bounds__(512, 1)
void k_wstats(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
              const double* __restrict__ Pg, const double* __restrict__ cvec,
              const double* __restrict__ shift, int ntiles, int64_t rows_per_group,
              const double* __restrict__ lse, double* __restrict__ part,
              double* __restrict__ npart, int accumulate) {
    // odd tile row stride: conflict-free E-step reads (see k_wlse)
    constexpr int NT = 512, NS = 4, DS = DP / NS, RS = DP + 1, NJ = DS / 16;
    // fp32 rows: the M waves copy the next tile's raw values into LDS with
    // buffer-to-LDS loads during the E phase, so no thread holds them in
    // registers (one dword per lane: the LDS copy has the rows' own layout).
    // bf16 rows are loaded into registers.
    constexpr bool RAWLDS = sizeof(XT) == 4;
    __shared__ __attribute__((aligned(16))) float xraw[RAWLDS ? WROWS * DP : 1];
    __shared__ __attribute__((aligned(16))) double fa[WROWS * RS];
    __shared__ double shl[DP];
    __shared__ __attribute__((aligned(16))) f64x4 xb[NS][64];
    __shared__ double ls[WROWS];

    const int tid = threadIdx.x;
    // the wave index as a scalar: the role branch below is then uniform and
    // each role's registers are allocated on their own
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = lane & 15, h = lane >> 4;
    const int s = w & 3;  // slice
    const int o = wide_block_order();
    const int g = o / ntiles;
    const int kt = o % ntiles;
    const int slot = kt * 16 + ci;
    for (int i = tid; i < DP; i += NT) shl[i] = shift[(i & 1) * (DP / 2) + (i >> 1)];

    const int64_t gr0 = (int64_t)g * rows_per_group;
    int64_t gr1 = gr0 + rows_per_group;
    if (gr1 > n) gr1 = n;
    const int64_t ntr = gr1 > gr0 ? (gr1 - gr0 + WROWS - 1) / WROWS : 0;
    WideStage<DP, NT, XT> stg(x, ldx, d, gr0, gr1, tid);
    // buffer-to-LDS copy of tile `it` by the 4 M waves (wave index mw): each
    // instruction moves 64 consecutive values of one row (lane i -> value
    // col + i; rows are whole 64-value segments); past the tile's last
    // valid value the buffer unit returns 0
    auto load_raw = [&](int64_t it, int mw) {
        if constexpr (RAWLDS) {
            constexpr int SEG = WROWS * DP / 64;
            static_assert(DP % 64 == 0 && SEG % NS == 0, "whole segments per wave");
            const int64_t rbase = gr0 + it * WROWS;
            int64_t nv = gr1 - rbase;
            nv = nv < 0 ? 0 : (nv > WROWS ? WROWS : nv);
            const int xbytes = nv > 0 ? (int)(((nv - 1) * ldx + d) * (int64_t)sizeof(XT)) : 0;
            const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(x + rbase * ldx), (short)0, xbytes, BUF_RSRC_WORD3);
#pragma unroll
            for (int k = 0; k < SEG / NS; ++k) {
                const int sg = mw * (SEG / NS) + k;
                const int row = sg / (DP / 64), col = (sg % (DP / 64)) * 64;
                const int soff = (int)(((int64_t)row * ldx + col) * (int64_t)sizeof(XT));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (__attribute__((address_space(3))) void*)(xraw + sg * 64), 4, lane * 4,
                    soff, 0, 0);
            }
        }
    };
    // LDS copy -> a = x - s; dims past d are zeroed
    auto store_raw = [&]() {
        constexpr int TPR = NT / WROWS, PR = DP / TPR;
        const int sr = tid / TPR, sl = tid % TPR;
        const int nvalid = d > sl ? (d - sl + TPR - 1) / TPR : 0;
        double* dst = fa + sr * RS + sl;
        const float* src = xraw + sr * DP + sl;
        // (a few values at a time: the M waves hold their accumulators here)
        if (d == DP) {  // (uniform) no padding dims: no select
#pragma unroll
            for (int u = 0; u < PR; ++u) {
                dst[TPR * u] = (double)src[TPR * u] - shl[sl + TPR * u];
                if (u % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < PR; ++u) {
                const float v = u < nvalid ? src[TPR * u] : 0.0f;
                dst[TPR * u] = (double)v - shl[sl + TPR * u];
                if (u % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    auto stage = [&](int64_t it) {
        if constexpr (RAWLDS) __builtin_amdgcn_s_waitcnt(0);  // own LDS copies landed
        __syncthreads();  // every wave is done with the previous tile's LDS
        if constexpr (RAWLDS) store_raw();
        else stg.template store<RS>(fa, shl, tid);
        if (tid < WROWS) {
            const int64_t row = gr0 + it * WROWS + tid;
            ls[tid] = row < gr1 ? lse[row] : INFINITY;
        }
        __syncthreads();
    };

    if (ntr > 0) {
        if constexpr (RAWLDS) {
            if (w >= NS) load_raw(0, w - NS);
        } else {
            stg.load(0);
        }
    }
    if (w < NS) {
        // E role
        double pr[DS / 2];
        wide_coefs<DP, DS>(pr, Pg, slot, s, h);
        const double* pa = fa + ci * RS + s * DS + h;
        for (int64_t it = 0; it < ntr; ++it) {
            stage(it);
            if constexpr (!RAWLDS) {
                if (it + 1 < ntr) stg.load(it + 1);
            }
            xb[s][lane] = wide_estep<DS>(pa, pr);
            __syncthreads();
        }
    } else {
        // M role
        const double cc = cvec[slot];
        f64x4 acc[2 * NJ];
#pragma unroll
        for (int j = 0; j < 2 * NJ; ++j) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
        double n64 = 0.0;
        const double* pm = fa + h * RS + s * DS + ci;
        for (int64_t it = 0; it < ntr; ++it) {
            stage(it);
            // the next tile is in flight during this one (the LDS copy area
            // was consumed before the barrier)
            if (it + 1 < ntr) {
                if constexpr (RAWLDS) load_raw(it + 1, s);
                else stg.load(it + 1);
            }
            __syncthreads();
            // fixed-order sum of the slices' partial l, one slice at a time
            f64x4 l = xb[0][lane];
#pragma unroll
            for (int v = 1; v < NS; ++v) {
                __builtin_amdgcn_sched_barrier(0);
                l += xb[v][lane];
            }
            double r[4];
            bool any = false;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                r[q] = exp_f64range(l[q] + cc - ls[4 * q + h]);
                n64 += r[q];
                any = any || r[q] != 0.0;
            }
            // a tile whose 256 responsibilities are all exactly zero adds
            // nothing. B = a (then a^2) of row 4q + h, dim s*DS + 16J + ci;
            // the reads of block J+1 are issued with block J's MFMAs.
            if (__builtin_amdgcn_ballot_w64(any) != 0) {
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
                    for (int q = 0; q < 4; ++q) acc[J] = mfma4d(r[q], av[cur][q], acc[J]);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[NJ + J] = mfma4d(r[q], av[cur][q] * av[cur][q], acc[NJ + J]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        const int64_t gbase = (int64_t)g * ntiles * 16;
        if (s == 0) {
            n64 += shfl_xor_d(n64, 16);
            n64 += shfl_xor_d(n64, 32);
            if (h == 0) {
                double* np = npart + gbase + slot;
                *np = (accumulate ? *np : 0.0) + n64;
            }
        }
        // register q of lane (h, ci) of block J: component 4q + h, column
        // s*DS + 16J + ci (first moment) or DP + that (second moment)
#pragma unroll
        for (int J = 0; J < 2 * NJ; ++J)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int comp = kt * 16 + 4 * q + h;
                const int col = (J < NJ ? 0 : DP) + s * DS + 16 * (J % NJ) + ci;
                double* p = part + (gbase + comp) * (2 * DP) + col;
                *p = (accumulate ? *p : 0.0) + acc[J][q];
            }
    }
}

// Statistics pass for fp32 rows: the same roles, arithmetic and order as
// k_wstats, run as a two-stage pipeline so that the roles overlap. In phase p
// the E waves contract tile p while the M waves run the M-step of tile p - 1
// on the same SIMDs, so the matrix units see both roles' MFMAs back to back.
// Rows stay fp32 in LDS, in three tile buffers (tile t in buffer t % 3): the
// copies of tile p + 1 are issued at the start of phase p by all 8 waves
// (buffer-to-LDS, two rows per wave, each row through its own buffer range:
// rows past the group and dims past d read as 0) and have landed by the end
// of phase p. Each wave forms a = x - s in fp64 for the values it reads (the
// expression the staged kernels store), so the results equal k_wstats's bit
// for bit. Per phase two barriers: after A the E waves publish their partial
// l of tile p; after B the M waves read them at the start of phase p + 1.
// Every wave runs the same ntr + 1 phases.
// ---------------------------------------------------------------------------
// ZS: every shift is 0, so a = x (x - 0.0 is x exactly, -0 included) and
// neither the shifts nor the subtraction are needed.
template <int DS, bool ZS = false>
__device__ __forceinline__ f64x4 wide_estep_raw(const float* px, const double* psh,
                                                const double (&pr)[DS / 2]) {
    constexpr int T1 = DS / 4, EB = 4;
    static_assert(T1 % EB == 0, "whole E batches");
    f64x4 e = {0.0, 0.0, 0.0, 0.0};
    float rx[2][EB];
    double rs[2][EB];
#pragma unroll
    for (int u = 0; u < EB; ++u) {
        rx[0][u] = px[4 * u];
        rs[0][u] = ZS ? 0.0 : psh[4 * u];
    }
#pragma unroll
    for (int bt = 0; bt < T1 / EB; ++bt) {
        const int cur = bt & 1;
        if (bt + 1 < T1 / EB) {
#pragma unroll
            for (int u = 0; u < EB; ++u) {
                rx[cur ^ 1][u] = px[4 * ((bt + 1) * EB + u)];
                rs[cur ^ 1][u] = ZS ? 0.0 : psh[4 * ((bt + 1) * EB + u)];
            }
        }
#pragma unroll
        for (int u = 0; u < EB; ++u) {
            const int j = bt * EB + u;
            const double v = ZS ? (double)rx[cur][u] : (double)rx[cur][u] - rs[cur][u];
            e = mfma4d(v, pr[2 * j], e);
            e = mfma4d(v * v, pr[2 * j + 1], e);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return e;
}

template <int DP>
__global__ __launch_bounds__(512, 1)
void k_wstats_p(const float* __restrict__ x, int64_t n, int d, int64_t ldx,
                const double* __restrict__ Pg, const double* __restrict__ cvec,
                const double* __restrict__ shift, int ntiles, int64_t rows_per_group,
                const double* __restrict__ lse, double* __restrict__ part,
                double* __restrict__ npart, int accumulate) {
    // RSF = DP + 2 floats: the E-step's reads (16 rows at one dim, 4 dims)
    // hit distinct banks within each half-wave
    constexpr int NT = 512, NS = 4, DS = DP / NS, NJ = DS / 16, NB = 3;
    constexpr int RSF = DP + 2, SEGR = DP / 64;
    static_assert(DP % 64 == 0, "whole 64-value segments per row");
    __shared__ __attribute__((aligned(16))) float xr[NB][WROWS * RSF];
    __shared__ double shl[DP];
    __shared__ __attribute__((aligned(16))) f64x4 xb[NS][64];
    __shared__ double ls[NB][WROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = lane & 15, h = lane >> 4;
    const int s = w & 3;  // slice
    const int o = wide_block_order();
    const int g = o / ntiles;
    const int kt = o % ntiles;
    const int slot = kt * 16 + ci;
    for (int i = tid; i < DP; i += NT) shl[i] = shift[(i & 1) * (DP / 2) + (i >> 1)];

    const int64_t gr0 = (int64_t)g * rows_per_group;
    int64_t gr1 = gr0 + rows_per_group;
    if (gr1 > n) gr1 = n;
    const int64_t ntr = gr1 > gr0 ? (gr1 - gr0 + WROWS - 1) / WROWS : 0;

    // copies of tile `it` into its buffer: wave w moves rows 2w and 2w + 1
    auto issue = [&](int64_t it) {
        float* dst = xr[(int)(it % NB)];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int row = 2 * w + rr;
            const int64_t grow = gr0 + it * WROWS + row;
            const int nbytes = grow < gr1 ? d * (int)sizeof(float) : 0;
            const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(x + (grow < gr1 ? grow : gr0) * ldx), (short)0, nbytes, BUF_RSRC_WORD3);
#pragma unroll
            for (int c = 0; c < SEGR; ++c)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xrs, (__attribute__((address_space(3))) void*)(dst + row * RSF + 64 * c), 4,
                    lane * 4, c * 64 * (int)sizeof(float), 0, 0);
        }
    };
    // normaliser of row tid of tile it (+inf past the group: r = 0)
    auto load_ls = [&](int64_t it) -> double {
        const int64_t row = gr0 + it * WROWS + tid;
        return row < gr1 ? lse[row] : INFINITY;
    };

    if (ntr > 0) {
        issue(0);
        if (tid < WROWS) ls[0][tid] = load_ls(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    // every shift 0 (uniform over the block): the roles skip the subtraction;
    // the vote is also the barrier after the first copies
    bool zl = true;
    for (int i = tid; i < DP; i += NT) zl = zl && shl[i] == 0.0;
    const bool zs = __syncthreads_and(zl) != 0;
    auto roles = [&](auto zsc) {
    constexpr bool ZS = decltype(zsc)::value;
    if (w < NS) {
        // E role
        double pr[DS / 2];
        wide_coefs<DP, DS>(pr, Pg, slot, s, h);
        const double* psh = shl + s * DS + h;
        for (int64_t p = 0; p <= ntr; ++p) {
            double lsn = INFINITY;
            if (p + 1 < ntr) {
                issue(p + 1);
                if (tid < WROWS) lsn = load_ls(p + 1);
            }
            f64x4 e = {0.0, 0.0, 0.0, 0.0};
            if (p < ntr) e = wide_estep_raw<DS, ZS>(xr[(int)(p % NB)] + ci * RSF + s * DS + h, psh, pr);
            if (p + 1 < ntr && tid < WROWS) ls[(int)((p + 1) % NB)][tid] = lsn;
            __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile p + 1 have landed
            __syncthreads();                // A
            if (p < ntr) xb[s][lane] = e;
            __syncthreads();                // B
        }
    } else {
        // M role
        const double cc = cvec[slot];
        f64x4 acc[2 * NJ];
#pragma unroll
        for (int j = 0; j < 2 * NJ; ++j) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
        double n64 = 0.0;
        const double* psm = shl + s * DS + ci;
        for (int64_t p = 0; p <= ntr; ++p) {
            if (p + 1 < ntr) issue(p + 1);
            if (p >= 1) {
                const int bm = (int)((p - 1) % NB);
                // fixed-order sum of the slices' partial l, one slice at a time
                f64x4 l = xb[0][lane];
#pragma unroll
                for (int v = 1; v < NS; ++v) {
                    __builtin_amdgcn_sched_barrier(0);
                    l += xb[v][lane];
                }
                double r[4];
                bool any = false;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    r[q] = exp_f64range(l[q] + cc - ls[bm][4 * q + h]);
                    n64 += r[q];
                    any = any || r[q] != 0.0;
                }
                // a tile whose 256 responsibilities are all exactly zero adds
                // nothing. B = a (then a^2) of row 4q + h, dim s*DS + 16J + ci;
                // the reads of block J+1 are issued with block J's MFMAs.
                if (__builtin_amdgcn_ballot_w64(any) != 0) {
                    const float* pm = xr[bm] + h * RSF + s * DS + ci;
                    float xv[2][4];
                    double sv[2];
#pragma unroll
                    for (int q = 0; q < 4; ++q) xv[0][q] = pm[4 * q * RSF];
                    sv[0] = ZS ? 0.0 : psm[0];
#pragma unroll
                    for (int J = 0; J < NJ; ++J) {
                        const int cur = J & 1;
                        if (J + 1 < NJ) {
#pragma unroll
                            for (int q = 0; q < 4; ++q) xv[cur ^ 1][q] = pm[4 * q * RSF + 16 * (J + 1)];
                            sv[cur ^ 1] = ZS ? 0.0 : psm[16 * (J + 1)];
                        }
                        double av[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            av[q] = ZS ? (double)xv[cur][q] : (double)xv[cur][q] - sv[cur];
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[J] = mfma4d(r[q], av[q], acc[J]);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[NJ + J] = mfma4d(r[q], av[q] * av[q], acc[NJ + J]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile p + 1 have landed
            __syncthreads();                // A
            __syncthreads();                // B
        }
        const int64_t gbase = (int64_t)g * ntiles * 16;
        if (s == 0) {
            n64 += shfl_xor_d(n64, 16);
            n64 += shfl_xor_d(n64, 32);
            if (h == 0) {
                double* np = npart + gbase + slot;
                *np = (accumulate ? *np : 0.0) + n64;
            }
        }
        // register q of lane (h, ci) of block J: component 4q + h, column
        // s*DS + 16J + ci (first moment) or DP + that (second moment)
#pragma unroll
        for (int J = 0; J < 2 * NJ; ++J)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int comp = kt * 16 + 4 * q + h;
                const int col = (J < NJ ? 0 : DP) + s * DS + 16 * (J % NJ) + ci;
                double* pp = part + (gbase + comp) * (2 * DP) + col;
                *pp = (accumulate ? *pp : 0.0) + acc[J][q];
            }
    }
    };
    if (zs) roles(std::true_type{});
    else roles(std::false_type{});
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
              int m_out, int32_t* __restrict__ idx_out, float* __restrict__ resp_out, int km) {
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
            // k-means mode: the row's value is its best log-density,
            // -|x - c_z|^2 (the row's contribution to -inertia)
            v = m + log(s);
            if constexpr (TM > 0) v = km ? tv[0] : v;
            if (lane == 0) {
                if (lse_out) lse_out[row] = v;
                if constexpr (TM > 0) {
                    for (int q = 0; q < m_out; ++q) {
                        const int sl = ti[q];
                        idx_out[row * m_out + q] = sl < k ? sl : -1;
                        if (resp_out) resp_out[row * m_out + q] = __expf((float)(tv[q] - v));
                    }
                }
            }
        }
        if (lane == 0) rowll[lr] = v;
    }
    __syncthreads();
    if (w == 0) {
        double tot = 0.0;
#pragma unroll
        for (int r = 0; r < LL_ROWS; r += 64) tot += rowll[r + lane];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) tot += shfl_xor_d(tot, off);
        if (lane == 0) llpart[blockIdx.x] = (ll_accumulate ? llpart[blockIdx.x] : 0.0) + tot;
    }
}

// ---------------------------------------------------------------------------
// k-means statistics (wide): the one-hot counterpart of the statistics pass.
// A block owns (row group, 16-centroid K-tile); wave w owns dim slice w (of
// 8, DP/8 dims) and walks all the group's rows in order: it selects the rows
// assigned to the tile with a ballot, loads the slice of up to KMW_BATCH of
// them at once (per-row buffer resources: dims past d or past the slice read
// 0) and adds them, in row order, into its LDS accumulator (a lane owns one
// or two dims). Each (centroid, dim) has one owner, so no cross-wave sum.
// ---------------------------------------------------------------------------
constexpr int KMW_BATCH = 16;
constexpr int KMW_ZB = 8;

template <int DP, typename XT>
__global__ __launch_bounds__(512)
void k_km_wstats(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
                 const double* __restrict__ shift, const int32_t* __restrict__ z, int ntiles,
                 int64_t rows_per_group, double* __restrict__ part, double* __restrict__ npart,
                 int accumulate) {
    constexpr int NW = 8, DPW = DP / NW, KS = 128;
    static_assert(DPW <= 128, "two dims per lane");
    __shared__ double kacc[NW][16 * KS];
    __shared__ int kcnt[16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x / ntiles, tile = blockIdx.x - g * ntiles;
    const int kp = ntiles * 16, c0 = tile * 16;
    double* my = kacc[w];
    for (int i = lane; i < 16 * KS; i += 64) my[i] = 0.0;
    if (tid < 16) kcnt[tid] = 0;
    const int d0 = w * DPW;  // first dim of the slice
    const int dA = lane, dB = lane + 64;  // slice-relative dims of this lane
    const double sA = (dA < DPW && d0 + dA < d) ? shift[((d0 + dA) & 1) * (DP / 2) + ((d0 + dA) >> 1)] : 0.0;
    const double sB = (dB < DPW && d0 + dB < d) ? shift[((d0 + dB) & 1) * (DP / 2) + ((d0 + dB) >> 1)] : 0.0;
    int sbytes = d - d0;
    sbytes = sbytes < 0 ? 0 : (sbytes > DPW ? DPW : sbytes);
    sbytes *= (int)sizeof(XT);
    const uint32_t oA = (uint32_t)(dA * sizeof(XT)), oB = (uint32_t)(dB * sizeof(XT));
    const int64_t r0 = (int64_t)g * rows_per_group;
    const int64_t r1 = r0 + rows_per_group < n ? r0 + rows_per_group : n;
    __syncthreads();
    for (int64_t rz = r0; rz < r1; rz += 64 * KMW_ZB) {
        int zc[KMW_ZB];
#pragma unroll
        for (int u = 0; u < KMW_ZB; ++u) {
            const int64_t r = rz + 64 * u + lane;
            zc[u] = (r < r1 ? z[r] : -1) - c0;
        }
#pragma unroll
        for (int u = 0; u < KMW_ZB; ++u) {
            const int64_t rb = rz + 64 * u;
            uint64_t mask = __builtin_amdgcn_ballot_w64((unsigned)zc[u] < 16u);
            while (mask) {
                int cb[KMW_BATCH];
                float xa[KMW_BATCH], xb[KMW_BATCH];
                int nb = 0;
#pragma unroll
                for (int i = 0; i < KMW_BATCH; ++i) {
                    const bool v = mask != 0;  // uniform
                    const int b = v ? __builtin_ctzll(mask) : 0;
                    mask = v ? mask & (mask - 1) : mask;
                    nb += v ? 1 : 0;
                    cb[i] = __builtin_amdgcn_readlane(zc[u], b);
                    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                        (void*)(x + (rb + b) * ldx + d0), (short)0, sbytes, BUF_RSRC_WORD3);
                    xa[i] = buf_load_x<XT>(xr, oA);
                    xb[i] = buf_load_x<XT>(xr, oB);
                }
#pragma unroll
                for (int i = 0; i < KMW_BATCH; ++i) {
                    if (i < nb) {
                        double* ar = my + cb[i] * KS;
                        ar[dA] += (double)xa[i] - sA;
                        ar[dB] += (double)xb[i] - sB;
                        if (w == 0 && lane == 0) kcnt[cb[i]] += 1;
                    }
                }
            }
        }
    }
    __syncthreads();
    for (int i = lane; i < 16 * DPW; i += 64) {
        const int cc = i / DPW, j = i - cc * DPW;
        if (d0 + j < d) {
            double* p = part + ((int64_t)g * kp + c0 + cc) * 2 * DP + d0 + j;
            *p = (accumulate ? *p : 0.0) + my[cc * KS + j];
        }
    }
    if (tid < 16) {
        double* np = npart + (int64_t)g * kp + c0 + tid;
        *np = (accumulate ? *np : 0.0) + (double)kcnt[tid];
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
    hipLaunchKernelGGL((k_wlse<DP, XT, TM>), dim3(groups * pl.ntiles), dim3(512), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.Pg, pl.cvec, pl.shift, pl.ntiles, rpg,
                       pl.wlpart, pl.wtval, pl.wtidx);
    return hipGetLastError();
}

template <int TM>
static hipError_t launch_wmerge_t(const Plan& pl, int64_t n, double* lse_out, int ll_acc, int m,
                                  int32_t* idx, float* resp, int km, hipStream_t st) {
    const int64_t blocks = (n + LL_ROWS - 1) / LL_ROWS;
    hipLaunchKernelGGL((k_wmerge<TM>), dim3((unsigned)blocks), dim3(256), 0, st, pl.wlpart,
                       pl.wtval, pl.wtidx, pl.ntiles, n, pl.k, lse_out, pl.llpart, ll_acc, m, idx,
                       resp, km);
    return hipGetLastError();
}

template <int DP, typename XT>
static hipError_t launch_wstats_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                  const double* lse, int acc, hipStream_t st) {
    const int64_t rpg = wide_rows_per_group(pl, n);
    // every row group gets a block per K-tile (empty groups write zeros)
    if constexpr (sizeof(XT) == 4)
        hipLaunchKernelGGL((k_wstats_p<DP>), dim3(pl.ngroups * pl.ntiles), dim3(512), 0, st,
                           (const float*)x, n, pl.d, ldx, pl.Pg, pl.cvec, pl.shift, pl.ntiles,
                           rpg, lse, pl.part, pl.npart, acc);
    else
        hipLaunchKernelGGL((k_wstats<DP, XT>), dim3(pl.ngroups * pl.ntiles), dim3(512), 0, st,
                           (const XT*)x, n, pl.d, ldx, pl.Pg, pl.cvec, pl.shift, pl.ntiles, rpg,
                           lse, pl.part, pl.npart, acc);
    return hipGetLastError();
}

#define GMM_WIDE_CASES(M) M(256) M(384) M(512) M(640) M(768)

hipError_t launch_wide_lse(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                           double* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                           hipStream_t st, int km) {
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
    if (tm == 0) return launch_wmerge_t<0>(pl, n, lse_out, ll_acc, 0, nullptr, nullptr, 0, st);
    if (tm == 2) return launch_wmerge_t<2>(pl, n, lse_out, ll_acc, m, idx, resp, km, st);
    return launch_wmerge_t<4>(pl, n, lse_out, ll_acc, m, idx, resp, km, st);
}

template <int DP, typename XT>
static hipError_t launch_km_wstats_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                     const int32_t* z, int acc, hipStream_t st) {
    int64_t rpg = (n + pl.ngroups - 1) / pl.ngroups;
    if (rpg < 1) rpg = 1;
    hipLaunchKernelGGL((k_km_wstats<DP, XT>), dim3(pl.ngroups * pl.ntiles), dim3(512), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.shift, z, pl.ntiles, rpg, pl.part, pl.npart,
                       acc);
    return hipGetLastError();
}

hipError_t launch_wide_km_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                                const int32_t* z, int acc, hipStream_t st) {
    switch (pl.dp) {
#define CASE(DPV)                                                                          \
    case DPV:                                                                              \
        return dtype == 0 ? launch_km_wstats_t<DPV, float>(pl, x, n, ldx, z, acc, st)    \
                          : launch_km_wstats_t<DPV, uint16_t>(pl, x, n, ldx, z, acc, st);
        GMM_WIDE_CASES(CASE)
#undef CASE
    }
    return hipErrorInvalidValue;
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
