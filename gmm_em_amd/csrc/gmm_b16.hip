// gmm_b16.hip - the E-step and M-step contractions on split bf16
// (v_mfma_f32_16x16x32_bf16) for data stored in bf16.
//
// The fused EM step ("Flash-GMM: A Memory-Efficient Kernel for Scalable Soft
// Clustering", section 3) contracts, per row n and component k,
//   l[n][k] = sum_d (P2[k][d] a^2 + P1[k][d] a) + c_k,  a = x - s,
//   P2 = -w/2, P1 = w b (w = 1/var, b = mu - s),
// and then the responsibilities r = exp(l - lse) with [a, a^2] over the rows.
// For bf16 data these contractions run on the bf16 matrix units with every
// operand split into bf16 parts whose products are exact in fp32:
//  * the path takes the shift s = 0, so a = x is a bf16 value (8 significant
//    bits), a^2 has at most 16 significant bits and is exactly a2hi + a2lo,
//    two bf16 values (the data pass checks that a^2 and its low bits stay in
//    the normal range);
//  * each coefficient (fp64) is split into three bf16 parts h + m + l, which
//    hold it to about 2^-25 relative;
//  * per 32-dim slice, eight products accumulate in fp32 in increasing order
//    of size (a2lo Pm, a2hi Pl, a Pl1, a2lo Ph, a2hi Pm, a Pm1, a2hi Ph, a Ph1)
//    and the slice sums are added in fp64, so the fp32 rounding acts on one
//    slice at a time: the log-density differs from the fp64 contraction by
//    about 2^-24 of the slice sums' magnitude (sum_d |P2 a^2| + |P1 a| at
//    most). The prologue computes that magnitude from the data's largest |x|
//    per dimension and selects this path only when 2^-23 times it stays
//    below B16_DELTA (2^-7 nats) for every component; otherwise the fp64
//    kernels run. The path has its own constants c_k (b = mu), and selecting
//    it sets the shift to 0 for the finalisation of the statistics.
//  * M-step: r in fp32 (below about 2^-100 it is taken as 0) is rounded to
//    r' = rh + rm, two bf16 parts each rounded to nearest (within 2^-18 of r,
//    relative; exact in fp32), and sum r' a = sum (rm + rh) a, sum r' a^2 =
//    sum (rm a2lo + rh a2lo + rm a2hi + rh a2hi), all products exact, in fp32
//    per 32-row tile and in fp64 across tiles. The mass sum r' is taken from
//    the same values, so the three sums are the statistics of one set of
//    weights r'.
// Both passes contract the E-step in the same order, so they compute the
// same log-densities bit for bit.
//
// MFMA layout (16x16x32 bf16, wave64, measured on gfx950): lane l = 16h + i
// holds A[i][8h .. 8h+7] and B[8h .. 8h+7][i]; register q of the result is
// C[4h + q][i].
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gmm_device.h"
#include "gmm_internal.h"

namespace gmm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf16(v4i a, v4i b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// bf16 bits of a finite fp32 value, rounded to nearest even
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two fp32 values rounded to nearest even bf16, packed (x in the low half):
// one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t bf16_pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// The three feature kinds of two bf16 values a, b, packed in pairs:
// a^2 hi, a^2 lo (a^2 = hi + lo exactly: at most 16 significant bits) and a
__device__ __forceinline__ void b16_features_pack(float a, float b, uint32_t& ph, uint32_t& pl,
                                                  uint32_t& pa) {
    const float a2 = a * a, b2 = b * b;  // exact
    ph = bf16_pack(a2, b2);
    pl = bf16_pack(a2 - bf16_lo(ph), b2 - bf16_hi(ph));  // exact remainders
    pa = bf16_pack(a, b);                                // exact
}

// Feature kind (0: a^2 hi, 1: a^2 lo, 2: a) and coefficient part of product
// m of a slice, in increasing order of size.
__host__ __device__ constexpr int b16_kind(int m) {
    return m == 0 || m == 3 ? 1 : (m == 2 || m == 5 || m == 7 ? 2 : 0);
}

// ---------------------------------------------------------------------------
// Coefficient pieces, one block per 16-component K-tile (256 threads: 16 per
// component). Piece (slice j, product m) holds, at [lane 16h + c][8 values],
// the coefficient part of product m for dims 32j + 8h .. +7 of component c
// (the MFMA B operand). Dims past d and components past k hold 0. Also the
// applicability checks: coefficient range, the rounding estimate, and (block
// 0) the data range per dimension.
// ---------------------------------------------------------------------------

// nearest value with 8 significant bits (fp64; values below 2^-126, where bf16
// loses bits, are flushed to 0)
__device__ __forceinline__ double round_bf16(double r) {
    if (!(fabs(r) >= 0x1p-126)) return 0.0;
    const double sc = ldexp(1.0, ilogb(r) - 7);
    return rint(r / sc) * sc;
}

// p = q0 + q1 + q2 + (residual below 2^-24 |p|); false if p is out of range
__device__ __forceinline__ bool split3(double p, uint32_t (&q)[3]) {
    if (!(fabs(p) < 0x1p126)) {
        q[0] = q[1] = q[2] = 0;
        return false;
    }
    double r = p;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const double v = round_bf16(r);
        q[i] = __float_as_uint((float)v) >> 16;  // exact: 8 significant bits
        r -= v;                                  // exact
    }
    return true;
}

__global__ __launch_bounds__(256) void k_b16_coef(const float* __restrict__ w,
                                                  const float* __restrict__ mu,
                                                  const float* __restrict__ var, int k, int d,
                                                  const unsigned long long* __restrict__ amax,
                                                  const int* __restrict__ lsb,
                                                  uint16_t* __restrict__ coef,
                                                  double* __restrict__ cvec,
                                                  int* __restrict__ status) {
    const int tile = blockIdx.x;
    const int c = threadIdx.x >> 4, sub = threadIdx.x & 15;
    const int slot = tile * 16 + c;
    const bool live = slot < k;
    const int dq = (d + 31) / 32 * 32;
    uint16_t* dst = coef + (size_t)tile * (B16_TILE_BYTES / 2);
    double mag = 0.0, csum = 0.0;
    bool ok = true;
    for (int dd = sub; dd < dq; dd += 16) {
        double p2 = 0.0, p1 = 0.0;
        if (live && dd < d) {
            const double v = (double)var[(int64_t)slot * d + dd];
            const double b = (double)mu[(int64_t)slot * d + dd];
            const double iw = 1.0 / v;
            p2 = -0.5 * iw;
            p1 = iw * b;
            csum += iw * b * b + log(v);
            const double am = __longlong_as_double((long long)amax[dd]);
            mag += fabs(p2) * am * am + fabs(p1) * am;
        }
        uint32_t q2[3], q1[3];
        ok &= split3(p2, q2);
        ok &= split3(p1, q1);
        // parts by product: P2m, P2l, P1l, P2h, P2m, P1m, P2h, P1h
        const uint32_t part[B16_PROD] = {q2[1], q2[2], q1[2], q2[0], q2[1], q1[1], q2[0], q1[0]};
        const int j = dd >> 5, h = (dd >> 3) & 3, e = dd & 7;
#pragma unroll
        for (int m = 0; m < B16_PROD; ++m)
            dst[((j * B16_PROD + m) * 64 + 16 * h + c) * 8 + e] = (uint16_t)part[m];
    }
    // the 16 threads of a component are 16 consecutive lanes
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        mag += __shfl_xor(mag, off);
        csum += __shfl_xor(csum, off);
    }
    if (!ok || (live && !(ldexp(mag, -23) <= B16_DELTA))) atomicOr(&status[I8S_B16FAIL], 1);
    // c_k = log pi_k - 1/2 sum_d (w b^2 + log var) - d/2 log 2 pi, with b = mu
    if (sub == 0) {
        const double LOG_2PI = 1.8378770664093454835606594728112;
        cvec[slot] = live ? log((double)w[slot]) - 0.5 * (csum + (double)d * LOG_2PI) : -INFINITY;
    }
    // a^2 = hi + lo exactly needs a^2 and its low bits in the normal range
    // (amax, lsb: the largest |x| and lowest set bit of x per dimension)
    if (tile == 0 && threadIdx.x < d) {
        const double am = __longlong_as_double((long long)amax[threadIdx.x]);
        if (am > 0.0 && (am >= 0x1p62 || lsb[threadIdx.x] < -63)) atomicOr(&status[I8S_B16FAIL], 1);
    }
}

// ---------------------------------------------------------------------------
// Pass 1 on split bf16: per-row logsumexp over all components. Block = 8
// waves (two per SIMD, so that one wave's VALU work overlaps the other's
// MFMAs), 32 rows per wave (two 16-row MFMA tiles), 256 rows. Each wave
// builds the bf16 features [a^2 hi | a^2 lo | a] of its rows once (through
// LDS, one kind at a time) and keeps them in registers as A operands; the
// K-tiles' coefficient pieces stream through two LDS buffers (tile t+1 is
// copied by buffer-to-LDS loads while tile t is contracted). Per tile and
// slice: eight MFMAs into one fp32 accumulator per row tile; the slice sums
// of the first half of the slices and those of the second half are added in
// fp64 separately, then together (the statistics pass gives the two halves
// to two waves and adds them the same way); the tile's values go into the
// online logsumexp (fp64 running maximum, fp32 scaled sum).
// ---------------------------------------------------------------------------
constexpr int L16_WAVES = 8;
constexpr int L16_RT = 2;  // 16-row tiles per wave
constexpr int L16_ROWS = L16_WAVES * L16_RT * 16;
static_assert(L16_ROWS % LL_ROWS == 0 && LL_ROWS % (L16_RT * 16) == 0,
              "whole log-likelihood partials per block");

// bf16 bits of feature kind kd (0: a^2 hi, 1: a^2 lo, 2: a) of a bf16 value a
__device__ __forceinline__ uint32_t b16_feature(float a, int kd) {
    if (kd == 2) return __float_as_uint(a) >> 16;
    const float a2 = a * a;  // exact: at most 16 significant bits
    const uint32_t hb = bf16_rne(a2);
    return kd == 0 ? hb : __float_as_uint(a2 - bf16_val(hb)) >> 16;  // the rest, exact
}

// rotated position of lane (h, i)'s 16-byte chunk in piece p of a row tile's
// operand pieces (below)
__device__ __forceinline__ int b16_chunk(int h, int i, int p) { return 16 * h + ((i + 4 * h + p) & 15); }

template <int DC>
__global__ __launch_bounds__(L16_WAVES * 64, 1)
void k_lse16(const uint16_t* __restrict__ x, int64_t n, int d, int64_t ldx,
             const uint16_t* __restrict__ coef, const double* __restrict__ cvec, int ntiles,
             double* __restrict__ lse_out, double* __restrict__ llpart, int ll_accumulate,
             uint32_t* __restrict__ pieces, const int* __restrict__ status) {
    constexpr int DQ = 32 * DC;
    constexpr int DCA = (DC + 1) / 2;  // slices of the first half
    constexpr int KS = DQ + 8;         // staged stride of one kind (bf16 values): conflict-free reads
    constexpr int NP = B16_PROD * DC;
    constexpr int NPE = 2 * 3 * DC;    // E pieces of a 32-row tile: (row tile, kind, slice)
    constexpr int NJ = DQ / 16;        // M pieces per kind: 16-column tiles
    constexpr int NPT = NPE + 3 * NJ;  // pieces of a 32-row tile
    constexpr int TBL = NP * 1024;
    constexpr int STG = L16_WAVES * 16 * KS * 2;
    constexpr int TB = TBL > STG ? TBL : STG;
    __shared__ __attribute__((aligned(16))) unsigned char cbuf[2][TB];
    __shared__ double rowll[L16_ROWS];
    if (status[I8S_MODE] != MODE1_B16) return;  // another pass-1 kernel runs instead

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = lane & 15, h = lane >> 4;
    const int64_t wrow = (int64_t)blockIdx.x * L16_ROWS + wave * (L16_RT * 16);

    // ---- features of the wave's rows; lane l handles dims l and l + 64.
    // With `pieces`, the wave's 32 rows (one row tile of the statistics pass)
    // also go out as that pass's MFMA operand pieces, 1 KB each, at
    // pieces[tile][piece]: E pieces (row tile rt, kind, slice j) as the A
    // operands below, and M pieces (kind, column tile J), in which lane (h, i)
    // holds column 16 J + i at rows 4h + q (elements q) and 16 + 4h + q
    // (elements 4 + q); each lane's 16-byte chunk at its rotated position.
    v4i A[L16_RT][3 * DC];
    {
        uint16_t* stg = (uint16_t*)&cbuf[1][wave * 16 * KS * 2];
        const int64_t ptile = wrow / (L16_RT * 16);
        uint32_t* pt = (pieces && wrow < n) ? pieces + ptile * (NPT * 256) : nullptr;
#pragma unroll
        for (int rt = 0; rt < L16_RT; ++rt) {  // unrolled: A stays in registers
            float xv[16][2];
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int64_t row = wrow + rt * 16 + r;
                    const int dd = lane + 64 * u;
                    // rows past n and dims past d are zeros
                    xv[r][u] = (row < n && dd < d) ? load_x(x + row * ldx + dd) : 0.0f;
                }
#pragma unroll
            for (int kd = 0; kd < 3; ++kd) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int dd = lane + 64 * u;
                        if (dd < DQ) stg[r * KS + dd] = (uint16_t)b16_feature(xv[r][u], kd);
                    }
                __syncthreads();
#pragma unroll
                for (int j = 0; j < DC; ++j)
                    A[rt][kd * DC + j] = *(const v4i*)(stg + ci * KS + 32 * j + 8 * h);
                if (pt) {
#pragma unroll
                    for (int j = 0; j < DC; ++j)
                        *(v4i*)(pt + ((rt * 3 + kd) * DC + j) * 256 + b16_chunk(h, ci, j) * 4) =
                            A[rt][kd * DC + j];
#pragma unroll
                    for (int J = 0; J < NJ; ++J) {
                        const uint16_t* col = stg + 4 * h * KS + 16 * J + ci;
                        *(uint2*)(pt + (NPE + kd * NJ + J) * 256 + b16_chunk(h, ci, J) * 4 + 2 * rt) =
                            uint2{(uint32_t)col[0] | ((uint32_t)col[KS] << 16),
                                  (uint32_t)col[2 * KS] | ((uint32_t)col[3 * KS] << 16)};
                    }
                }
                __syncthreads();
            }
        }
    }

    // ---- stream the K-tiles
    auto issue_tile = [&](int t, int buf) {
        const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(coef + (int64_t)t * (B16_TILE_BYTES / 2)), (short)0, TBL, BUF_RSRC_WORD3);
        for (int p = wave; p < NP; p += L16_WAVES)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                cr, (__attribute__((address_space(3))) void*)(cbuf[buf] + p * 1024), 16, lane * 16,
                p * 1024, 0, 0);
    };
    double m[L16_RT][4];
    float s[L16_RT][4];
#pragma unroll
    for (int rt = 0; rt < L16_RT; ++rt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            m[rt][q] = -1.0e300;
            s[rt][q] = 0.0f;
        }
    issue_tile(0, 0);
    double ccn = cvec[ci];  // the next tile's constant, loaded one tile ahead
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
        const double cc = ccn;
        if (t + 1 < ntiles) ccn = cvec[(t + 1) * 16 + ci];
        const unsigned char* cb = cbuf[buf] + lane * 16;
        double la[L16_RT][4], lb[L16_RT][4];
#pragma unroll
        for (int rt = 0; rt < L16_RT; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                la[rt][q] = 0.0;
                lb[rt][q] = 0.0;
            }
#pragma unroll
        for (int j = 0; j < DC; ++j) {
            f32x4 acc[L16_RT];
#pragma unroll
            for (int rt = 0; rt < L16_RT; ++rt) acc[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int mm = 0; mm < B16_PROD; ++mm) {
                const v4i b = *(const v4i*)(cb + (j * B16_PROD + mm) * 1024);
#pragma unroll
                for (int rt = 0; rt < L16_RT; ++rt)
                    acc[rt] = mfma_bf16(A[rt][b16_kind(mm) * DC + j], b, acc[rt]);
            }
#pragma unroll
            for (int rt = 0; rt < L16_RT; ++rt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (j < DCA) la[rt][q] += (double)acc[rt][q];
                    else lb[rt][q] += (double)acc[rt][q];
                }
        }
#pragma unroll
        for (int rt = 0; rt < L16_RT; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) lse_push(m[rt][q], s[rt][q], (la[rt][q] + lb[rt][q]) + cc);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile t+1 have landed
        __syncthreads();                // ... and every wave's; tile t's buffer is free
    }

    // ---- merge the 16 lanes holding the same rows (fixed butterfly order)
#pragma unroll
    for (int rt = 0; rt < L16_RT; ++rt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll 1
            for (int off = 1; off < 16; off <<= 1) {
                const double m2 = shfl_xor_d(m[rt][q], off);
                const float s2 = __shfl_xor(s[rt][q], off);
                lse_merge(m[rt][q], s[rt][q], m2, s2);
            }
        }
    if (ci == 0) {
#pragma unroll
        for (int rt = 0; rt < L16_RT; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int lr = wave * (L16_RT * 16) + rt * 16 + 4 * h + q;
                const int64_t row = (int64_t)blockIdx.x * L16_ROWS + lr;
                double v = 0.0;
                if (row < n) {
                    v = m[rt][q] + log((double)s[rt][q]);
                    if (lse_out) lse_out[row] = v;
                }
                rowll[lr] = v;
            }
    }
    __syncthreads();
    // one partial per 64 rows (fixed order)
    if (wave < L16_ROWS / LL_ROWS) {
        double tot = rowll[wave * LL_ROWS + lane];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) tot += shfl_xor_d(tot, off);
        const int64_t pi = (int64_t)blockIdx.x * (L16_ROWS / LL_ROWS) + wave;
        if (lane == 0 && pi * LL_ROWS < n) llpart[pi] = (ll_accumulate ? llpart[pi] : 0.0) + tot;
    }
}

// ---------------------------------------------------------------------------
// Pass 2 on split bf16: statistics. Block = 8 waves for 4 K-tiles (two waves
// per SIMD): waves 0-3 are E-waves, waves 4-7 M-waves, and the two waves of
// a SIMD own the same K-tile kg*4 + (wave & 3). The block walks its row group
// in 32-row tiles, one barrier per tile, as a two-stage pipeline:
//  * the next tile's bf16 features arrive in LDS by buffer-to-LDS copies of
//    the 1 KB MFMA operand pieces the normaliser pass wrote for it (every
//    wave copies some): E pieces (row tile, kind, slice) for the E-step's A
//    operand, M pieces (kind, 16-column tile) for the M-step's, in which
//    lane (h, i) holds column i at the rows 4h .. 4h+3 and 16+4h .. 16+4h+3;
//    a piece's 16-byte lane chunks are rotated (chunk 16h + (i + 4h + p) mod
//    16 for piece p) so that the MFMA lanes' reads hit distinct banks;
//  * the E-wave keeps all the K-tile's coefficient pieces in registers,
//    contracts the tile exactly as the normaliser pass does (same order,
//    same bits), forms r = exp(l - lse), rounds it to two bf16 parts and
//    hands them to its M-wave through LDS (the E-step result leaves lane
//    (h, i) with rows 16 rt + 4h + q of component i, which are the lane's 8
//    positions of the M-step contraction);
//  * the M-wave, one tile behind, contracts those parts with the tile's M
//    pieces into fp32 per tile and fp64 totals (skipping a tile whose
//    responsibilities are all 0).
// The two roles run different code on a SIMD at the same time, so one
// wave's VALU work (exponentials, splits, fp64 folds) overlaps the other's
// MFMAs. The features are triple-buffered for the M-waves' lag.
// ---------------------------------------------------------------------------
template <int DC>
__global__ __launch_bounds__(512, 1)
void k_stats16(int64_t n, int dp, const uint32_t* __restrict__ pieces,
               const uint16_t* __restrict__ coef, const double* __restrict__ cvec, int ntiles,
               const double* __restrict__ lse, int64_t rows_per_group, double* __restrict__ part,
               double* __restrict__ npart, int accumulate, const int* __restrict__ status) {
    constexpr int KT = 4;       // K-tiles per block
    constexpr int DQ = 32 * DC;
    constexpr int DCA = (DC + 1) / 2;   // slices of the first half
    constexpr int NJ = DQ / 16;         // 16-column M-step tiles per feature kind
    constexpr int NPE = 2 * 3 * DC;     // E pieces per tile: (row tile, kind, slice)
    constexpr int NPM = 3 * NJ;         // M pieces per tile: (kind, column tile)
    constexpr int NPT = NPE + NPM;
    __shared__ __attribute__((aligned(16))) uint32_t fe[2][NPE * 256];
    __shared__ __attribute__((aligned(16))) uint32_t fm[3][NPM * 256];
    __shared__ __attribute__((aligned(16))) uint32_t rr[2][KT][2 * 256];  // r parts per K-tile
    __shared__ double ls[2][STATS_ROWS];
    __shared__ int anyr[2][KT];
    if (status[I8S_MODE2] != MODE2_B16) return;  // another statistics pass runs instead

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = lane & 15, h = lane >> 4;
    const int kq = wave & 3;
    const bool ewave = wave < 4;
    const int kgroups = ntiles / KT;
    const int nb = gridDim.x;
    // blocks of one XCD take consecutive (row group, K-group) pairs: the
    // K-groups of a row group share that XCD's L2 copy of the rows
    const int o = (nb % 8 == 0) ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
    const int g = o / kgroups;
    const int tile = (o % kgroups) * KT + kq;
    const int slot = tile * 16 + ci;

    const int64_t gr0 = (int64_t)g * rows_per_group;
    int64_t gr1 = gr0 + rows_per_group;
    if (gr1 > n) gr1 = n;
    const int64_t ntile_rows = gr1 > gr0 ? (gr1 - gr0 + STATS_ROWS - 1) / STATS_ROWS : 0;

    // tile it's pieces into E buffer be and M buffer bm (every wave copies
    // some), and the normaliser of row tid (+inf past the row group: r = 0)
    auto issue = [&](int64_t it, int be, int bm) {
        const int64_t tile_g = (gr0 + it * STATS_ROWS) / STATS_ROWS;
        const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(pieces + tile_g * (NPT * 256)), (short)0, NPT * 1024, BUF_RSRC_WORD3);
        for (int p = wave; p < NPT; p += 8) {
            uint32_t* dst = p < NPE ? fe[be] + p * 256 : fm[bm] + (p - NPE) * 256;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(pr, (__attribute__((address_space(3))) void*)dst, 16,
                                                     lane * 16, p * 1024, 0, 0);
        }
    };
    auto load_ls = [&](int64_t it) -> double {
        const int64_t rbase = gr0 + it * STATS_ROWS;
        const int64_t nv = gr1 - rbase;
        return tid < nv ? lse[rbase + tid] : INFINITY;
    };
    // the pipeline's shared step: copy tile it+1 (it lands before the barrier)
    double lsn = 0.0;
    auto next_issue = [&](int64_t it) {
        if (it + 1 < ntile_rows) {
            issue(it + 1, (int)((it + 1) & 1), (int)((it + 1) % 3));
            if (tid < STATS_ROWS) lsn = load_ls(it + 1);
        }
    };
    auto next_finish = [&](int64_t it) {
        if (it + 1 < ntile_rows && tid < STATS_ROWS) ls[(it + 1) & 1][tid] = lsn;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
    };

    if (ntile_rows > 0) {
        issue(0, 0, 0);
        if (tid < STATS_ROWS) ls[0][tid] = load_ls(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    if (ewave) {
        // ---- E-wave: E-step, responsibilities and their parts for tile it
        v4i qb[B16_PROD * DC];  // the K-tile's coefficient pieces (B operands), resident
        {
            const uint16_t* cp = coef + (int64_t)tile * (B16_TILE_BYTES / 2) + lane * 8;
#pragma unroll
            for (int p = 0; p < B16_PROD * DC; ++p) qb[p] = *(const v4i*)(cp + p * 512);
        }
        const double cc = cvec[slot];
        double n64 = 0.0;
        for (int64_t it = 0; it <= ntile_rows; ++it) {
            next_issue(it);
            if (it < ntile_rows) {
                const int be = (int)(it & 1);
                const uint32_t* F = fe[be];
                double la[2][4], lb[2][4];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        la[rt][q] = 0.0;
                        lb[rt][q] = 0.0;
                    }
#pragma unroll
                for (int j = 0; j < DC; ++j) {
                    v4i a[2][3];
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                        for (int kd = 0; kd < 3; ++kd)
                            a[rt][kd] = *(const v4i*)(F + ((rt * 3 + kd) * DC + j) * 256 +
                                                      b16_chunk(h, ci, j) * 4);
                    f32x4 acc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
                    for (int mm = 0; mm < B16_PROD; ++mm)
#pragma unroll
                        for (int rt = 0; rt < 2; ++rt)
                            acc[rt] = mfma_bf16(a[rt][b16_kind(mm)], qb[j * B16_PROD + mm], acc[rt]);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if (j < DCA) la[rt][q] += (double)acc[rt][q];
                            else lb[rt][q] += (double)acc[rt][q];
                        }
                }
                // responsibilities of rows 16 rt + 4h + q (element 4 rt + q of
                // the M-step's B operands), rounded to two bf16 parts below
                float rv[8];
                bool any = false;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // the exponent in fp64, then fp32 (|t| < 70 where r is kept)
                        const float tf = (float)(((la[rt][q] + lb[rt][q]) + cc) -
                                                 ls[be][16 * rt + 4 * h + q]);
                        const float r = tf > -69.3147181f ? __builtin_amdgcn_exp2f(tf * 1.44269504f)
                                                          : 0.0f;  // below about 2^-100: 0
                        any |= r != 0.0f;
                        rv[4 * rt + q] = r;
                    }
                uint32_t* R = rr[be][kq];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    uint32_t ph[2], pm[2];
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        // r' = rh + rm (each rounded to nearest), exact in fp32;
                        // the mass takes the same r' as the moments
                        const float x = rv[4 * w + 2 * v], y = rv[4 * w + 2 * v + 1];
                        ph[v] = bf16_pack(x, y);
                        pm[v] = bf16_pack(x - bf16_lo(ph[v]), y - bf16_hi(ph[v]));
                        n64 += (double)(bf16_lo(ph[v]) + bf16_lo(pm[v]));
                        n64 += (double)(bf16_hi(ph[v]) + bf16_hi(pm[v]));
                    }
                    *(uint2*)(R + lane * 4 + 2 * w) = uint2{ph[0], ph[1]};
                    *(uint2*)(R + 256 + lane * 4 + 2 * w) = uint2{pm[0], pm[1]};
                }
                const bool wany = __builtin_amdgcn_ballot_w64(any) != 0;
                if (lane == 0) anyr[be][kq] = wany ? 1 : 0;
            }
            next_finish(it);
            __syncthreads();
        }
        // responsibility mass: lanes ci, ci+16, ci+32, ci+48 hold disjoint rows
        n64 += shfl_xor_d(n64, 16);
        n64 += shfl_xor_d(n64, 32);
        if (h == 0) {
            double* np = npart + (int64_t)g * ntiles * 16 + slot;
            *np = (accumulate ? *np : 0.0) + n64;
        }
    } else {
        // ---- M-wave: M-step of tile it - 1
        double tA[NJ][4], tB[NJ][4];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                tA[j][q] = 0.0;
                tB[j][q] = 0.0;
            }
        for (int64_t it = 0; it <= ntile_rows; ++it) {
            next_issue(it);
            if (it >= 1) {
                const int be = (int)((it - 1) & 1), bm = (int)((it - 1) % 3);
                if (anyr[be][kq] != 0) {
                    const uint32_t* R = rr[be][kq];
                    const v4i Rh = *(const v4i*)(R + lane * 4);
                    const v4i Rm = *(const v4i*)(R + 256 + lane * 4);
                    const uint32_t* M = fm[bm];
#pragma unroll
                    for (int J = 0; J < NJ; ++J) {
                        const int co = b16_chunk(h, ci, J) * 4;
                        const v4i fh = *(const v4i*)(M + J * 256 + co);
                        const v4i fl = *(const v4i*)(M + (NJ + J) * 256 + co);
                        const v4i fa = *(const v4i*)(M + (2 * NJ + J) * 256 + co);
                        f32x4 sa = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, sb = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                        sa = mfma_bf16(fa, Rm, sa);
                        sa = mfma_bf16(fa, Rh, sa);
                        sb = mfma_bf16(fl, Rm, sb);
                        sb = mfma_bf16(fl, Rh, sb);
                        sb = mfma_bf16(fh, Rm, sb);
                        sb = mfma_bf16(fh, Rh, sb);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            tA[J][q] += (double)sa[q];
                            tB[J][q] += (double)sb[q];
                        }
                    }
                }
            }
            next_finish(it);
            __syncthreads();
        }
        double* pp = part + ((int64_t)g * ntiles * 16 + slot) * (2 * (int64_t)dp);
#pragma unroll
        for (int J = 0; J < NJ; ++J)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int dd = 16 * J + 4 * h + q;
                if (dd < dp) {
                    pp[dd] = (accumulate ? pp[dd] : 0.0) + tA[J][q];
                    pp[dp + dd] = (accumulate ? pp[dp + dd] : 0.0) + tB[J][q];
                }
            }
    }
}
// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_b16_coef(const Plan& pl, const float* w, const float* mu, const float* var,
                           hipStream_t st) {
    hipLaunchKernelGGL(k_b16_coef, dim3(pl.ntiles), dim3(256), 0, st, w, mu, var, pl.k, pl.d,
                       pl.b16_amax, pl.b16_lsb, pl.b16_coef, pl.b16_cvec, pl.status);
    return hipGetLastError();
}

hipError_t launch_lse16(const Plan& pl, const void* x, int64_t n, int64_t ldx, double* lse_out,
                        int ll_acc, bool pieces, hipStream_t st) {
    if (pieces && n > pl.b16_chunk) return hipErrorInvalidValue;  // the pieces buffer's rows
    if (n <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n + L16_ROWS - 1) / L16_ROWS)), block(L16_WAVES * 64);
    const uint16_t* xb = (const uint16_t*)x;
    switch ((pl.d + 31) / 32) {
#define CASE(DCV)                                                                               \
    case DCV:                                                                                   \
        hipLaunchKernelGGL((k_lse16<DCV>), grid, block, 0, st, xb, n, pl.d, ldx, pl.b16_coef,   \
                           pl.b16_cvec, pl.ntiles, lse_out, pl.llpart, ll_acc,                  \
                           pieces ? pl.b16_pieces : nullptr, pl.status);                        \
        break;
        CASE(1) CASE(2) CASE(3) CASE(4)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_stats16(const Plan& pl, int64_t n, const double* lse, int acc, hipStream_t st) {
    if (n > pl.b16_chunk) return hipErrorInvalidValue;  // the pieces the normaliser pass wrote
    int64_t rpg = ((n + pl.ngroups - 1) / pl.ngroups + STATS_ROWS - 1) / STATS_ROWS * STATS_ROWS;
    if (rpg < STATS_ROWS) rpg = STATS_ROWS;
    const dim3 grid(pl.ngroups * (pl.ntiles / 4)), block(512);
    switch ((pl.d + 31) / 32) {
#define CASE(DCV)                                                                              \
    case DCV:                                                                                  \
        hipLaunchKernelGGL((k_stats16<DCV>), grid, block, 0, st, n, pl.dp, pl.b16_pieces,      \
                           pl.b16_coef, pl.b16_cvec, pl.ntiles, lse, rpg, pl.part, pl.npart,   \
                           acc, pl.status);                                                    \
        break;
        CASE(1) CASE(2) CASE(3) CASE(4)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gmm
