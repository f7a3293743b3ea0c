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
// Arithmetic layout
// -----------------
// For component k and a per-tile shift vector t (all components of one
// 16-wide K-tile share t), with a = x - t, w = 1/var, b = mu - t:
//   l[n][k] = sum_d ( w b a  - w a^2 / 2 ) + c_k,
//   c_k     = log pi_k - 1/2 sum_d ( w b^2 + log var ) - D/2 log 2 pi.
// The sum over d is a dense contraction of the feature rows [a, a^2] with the
// coefficient rows [w b, -w/2]: v_mfma_f32_16x16x4_f32, fp32 in and fp32
// accumulate. The shift keeps the features small, which keeps fp32 rounding
// in the expanded form small.
//
// MFMA operand layout (16x16x4 f32, wave64): lane l = 16*h + i.
//   A operand: A[i][h], B operand: B[h][i], C: lane holds C[4h + q][i], q=0..3.
// E-step: A = features (row i of a 16-row block), B = coefficients (component
//   i of a 16-wide K-tile); step t uses feature (dim 2t + (h>>1), power 1 +
//   (h&1)); C[row 4h+q][comp i] = l.
// M-step: the E-step C registers are used unchanged as the A operand
//   (A[comp i][row 4h+q] for step q), the B operand is feature column
//   16j + i of row 4h + q; C[comp 4h+q][feature 16j+i] accumulates
//   sum_n r[n][comp] * feature[n]. The responsibilities never leave registers.
//
// Two passes per row chunk (the M-step of a component needs each row's
// normaliser over ALL components before any of its responsibilities exist):
//   pass 1 (k_lse):   row-stationary; every K-tile streams through LDS; a
//                     per-row online logsumexp; writes lse per row and fp64
//                     log-likelihood partials.
//   pass 2 (k_stats): K-tile-stationary (coefficients in registers, fp32
//                     statistics in MFMA accumulators, flushed into fp64
//                     registers every 64-row tile); recomputes l with the same
//                     instruction sequence as pass 1, so both passes see
//                     bitwise identical log-densities.
// Partials are summed in a fixed order in fp64 by k_finalize: no atomics on
// floating-point data, bitwise reproducible results.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "gmm_internal.h"

namespace gmm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_x(const float* p) { return *p; }
__device__ __forceinline__ float load_x(const uint16_t* p) {
    return __uint_as_float(((uint32_t)(*p)) << 16);
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Feature value of one E-step operand: a = x - s, and a or a^2.
__device__ __forceinline__ float feat(float x, float s, bool sq) {
    float a = x - s;
    return a * (sq ? a : 1.0f);
}

// Online logsumexp update of (m, s) with value v.
__device__ __forceinline__ void lse_push(float& m, float& s, float v) {
    float mn = fmaxf(m, v);
    s = s * __expf(m - mn) + __expf(v - mn);
    m = mn;
}
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    float mn = fmaxf(m, m2);
    s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
    m = mn;
}

// ---------------------------------------------------------------------------
// Prologue: parameter checks, shift, coefficient rows and constants.
// ---------------------------------------------------------------------------
__global__ void k_status_reset(int* status) {
    if (threadIdx.x < 4) status[threadIdx.x] = 0;
}

__global__ void k_validate(const float* __restrict__ w, const float* __restrict__ mu,
                           const float* __restrict__ var, int k, int d, int* status) {
    int64_t total = (int64_t)k * d;
    int bad = 0, anypos = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        float m = mu[i], v = var[i];
        if (!isfinite(m) || !isfinite(v) || !(v > 0.0f)) bad = 1;
        if (i < k) {
            float wi = w[i];
            if (!isfinite(wi) || wi < 0.0f) bad = 1;
            if (wi > 0.0f) anypos = 1;
        }
    }
    if (bad) atomicOr(&status[0], 1);
    if (anypos) atomicOr(&status[1], 1);
}

// Global shift: s_d = rint(mean_k mu[k][d]) (fp64 mean). Written for every
// K-tile in the permuted dim order used by the kernels:
// pos(d) = (d & 1) * DP/2 + d / 2.
__global__ void k_shift(const float* __restrict__ mu, int k, int d, int dp, int ntiles,
                        float* __restrict__ tshift) {
    int dd = blockIdx.x * blockDim.x + threadIdx.x;
    if (dd >= dp) return;
    float sv = 0.0f;
    if (dd < d) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j) acc += (double)mu[(int64_t)j * d + dd];
        sv = (float)rint(acc / (double)k);
        if (!isfinite(sv)) sv = 0.0f;
    }
    int pos = (dd & 1) * (dp >> 1) + (dd >> 1);
    for (int j = 0; j < ntiles; ++j) tshift[(int64_t)j * dp + pos] = sv;
}

// Coefficients for slot `blockIdx.x` (component perm[slot], or padding):
//   Pg[slot][h][t]: h&1 = 0 -> w*b of dim 2t+(h>>1), h&1 = 1 -> -w/2.
//   cvec[slot] = log pi - 1/2 sum_d (w b^2 + log var) - D/2 log 2pi.
__global__ void k_params(const float* __restrict__ w, const float* __restrict__ mu,
                         const float* __restrict__ var, const int* __restrict__ perm, int k, int d,
                         int dp, const float* __restrict__ tshift, float* __restrict__ Pg,
                         float* __restrict__ cvec) {
    __shared__ double red[256];
    const int slot = blockIdx.x;
    const int comp = perm[slot];
    const int tile = slot >> 4;
    const int dph = dp >> 1;
    double part = 0.0;
    for (int dd = threadIdx.x; dd < dp; dd += blockDim.x) {
        float cb = 0.0f, cq = 0.0f;
        if (comp >= 0 && dd < d) {
            double v = (double)var[(int64_t)comp * d + dd];
            double s = (double)tshift[(int64_t)tile * dp + (dd & 1) * dph + (dd >> 1)];
            double b = (double)mu[(int64_t)comp * d + dd] - s;
            double iw = 1.0 / v;
            cb = (float)(iw * b);
            cq = (float)(-0.5 * iw);
            part += iw * b * b + log(v);
        }
        const int t = dd >> 1, hh = (dd & 1) << 1;
        float* row = Pg + (int64_t)slot * 2 * dp;
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
        if (comp < 0) {
            cvec[slot] = -INFINITY;
        } else {
            const double LOG_2PI = 1.8378770664093454835606594728112;
            double wk = (double)w[comp];
            double c = log(wk) - 0.5 * (red[0] + (double)d * LOG_2PI);
            cvec[slot] = (float)c;
        }
    }
}

// ---------------------------------------------------------------------------
// Pass 1: per-row logsumexp over all components.
// Block: 4 waves x 2 row blocks of 16 rows = 128 rows. Each lane keeps the
// features' source values (x of dims 2t + (h>>1)) of its two rows in
// registers; the K-tiles' coefficient rows, shifts and constants stream
// through double-buffered LDS.
// ---------------------------------------------------------------------------
// Ordered insertion of (v, i) into a top list sorted by larger value first,
// then smaller index (empty entries hold -inf and the largest index).
template <int TM>
__device__ __forceinline__ void top_push(float (&tv)[TM], int (&ti)[TM], float v, int i) {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const bool gt = v > tv[j] || (v == tv[j] && i < ti[j]);
        const float ov = tv[j];
        const int oi = ti[j];
        tv[j] = gt ? v : ov;
        ti[j] = gt ? i : oi;
        v = gt ? ov : v;
        i = gt ? oi : i;
    }
}

// Merge with the top list of lane (lane ^ off): both lanes end with the same
// top TM of the union (order: larger value first, then smaller index).
template <int TM>
__device__ __forceinline__ void top_merge(float (&tv)[TM], int (&ti)[TM], int off) {
    float ov[TM];
    int oi[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        ov[j] = __shfl_xor(tv[j], off);
        oi[j] = __shfl_xor(ti[j], off);
    }
    float rv[TM];
    int ri[TM];
    int a = 0, b = 0;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        float va = tv[0], vb = ov[0];
        int ia = ti[0], ib = oi[0];
#pragma unroll
        for (int u = 1; u < TM; ++u) {
            if (a == u) { va = tv[u]; ia = ti[u]; }
            if (b == u) { vb = ov[u]; ib = oi[u]; }
        }
        const bool take_a = (va > vb) || (va == vb && ia < ib);
        rv[j] = take_a ? va : vb;
        ri[j] = take_a ? ia : ib;
        a += take_a ? 1 : 0;
        b += take_a ? 0 : 1;
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) { tv[j] = rv[j]; ti[j] = ri[j]; }
}

template <int DP, typename XT, int TM>
__global__ __launch_bounds__(256, DP <= 64 ? 2 : 1)
void k_lse(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
           const float* __restrict__ Pg, const float* __restrict__ cvec,
           const float* __restrict__ tshift, int ntiles, float* __restrict__ lse_out,
           double* __restrict__ llpart, int ll_accumulate, const int* __restrict__ status,
           int m_out, const int* __restrict__ perm, int32_t* __restrict__ idx_out,
           float* __restrict__ resp_out) {
    constexpr int TMA = TM > 0 ? TM : 1;
    constexpr int DPH = DP / 2;
    constexpr int PSTR = 2 * DP + 4;  // LDS stride of one component's coefficients
    __shared__ __attribute__((aligned(16))) float Pt[2][16 * PSTR];
    __shared__ __attribute__((aligned(16))) float St[2][DP];
    __shared__ float Ct[2][16];
    __shared__ double rowll[128];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ci = lane & 15, h = lane >> 4, half = h >> 1;
    const bool sq = h & 1;
    const int64_t row0 = (int64_t)blockIdx.x * 128 + wave * 32;

    // x values for this lane's two rows: dims 2t + half.
    float xr[2][DPH];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int64_t row = row0 + rb * 16 + ci;
        const bool ok = row < n;
        const XT* xp = x + (ok ? row : 0) * ldx;
#pragma unroll
        for (int t = 0; t < DPH; ++t) {
            const int dd = 2 * t + half;
            xr[rb][t] = (ok && dd < d) ? load_x(xp + dd) : 0.0f;
        }
    }

    auto stage = [&](int tile, int buf) {
        const float* src = Pg + (int64_t)tile * 16 * 2 * DP;
        for (int i = tid; i < 16 * 2 * DP / 4; i += 256) {
            const int e = i * 4;
            const int comp = e / (2 * DP), off = e % (2 * DP);
            *(float4*)&Pt[buf][comp * PSTR + off] = *(const float4*)(src + e);
        }
        for (int i = tid; i < DP; i += 256) St[buf][i] = tshift[(int64_t)tile * DP + i];
        if (tid < 16) Ct[buf][tid] = cvec[tile * 16 + tid];
    };

    float m[2][4], s[2][4];
    float tv[2][4][TMA];
    int ti[2][4][TMA];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            m[rb][q] = -3.0e38f;
            s[rb][q] = 0.0f;
#pragma unroll
            for (int j = 0; j < TMA; ++j) { tv[rb][q][j] = -INFINITY; ti[rb][q][j] = 0x7fffffff; }
        }

    stage(0, 0);
    __syncthreads();
    for (int tile = 0; tile < ntiles; ++tile) {
        const int buf = tile & 1;
        if (tile + 1 < ntiles) stage(tile + 1, buf ^ 1);
        const float* pp = &Pt[buf][ci * PSTR + h * DPH];
        const float* sp = &St[buf][half * DPH];
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DPH; t += 4) {
            const float4 pv = *(const float4*)(pp + t);
            const float4 sv = *(const float4*)(sp + t);
            acc0 = mfma4(feat(xr[0][t + 0], sv.x, sq), pv.x, acc0);
            acc1 = mfma4(feat(xr[1][t + 0], sv.x, sq), pv.x, acc1);
            acc0 = mfma4(feat(xr[0][t + 1], sv.y, sq), pv.y, acc0);
            acc1 = mfma4(feat(xr[1][t + 1], sv.y, sq), pv.y, acc1);
            acc0 = mfma4(feat(xr[0][t + 2], sv.z, sq), pv.z, acc0);
            acc1 = mfma4(feat(xr[1][t + 2], sv.z, sq), pv.z, acc1);
            acc0 = mfma4(feat(xr[0][t + 3], sv.w, sq), pv.w, acc0);
            acc1 = mfma4(feat(xr[1][t + 3], sv.w, sq), pv.w, acc1);
        }
        const float c = Ct[buf][ci];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float l0 = acc0[q] + c, l1 = acc1[q] + c;
            lse_push(m[0][q], s[0][q], l0);
            lse_push(m[1][q], s[1][q], l1);
            if constexpr (TM > 0) {
                top_push<TM>(tv[0][q], ti[0][q], l0, tile * 16 + ci);
                top_push<TM>(tv[1][q], ti[1][q], l1, tile * 16 + ci);
            }
        }
        __syncthreads();
    }

    // Merge the 16 lanes that hold the same rows (fixed butterfly order).
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll 1
            for (int off = 1; off < 16; off <<= 1) {
                float m2 = __shfl_xor(m[rb][q], off);
                float s2 = __shfl_xor(s[rb][q], off);
                lse_merge(m[rb][q], s[rb][q], m2, s2);
                if constexpr (TM > 0) top_merge<TM>(tv[rb][q], ti[rb][q], off);
            }
        }
    if (ci == 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int lr = wave * 32 + rb * 16 + 4 * h + q;
                const int64_t row = (int64_t)blockIdx.x * 128 + lr;
                double v = 0.0;
                if (row < n) {
                    const float lse = m[rb][q] + __logf(s[rb][q]);
                    if (lse_out) lse_out[row] = lse;
                    v = (double)m[rb][q] + log((double)s[rb][q]);
                    if constexpr (TM > 0) {
                        for (int j = 0; j < m_out; ++j) {
                            const int sl = ti[rb][q][j];
                            idx_out[row * m_out + j] = perm[sl];
                            resp_out[row * m_out + j] = __expf(tv[rb][q][j] - lse);
                        }
                    }
                }
                rowll[lr] = v;
            }
    }
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int i = 0; i < 128; ++i) tot += rowll[i];
        llpart[blockIdx.x] = (ll_accumulate ? llpart[blockIdx.x] : 0.0) + tot;
    }
    (void)status;
}

// ---------------------------------------------------------------------------
// Pass 2: statistics. Block = 4 waves; wave w owns K-tile kg*4 + w (16
// components): its coefficients stay in registers, its fp32 statistics in
// MFMA accumulators. The block walks the rows of its row group in 64-row
// tiles staged (double-buffered) in LDS in the permuted dim order.
// ---------------------------------------------------------------------------
template <int DP, typename XT>
__global__ __launch_bounds__(256, DP <= 64 ? 2 : 1)
void k_stats(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
             const float* __restrict__ Pg, const float* __restrict__ cvec,
             const float* __restrict__ tshift, int ntiles, const float* __restrict__ lse,
             int64_t rows_per_group, int ngroups, double* __restrict__ part,
             double* __restrict__ npart, int accumulate) {
    constexpr int DPH = DP / 2;
    constexpr int XS = DP + 4;      // LDS row stride (floats)
    constexpr int NJ = DP / 16;     // 16-dim column blocks per power
    __shared__ __attribute__((aligned(16))) float xs[2][64 * XS];
    __shared__ __attribute__((aligned(16))) float ts[4][DP];
    __shared__ float ls[2][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ci = lane & 15, h = lane >> 4, half = h >> 1;
    const bool sq = h & 1;
    const int kgroups = ntiles >> 2;
    const int g = blockIdx.x / kgroups;
    const int tile = (blockIdx.x % kgroups) * 4 + wave;
    const int slot = tile * 16 + ci;

    // Stationary coefficients: P[slot][h][t], t = 0..DPH-1.
    float pr[DPH];
    {
        const float* src = Pg + (int64_t)slot * 2 * DP + h * DPH;
#pragma unroll
        for (int t = 0; t < DPH; t += 4) {
            float4 v = *(const float4*)(src + t);
            pr[t] = v.x; pr[t + 1] = v.y; pr[t + 2] = v.z; pr[t + 3] = v.w;
        }
    }
    const float cc = cvec[slot];
    for (int i = lane; i < DP; i += 64) ts[wave][i] = tshift[(int64_t)tile * DP + i];
    // Shift of dims 16j + ci for the M-step features.
    float tm[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int dd = 16 * j + ci;
        tm[j] = tshift[(int64_t)tile * DP + (dd & 1) * DPH + (dd >> 1)];
    }

    f32x4 acc[2 * NJ];
    double acc64[2 * NJ][4];
#pragma unroll
    for (int j = 0; j < 2 * NJ; ++j) {
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) acc64[j][q] = 0.0;
    }
    double n64 = 0.0;

    const int64_t gr0 = (int64_t)g * rows_per_group;
    int64_t gr1 = gr0 + rows_per_group;
    if (gr1 > n) gr1 = n;
    const int64_t ntile_rows = gr1 > gr0 ? (gr1 - gr0 + 63) / 64 : 0;

    auto stage = [&](int64_t it, int buf) {
        const int64_t rbase = gr0 + it * 64;
        for (int i = tid; i < 64 * DP; i += 256) {
            const int r = i / DP, dd = i % DP;
            const int64_t row = rbase + r;
            float v = 0.0f;
            if (row < gr1 && dd < d) v = load_x(x + row * ldx + dd);
            xs[buf][r * XS + (dd & 1) * DPH + (dd >> 1)] = v;
        }
        if (tid < 64) {
            const int64_t row = rbase + tid;
            ls[buf][tid] = row < gr1 ? lse[row] : INFINITY;
        }
    };

    if (ntile_rows > 0) stage(0, 0);
    __syncthreads();
    for (int64_t it = 0; it < ntile_rows; ++it) {
        const int buf = it & 1;
        if (it + 1 < ntile_rows) stage(it + 1, buf ^ 1);
        const float* xb = xs[buf];
#pragma unroll 1
        for (int rb = 0; rb < 4; ++rb) {
            // E-step: l for rows 16rb + 4h + q, component slot.
            const float* xa = xb + (rb * 16 + ci) * XS + half * DPH;
            const float* sa = &ts[wave][half * DPH];
            f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < DPH; t += 4) {
                const float4 xv = *(const float4*)(xa + t);
                const float4 sv = *(const float4*)(sa + t);
                e = mfma4(feat(xv.x, sv.x, sq), pr[t + 0], e);
                e = mfma4(feat(xv.y, sv.y, sq), pr[t + 1], e);
                e = mfma4(feat(xv.z, sv.z, sq), pr[t + 2], e);
                e = mfma4(feat(xv.w, sv.w, sq), pr[t + 3], e);
            }
            float r[4];
            float rsum = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float l = e[q] + cc;
                r[q] = __expf(l - ls[buf][rb * 16 + 4 * h + q]);
                rsum += r[q];
            }
            n64 += (double)rsum;
            // M-step: A = r (component ci, row 4h+q), B = feature column 16j+ci.
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float* xm = xb + (rb * 16 + 4 * h + q) * XS;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int dd = 16 * j + ci;
                    const float a = xm[(dd & 1) * DPH + (dd >> 1)] - tm[j];
                    acc[j] = mfma4(r[q], a, acc[j]);
                    acc[NJ + j] = mfma4(r[q], a * a, acc[NJ + j]);
                }
            }
        }
        // Flush the 64-row fp32 partial into fp64.
#pragma unroll
        for (int j = 0; j < 2 * NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc64[j][q] += (double)acc[j][q];
                acc[j][q] = 0.0f;
            }
        __syncthreads();
    }

    // Responsibility mass: lanes ci, ci+16, ci+32, ci+48 hold disjoint rows.
    {
        double o = __shfl_xor(n64, 16);
        n64 += o;
        o = __shfl_xor(n64, 32);
        n64 += o;
    }
    const int64_t gbase = (int64_t)g * ntiles * 16;
    if (h == 0) {
        double* np = npart + gbase + slot;
        *np = (accumulate ? *np : 0.0) + n64;
    }
#pragma unroll
    for (int j = 0; j < 2 * NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int comp = tile * 16 + 4 * h + q;
            double* p = part + (gbase + comp) * (2 * DP) + 16 * j + ci;
            *p = (accumulate ? *p : 0.0) + acc64[j][q];
        }
}

// ---------------------------------------------------------------------------
// Finalize: fixed-order fp64 sum over row groups, then the M-step update.
// ---------------------------------------------------------------------------
__global__ void k_finalize(const double* __restrict__ part, const double* __restrict__ npart,
                           int ngroups, int kp, int dp, int d, const int* __restrict__ perm,
                           const float* __restrict__ tshift, int64_t n, float var_floor,
                           float* __restrict__ w, float* __restrict__ mu, float* __restrict__ var,
                           const int* __restrict__ status) {
    const int slot = blockIdx.x;
    const int comp = perm[slot];
    if (comp < 0) return;
    const bool bad = status[0] != 0 || status[1] == 0;
    double N = 0.0;
    for (int gg = 0; gg < ngroups; ++gg) N += npart[(int64_t)gg * kp + slot];
    const int tile = slot >> 4, dph = dp >> 1;
    for (int dd = threadIdx.x; dd < d; dd += blockDim.x) {
        double s1 = 0.0, s2 = 0.0;
        for (int gg = 0; gg < ngroups; ++gg) {
            const double* p = part + ((int64_t)gg * kp + slot) * 2 * dp;
            s1 += p[dd];
            s2 += p[dp + dd];
        }
        const int64_t e = (int64_t)comp * d + dd;
        if (bad) {
            mu[e] = NAN;
            var[e] = NAN;
        } else if (N > 0.0) {
            const double sh = (double)tshift[(int64_t)tile * dp + (dd & 1) * dph + (dd >> 1)];
            const double m1 = s1 / N;
            const double v = s2 / N - m1 * m1;
            mu[e] = (float)(sh + m1);
            var[e] = (float)(v > (double)var_floor ? v : (double)var_floor);
        }
    }
    if (threadIdx.x == 0) w[comp] = bad ? NAN : (N > 0.0 ? (float)(N / (double)n) : 0.0f);
}

// Fixed-order fp64 sum of the per-block log-likelihood partials.
__global__ void k_ll_final(const double* __restrict__ llpart, int nparts, double* __restrict__ out,
                           const int* __restrict__ status) {
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
    if (threadIdx.x == 0) *out = (status[0] != 0 || status[1] == 0) ? NAN : red[0];
}

__global__ void k_identity_perm(int* perm, int kp, int k) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < kp) perm[i] = i < k ? i : -1;
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI in gmm_api.hip).
// ---------------------------------------------------------------------------
template <int DP, typename XT, int TM>
static hipError_t launch_lse_tm(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                float* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                                hipStream_t st) {
    const int64_t blocks = (n + 127) / 128;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_lse<DP, XT, TM>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.Pg, pl.cvec, pl.tshift, pl.ntiles, lse_out,
                       pl.llpart, ll_acc, pl.status, m, pl.perm, idx, resp);
    return hipGetLastError();
}

template <int DP, typename XT>
static hipError_t launch_lse_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                               float* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                               hipStream_t st) {
    if (m <= 0) return launch_lse_tm<DP, XT, 0>(pl, x, n, ldx, lse_out, ll_acc, 0, idx, resp, st);
    if (m <= 2) return launch_lse_tm<DP, XT, 2>(pl, x, n, ldx, lse_out, ll_acc, m, idx, resp, st);
    return launch_lse_tm<DP, XT, 4>(pl, x, n, ldx, lse_out, ll_acc, m, idx, resp, st);
}

template <int DP, typename XT>
static hipError_t launch_stats_t(const Plan& pl, const void* x, int64_t n, int64_t ldx,
                                 const float* lse, int acc, hipStream_t st) {
    const int64_t rpg = ((n + pl.ngroups - 1) / pl.ngroups + 63) / 64 * 64;
    hipLaunchKernelGGL((k_stats<DP, XT>), dim3(pl.ngroups * (pl.ntiles / 4)), dim3(256), 0, st,
                       (const XT*)x, n, pl.d, ldx, pl.Pg, pl.cvec, pl.tshift, pl.ntiles, lse,
                       rpg > 0 ? rpg : 64, pl.ngroups, pl.part, pl.npart, acc);
    return hipGetLastError();
}

#define GMM_DP_CASES(M) M(16) M(32) M(48) M(64) M(80) M(96) M(112) M(128)

hipError_t launch_lse(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                      float* lse_out, int ll_acc, int m, int32_t* idx, float* resp,
                      hipStream_t st) {
    switch (pl.dp) {
#define CASE(DPV)                                                                        \
    case DPV:                                                                            \
        return dtype == 0                                                                \
                   ? launch_lse_t<DPV, float>(pl, x, n, ldx, lse_out, ll_acc, m, idx, resp, st) \
                   : launch_lse_t<DPV, uint16_t>(pl, x, n, ldx, lse_out, ll_acc, m, idx, resp, st);
        GMM_DP_CASES(CASE)
#undef CASE
    }
    return hipErrorInvalidValue;
}

hipError_t launch_stats(const Plan& pl, const void* x, int64_t n, int64_t ldx, int dtype,
                        const float* lse, int acc, hipStream_t st) {
    switch (pl.dp) {
#define CASE(DPV)                                                                          \
    case DPV:                                                                              \
        return dtype == 0 ? launch_stats_t<DPV, float>(pl, x, n, ldx, lse, acc, st)       \
                          : launch_stats_t<DPV, uint16_t>(pl, x, n, ldx, lse, acc, st);
        GMM_DP_CASES(CASE)
#undef CASE
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prologue(const Plan& pl, const float* w, const float* mu, const float* var,
                           hipStream_t st) {
    hipLaunchKernelGGL(k_status_reset, dim3(1), dim3(64), 0, st, pl.status);
    const int64_t total = (int64_t)pl.k * pl.d;
    int vb = (int)((total + 255) / 256);
    if (vb > 1024) vb = 1024;
    hipLaunchKernelGGL(k_validate, dim3(vb), dim3(256), 0, st, w, mu, var, pl.k, pl.d, pl.status);
    hipLaunchKernelGGL(k_identity_perm, dim3((pl.kp + 255) / 256), dim3(256), 0, st, pl.perm,
                       pl.kp, pl.k);
    hipLaunchKernelGGL(k_shift, dim3((pl.dp + 63) / 64), dim3(64), 0, st, mu, pl.k, pl.d, pl.dp,
                       pl.ntiles, pl.tshift);
    hipLaunchKernelGGL(k_params, dim3(pl.kp), dim3(128), 0, st, w, mu, var, pl.perm, pl.k, pl.d,
                       pl.dp, pl.tshift, pl.Pg, pl.cvec);
    return hipGetLastError();
}

hipError_t launch_finalize(const Plan& pl, int64_t n, float var_floor, float* w, float* mu,
                           float* var, hipStream_t st) {
    hipLaunchKernelGGL(k_finalize, dim3(pl.kp), dim3(128), 0, st, pl.part, pl.npart, pl.ngroups,
                       pl.kp, pl.dp, pl.d, pl.perm, pl.tshift, n, var_floor, w, mu, var,
                       pl.status);
    return hipGetLastError();
}

hipError_t launch_ll_final(const Plan& pl, int nparts, double* out, hipStream_t st) {
    hipLaunchKernelGGL(k_ll_final, dim3(1), dim3(256), 0, st, pl.llpart, nparts, out, pl.status);
    return hipGetLastError();
}

}  // namespace gmm
