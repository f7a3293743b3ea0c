// gmm_ivf.hip - inverted lists of an IVF coarse quantizer from top-m soft
// assignments (gmm_ivf_build, declared in include/gmm_em.h).
//
// The Flash-GMM pages use GMM responsibilities to store border vectors in
// several IVF lists ("Flash-GMM: A Memory-Efficient Kernel for Scalable Soft
// Clustering", abstract; the review page, section 1, defines the IVF index).
// Entry e = n*m + j of the top-m arrays goes to list idx[e] when j == 0 or
// resp[e] >= min_resp; each list holds its rows in increasing order.
//
// A stable counting sort over the entries in row order, in fixed tiles of T
// entries (integer work, the same result on every run):
//   1. k_ivf_hist:    per tile, the count of kept entries of every list
//                     (LDS counters), written as one row of a tiles x K matrix;
//   2. k_ivf_colscan: per list, the exclusive prefix of its counts over the
//                     tiles (in place) and its total;
//   3. k_ivf_offsets: exclusive prefix of the totals -> list offsets;
//   4. k_ivf_scatter: per tile, one wave walks its entries in order, 64 at a
//                     time; each lane finds the lanes holding its list id
//                     with one ballot per id bit and is ranked among them by
//                     lane order, so each row lands at
//                     offset[list] + (kept entries of that list before it).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gmm_em.h"

namespace gmm {

constexpr int IVF_MAX_K = 16384;  // LDS counters per workgroup (at most 64 KB)
constexpr int64_t IVF_MIN_TILE = 4096;
constexpr int64_t IVF_MAX_MATRIX = int64_t(1) << 24;  // tiles x K counters

struct IvfPlan {
    int64_t entries = 0, tile = 0, ntiles = 0;
    size_t bytes = 0;
    size_t o_count = 0, o_mat = 0;
};

static size_t ivf_align(size_t v) { return (v + 255) & ~(size_t)255; }

static bool ivf_plan(int64_t n, int32_t m, int32_t k, IvfPlan* p) {
    if (n < 0 || m < 1 || k < 1 || k > IVF_MAX_K) return false;
    if (n > 0 && (int64_t)m > (int64_t(0x7fffffff) - 1) / n) return false;  // 32-bit positions
    IvfPlan q;
    q.entries = n * m;
    q.tile = IVF_MIN_TILE;
    for (;;) {
        q.ntiles = (q.entries + q.tile - 1) / q.tile;
        if (q.ntiles * k <= IVF_MAX_MATRIX) break;
        q.tile *= 2;
    }
    q.o_count = 0;
    q.o_mat = ivf_align((size_t)k * sizeof(int32_t));
    q.bytes = ivf_align(q.o_mat + (size_t)(q.ntiles > 0 ? q.ntiles : 1) * k * sizeof(int32_t));
    *p = q;
    return true;
}

__device__ __forceinline__ bool ivf_keep(const int32_t* idx, const float* resp, int64_t e,
                                         int m, int k, float min_resp, int32_t* key) {
    const int32_t c = idx[e];
    *key = c;
    if (c < 0 || c >= k) return false;
    if (e % m == 0) return true;
    return resp ? resp[e] >= min_resp : true;
}

__global__ __launch_bounds__(256) void k_ivf_hist(const int32_t* __restrict__ idx,
                                                  const float* __restrict__ resp, int64_t entries,
                                                  int m, int k, float min_resp, int64_t tile,
                                                  int32_t* __restrict__ mat) {
    extern __shared__ int32_t h[];  // k counters
    for (int c = threadIdx.x; c < k; c += blockDim.x) h[c] = 0;
    __syncthreads();
    const int64_t e0 = (int64_t)blockIdx.x * tile;
    const int64_t e1 = e0 + tile < entries ? e0 + tile : entries;
    for (int64_t e = e0 + threadIdx.x; e < e1; e += blockDim.x) {
        int32_t c;
        if (ivf_keep(idx, resp, e, m, k, min_resp, &c)) atomicAdd(&h[c], 1);
    }
    __syncthreads();
    int32_t* row = mat + (int64_t)blockIdx.x * k;
    for (int c = threadIdx.x; c < k; c += blockDim.x) row[c] = h[c];
}

// 64 lists per block, their tiles split into 16 segments (one wave each):
// each wave sums its segment, then rewrites it as exclusive prefixes from
// the sum of the segments before it.
constexpr int IVF_SEGS = 16;
__global__ __launch_bounds__(64 * IVF_SEGS) void k_ivf_colscan(int32_t* __restrict__ mat,
                                                              int64_t ntiles, int k,
                                                              int32_t* __restrict__ count) {
    __shared__ int32_t seg[IVF_SEGS][64];
    const int col = threadIdx.x & 63, sg = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + col;
    const int64_t per = (ntiles + IVF_SEGS - 1) / IVF_SEGS;
    const int64_t t0 = (int64_t)sg * per < ntiles ? (int64_t)sg * per : ntiles;
    const int64_t t1 = t0 + per < ntiles ? t0 + per : ntiles;
    int32_t sum = 0;
    if (c < k) {
        int64_t t = t0;
        // eight tiles' counts in flight at a time
        for (; t + 8 <= t1; t += 8) {
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = mat[(t + u) * k + c];
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        for (; t < t1; ++t) sum += mat[t * k + c];
    }
    seg[sg][col] = sum;
    __syncthreads();
    if (c >= k) return;
    int32_t run = 0;
    for (int q = 0; q < sg; ++q) run += seg[q][col];
    int64_t t = t0;
    for (; t + 8 <= t1; t += 8) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = mat[(t + u) * k + c];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            mat[(t + u) * k + c] = run;
            run += v[u];
        }
    }
    for (; t < t1; ++t) {
        const int32_t v = mat[t * k + c];
        mat[t * k + c] = run;
        run += v;
    }
    if (sg == IVF_SEGS - 1) count[c] = run;
}

__global__ __launch_bounds__(1024) void k_ivf_offsets(const int32_t* __restrict__ count, int k,
                                                      int64_t* __restrict__ offsets) {
    __shared__ int64_t part[1024];
    const int per = (k + 1023) / 1024;
    const int lo = threadIdx.x * per;
    const int hi = lo + per < k ? lo + per : k;
    int64_t s = 0;
    for (int c = lo; c < hi; ++c) s += count[c];
    part[threadIdx.x] = s;
    __syncthreads();
    // inclusive Hillis-Steele scan over the 1024 partial sums
    for (int off = 1; off < 1024; off <<= 1) {
        const int64_t v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
        __syncthreads();
        part[threadIdx.x] += v;
        __syncthreads();
    }
    int64_t run = threadIdx.x > 0 ? part[threadIdx.x - 1] : 0;
    for (int c = lo; c < hi; ++c) {
        offsets[c] = run;
        run += count[c];
    }
    if (threadIdx.x == 1023) offsets[k] = part[1023];
}

// One wave per tile; base[c] = kept entries of list c in earlier tiles, then
// advanced as this tile's entries are placed.
__global__ __launch_bounds__(64) void k_ivf_scatter(const int32_t* __restrict__ idx,
                                                    const float* __restrict__ resp,
                                                    int64_t entries, int m, int k, float min_resp,
                                                    int64_t tile, const int32_t* __restrict__ mat,
                                                    const int64_t* __restrict__ offsets,
                                                    int32_t* __restrict__ rows_out,
                                                    float* __restrict__ vals_out) {
    extern __shared__ int32_t base[];  // k counters
    const int lane = threadIdx.x;
    const int32_t* row = mat + (int64_t)blockIdx.x * k;
    for (int c = lane; c < k; c += 64) base[c] = row[c];
    __syncthreads();
    const uint64_t below = (uint64_t(1) << lane) - 1;  // lanes before this one
    const int nbits = k > 1 ? 32 - __builtin_clz((unsigned)(k - 1)) : 0;  // bits of a list id
    const int64_t e0 = (int64_t)blockIdx.x * tile;
    const int64_t e1 = e0 + tile < entries ? e0 + tile : entries;
    constexpr int U = 4;  // 64-entry chunks whose ids and values are loaded at once
    for (int64_t eb = e0; eb < e1; eb += 64 * U) {
        int32_t cu[U];
        float ru[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = eb + 64 * u + lane;
            cu[u] = e < e1 ? idx[e] : -1;
            ru[u] = (resp && e < e1) ? resp[e] : 1.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = eb + 64 * u + lane;
            const int32_t c = cu[u];
            // the rule of ivf_keep: a valid list id, and the row's first
            // entry or a responsibility at or above the threshold
            const bool keep = e < e1 && c >= 0 && c < k &&
                              (e % m == 0 || !resp || ru[u] >= min_resp);
            // the kept lanes whose list id equals this lane's, one id bit at
            // a time (meaningful for kept lanes only)
            uint64_t same = __builtin_amdgcn_ballot_w64(keep);
            for (int bit = 0; bit < nbits; ++bit) {
                const bool set = ((c >> bit) & 1) != 0;
                const uint64_t v = __builtin_amdgcn_ballot_w64(keep && set);
                same &= set ? v : ~v;
            }
            if (keep) {
                const int32_t b = base[c];
                const int64_t pos = offsets[c] + b + __popcll(same & below);
                rows_out[pos] = (int32_t)(e / m);
                if (vals_out) vals_out[pos] = ru[u];
                // the first lane of each id advances its counter (one wave:
                // its LDS accesses complete in program order, so every
                // lane's read of base[c] above precedes this update)
                if ((same & below) == 0) base[c] = b + __popcll(same);
            }
        }
    }
}

}  // namespace gmm

using namespace gmm;

extern "C" {

size_t gmm_ivf_workspace_bytes(int64_t n, int32_t m, int32_t k) {
    IvfPlan p;
    return ivf_plan(n, m, k, &p) ? p.bytes : 0;
}

int gmm_ivf_build(const int32_t* idx_dev, const float* resp_dev, int64_t n, int32_t m, int32_t k,
                  float min_resp, int64_t* offsets_dev, int32_t* rows_dev, float* values_dev,
                  void* workspace, size_t workspace_bytes, void* stream) {
    IvfPlan p;
    if (!ivf_plan(n, m, k, &p)) return (n < 0 || m < 1 || k < 1) ? GMM_E_INVALID : GMM_E_UNSUPPORTED;
    if (!offsets_dev) return GMM_E_INVALID;
    if (n > 0 && (!idx_dev || !rows_dev)) return GMM_E_INVALID;
    if (min_resp != min_resp) return GMM_E_INVALID;  // NaN threshold
    if (!workspace || workspace_bytes < p.bytes || (uintptr_t)workspace % 256 != 0)
        return GMM_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    int32_t* count = (int32_t*)((char*)workspace + p.o_count);
    int32_t* mat = (int32_t*)((char*)workspace + p.o_mat);
    const size_t lds = (size_t)k * sizeof(int32_t);  // at most 64 KB
    if (p.ntiles > 0) {
        hipLaunchKernelGGL(k_ivf_hist, dim3((unsigned)p.ntiles), dim3(256), lds, st, idx_dev,
                           resp_dev, p.entries, m, k, min_resp, p.tile, mat);
    }
    hipLaunchKernelGGL(k_ivf_colscan, dim3((k + 63) / 64), dim3(64 * IVF_SEGS), 0, st, mat,
                       p.ntiles, k, count);
    hipLaunchKernelGGL(k_ivf_offsets, dim3(1), dim3(1024), 0, st, count, k, offsets_dev);
    if (p.ntiles > 0) {
        hipLaunchKernelGGL(k_ivf_scatter, dim3((unsigned)p.ntiles), dim3(64), lds, st, idx_dev,
                           resp_dev, p.entries, m, k, min_resp, p.tile, mat, offsets_dev, rows_dev,
                           values_dev);
    }
    return hipGetLastError() == hipSuccess ? GMM_OK : GMM_E_HIP;
}

}  // extern "C"
