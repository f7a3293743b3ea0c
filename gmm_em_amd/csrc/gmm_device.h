// gmm_device.h - device helpers shared by the kernels of the EM step: MFMA
// wrapper, buffer-resource loads, online logsumexp, ordered top-m lists.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace gmm {

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_x(const float* p) { return *p; }
__device__ __forceinline__ float load_x(const uint16_t* p) {
    return __uint_as_float(((uint32_t)(*p)) << 16);
}

// Buffer-resource loads (the buffer unit returns 0 for an offset past the
// resource's range instead of accessing memory). Word 3 of the resource:
// raw (untyped) buffer, 32-bit data format field, as used by the CDNA
// compute libraries.
constexpr int BUF_RSRC_WORD3 = 0x00020000;
template <typename XT>
__device__ __forceinline__ float buf_load_x(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ float buf_load_x<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
template <>
__device__ __forceinline__ float buf_load_x<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0)) << 16);
}
__device__ __forceinline__ double buf_load_f64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + 4), 0, 0);
    return __hiloint2double((int)hi, (int)lo);
}

__device__ __forceinline__ f64x4 mfma4d(double a, double b, f64x4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// E-step operand: a = x - s (exact in fp64 for fp32 x), then a or a^2.
__device__ __forceinline__ double feat(float x, double s, bool sq) {
    const double a = (double)x - s;
    return sq ? a * a : a;
}

// Online logsumexp with the running maximum in fp64 and the scaled sum in
// fp32 (every exponent argument is <= 0). One of the two rescaling factors
// is always exp(0) = 1, so a push takes a single exponential: with
// t = v - m, s <- s * exp(-t) + 1 and m <- v when t > 0, else s <- s + exp(t).
__device__ __forceinline__ void lse_push(double& m, float& s, double v) {
    const float t = (float)(v - m);
    const float e = __expf(-fabsf(t));
    const bool up = t > 0.0f;
    s = up ? fmaf(s, e, 1.0f) : s + e;
    m = up ? v : m;
}
__device__ __forceinline__ void lse_merge(double& m, float& s, double m2, float s2) {
    const double mn = fmax(m, m2);
    s = s * __expf((float)(m - mn)) + s2 * __expf((float)(m2 - mn));
    m = mn;
}

// exp(t) for t <= 0 with fp32-level relative accuracy over the whole fp64
// range: exp(t) = 2^j * 2^f with j = rint(t log2 e) and |f| <= 1/2, the
// fraction through the hardware base-2 exponential (fp32) and the power of two
// through ldexp (fp64, gradual underflow, exactly 0 below 2^-1075). A
// responsibility therefore vanishes where exp underflows in fp64, not where it
// underflows in fp32 (about exp(-104)). t = -inf (padding) gives 0.
__device__ __forceinline__ double exp_f64range(double t) {
    const double y = fmax(t, -1100.0) * 1.4426950408889634074;
    const double j = rint(y);
    const float f = (float)(y - j);
    return ldexp((double)__builtin_amdgcn_exp2f(f), (int)j);
}

__device__ __forceinline__ double shfl_xor_d(double v, int off) {
    return __shfl_xor(v, off);
}

// Ordered insertion of (v, i) into a list sorted by larger value first, then
// smaller index (empty entries hold -inf and the largest index).
template <int TM>
__device__ __forceinline__ void top_push(double (&tv)[TM], int (&ti)[TM], double v, int i) {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const bool gt = v > tv[j] || (v == tv[j] && i < ti[j]);
        const double ov = tv[j];
        const int oi = ti[j];
        tv[j] = gt ? v : ov;
        ti[j] = gt ? i : oi;
        v = gt ? ov : v;
        i = gt ? oi : i;
    }
}

// The same insertion when i is larger than the index of every entry already
// in the list (a lane that pushes its components in increasing order): an
// equal value then never displaces an entry, and an empty entry (index
// 0x7fffffff) always takes the value, so no index comparison is needed.
template <int TM>
__device__ __forceinline__ void top_push_inc(double (&tv)[TM], int (&ti)[TM], double v, int i) {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const bool gt = v > tv[j] || ti[j] == 0x7fffffff;
        const double ov = tv[j];
        const int oi = ti[j];
        tv[j] = gt ? v : ov;
        ti[j] = gt ? i : oi;
        v = gt ? ov : v;
        i = gt ? oi : i;
    }
}

// Merge with the list of lane (lane ^ off): both lanes end with the same top
// TM of the union.
template <int TM>
__device__ __forceinline__ void top_merge(double (&tv)[TM], int (&ti)[TM], int off) {
    double ov[TM];
    int oi[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        ov[j] = shfl_xor_d(tv[j], off);
        oi[j] = __shfl_xor(ti[j], off);
    }
    double rv[TM];
    int ri[TM];
    int a = 0, b = 0;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        double va = tv[0], vb = ov[0];
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

}  // namespace gmm
