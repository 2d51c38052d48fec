// kvq_device.hpp -- device helpers shared by the libkvq HIP kernels (gfx950,
// wave64).  Only exact operations live here: fp16 <-> fp32 conversions, the
// fixed fp64 summation tree, and the bound / fallback arithmetic.
//
// Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1
// (INT8 keys / INT4 values with per-block error annotations) and Methodology 2
// (key and value terms evaluated online from scales and query norms).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.hpp"

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return __half2float(__ushort_as_half((unsigned short)bits16));
}

__device__ __forceinline__ uint32_t f2h_rn(float f) {
    return __half_as_ushort(__float2half_rn(f));
}

// Shuffle-xor of a double inside a wave (two 32-bit lane exchanges).
__device__ __forceinline__ double shfl_xor_d(double v, int mask) {
    return __shfl_xor(v, mask);
}

// Sum of 128 fp64 terms held as 8 contiguous terms per lane in 16 consecutive
// lanes (lane l of the group holds terms 8l .. 8l+7).  Fixed pairing: within
// the lane strides 1, 2, 4; across lanes xor 8, 4, 2, 1 (term strides 64, 32,
// 16, 8).  Every lane of the group returns the same value.  IEEE addition is
// commutative, so lane l and lane l^m form the same sum.
__device__ __forceinline__ double tree128(const double x[8]) {
    double a = x[0] + x[1], b = x[2] + x[3], c = x[4] + x[5], d = x[6] + x[7];
    double s = (a + b) + (c + d);
    s = s + shfl_xor_d(s, 8);
    s = s + shfl_xor_d(s, 4);
    s = s + shfl_xor_d(s, 2);
    s = s + shfl_xor_d(s, 1);
    return s;
}

// Exact square of an fp16-valued float in fp64 (22 significant bits).
__device__ __forceinline__ double sq64(float x) {
    double d = (double)x;
    return d * d;
}

// ||q||_2 of one 128-channel fp16 row spread over 16 lanes (8 per lane):
// f32(sqrt(T128(q_j^2))).
__device__ __forceinline__ float qnorm16(const uint4 raw) {
    uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    double sq[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sq[2 * i] = sq64(h2f(w[i] & 0xFFFFu));
        sq[2 * i + 1] = sq64(h2f(w[i] >> 16));
    }
    return (float)__dsqrt_rn(tree128(sq));
}

// Max of two non-negative-or-NaN floats that keeps NaN (as an unsigned
// compare of the bit patterns, NaN > +Inf > finite >= 0).
__device__ __forceinline__ float max_keep_nan(float a, float b) {
    uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    return ua > ub ? a : b;
}

// Key bound of one block: ((sm*qn)*k_err)*(1+2^-16), each product rounded to
// fp32 (explicit round-to-nearest multiplies: never contracted).
__device__ __forceinline__ float key_bound(float sm, float qn, float kerr) {
    float p = __fmul_rn(sm, qn);
    p = __fmul_rn(p, kerr);
    return __fmul_rn(p, 1.0f + 0x1p-16f);
}

// A block keeps its quantized tile only when its bound is finite and not
// above the tolerance.
__device__ __forceinline__ uint32_t falls_back(float bound, float tau) {
    return !(__builtin_isfinite(bound) && bound <= tau);
}

__device__ __forceinline__ uint32_t block_mask(float sm, float qn, float kerr, float verr,
                                               float tau_k, float tau_v) {
    return falls_back(key_bound(sm, qn, kerr), tau_k) | (falls_back(verr, tau_v) << 1);
}

}  // namespace kvq
