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

// The value of lane l ^ M (M = 1, 2, 4 or 8) of the same 16-lane DPP row, on
// VALU lane moves (no LDS round trip): xor 1 and xor 2 are quad
// permutations, xor 8 the rotation of the row by 8; xor 4 is a shift left by
// 4 (lane l reads l + 4) written to the lanes with bit 2 clear (bank mask
// 0x5: lanes 0-3 and 8-11 of the row), then a shift right by 4 written to
// the others (0xA).  Every lane of the row must be active.
template <int M>
__device__ __forceinline__ int xor16(int v) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8, "lane xor inside a row of 16");
    if constexpr (M == 1) {
        return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (M == 8) {
        return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else {
        const int t = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0x5, false);  // row_shl:4
        return __builtin_amdgcn_update_dpp(t, v, 0x114, 0xF, 0xA, false);        // row_shr:4
    }
}
// m is a compile-time constant once the caller's loop is unrolled.
__device__ __forceinline__ uint32_t xor16u(uint32_t v, int m) {
    const int x = (int)v;
    return (uint32_t)(m == 1 ? xor16<1>(x) : m == 2 ? xor16<2>(x) : m == 4 ? xor16<4>(x) : xor16<8>(x));
}
__device__ __forceinline__ float xor16f(float v, int m) { return __uint_as_float(xor16u(__float_as_uint(v), m)); }
__device__ __forceinline__ double xor16d(double v, int m) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = xor16u((uint32_t)b, m), hi = xor16u((uint32_t)(b >> 32), m);
    return __longlong_as_double((long long)((hi << 32) | lo));
}

// Sum of 128 fp64 terms held as 8 contiguous terms per lane in the 16 lanes
// of a DPP row (lane l of the row holds terms 8l .. 8l+7).  Fixed pairing:
// within the lane strides 1, 2, 4; across lanes xor 8, 4, 2, 1 (term strides
// 64, 32, 16, 8).  Every lane of the row returns the same value.  IEEE
// addition is commutative, so lane l and lane l^m form the same sum.
__device__ __forceinline__ double tree128(const double x[8]) {
    double a = x[0] + x[1], b = x[2] + x[3], c = x[4] + x[5], d = x[6] + x[7];
    double s = (a + b) + (c + d);
    s = s + xor16d(s, 8);
    // lanes l and l^8 now agree, so the row rotation by 4 reads lane l^4's value
    {
        const uint64_t b = (uint64_t)__double_as_longlong(s);
        const uint64_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, 0x124, 0xF, 0xF, false);
        const uint64_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), 0x124, 0xF, 0xF, false);
        s = s + __longlong_as_double((long long)((hi << 32) | lo));
    }
    s = s + xor16d(s, 2);
    s = s + xor16d(s, 1);
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

// Wave-wide totals in every lane, on DPP moves (no LDS round trip): inclusive
// scans inside each 16-lane row (row shifts by 1, 2, 4, 8; lanes shifted in
// from outside the row read the identity), then the row totals carried up by
// the broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and
// 3); lane 63 ends with the total, read back as a wave-uniform value.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_from(int identity, int v) {
    return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ float wave_total_sum(float v) {
    constexpr int Z = 0;  // bits of 0.0f
    v += __int_as_float(dpp_from<0x111, 0xF>(Z, __float_as_int(v)));
    v += __int_as_float(dpp_from<0x112, 0xF>(Z, __float_as_int(v)));
    v += __int_as_float(dpp_from<0x114, 0xF>(Z, __float_as_int(v)));
    v += __int_as_float(dpp_from<0x118, 0xF>(Z, __float_as_int(v)));
    v += __int_as_float(dpp_from<0x142, 0xA>(Z, __float_as_int(v)));
    v += __int_as_float(dpp_from<0x143, 0xC>(Z, __float_as_int(v)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_total_max(float v) {
    constexpr int NI = (int)0xFF800000u;  // bits of -inf
    v = fmaxf(v, __int_as_float(dpp_from<0x111, 0xF>(NI, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_from<0x112, 0xF>(NI, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_from<0x114, 0xF>(NI, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_from<0x118, 0xF>(NI, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_from<0x142, 0xA>(NI, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_from<0x143, 0xC>(NI, __float_as_int(v))));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Inclusive prefix sum over the lanes (the same moves), per lane.
__device__ __forceinline__ int wave_incl_scan_int(int v) {
    v += dpp_from<0x111, 0xF>(0, v);
    v += dpp_from<0x112, 0xF>(0, v);
    v += dpp_from<0x114, 0xF>(0, v);
    v += dpp_from<0x118, 0xF>(0, v);
    v += dpp_from<0x142, 0xA>(0, v);
    v += dpp_from<0x143, 0xC>(0, v);
    return v;
}
// Inclusive running maximum over the lanes (the same moves), per lane.
__device__ __forceinline__ int wave_incl_scan_max_int(int v) {
    constexpr int LO = (int)0x80000000u;
    v = max(v, dpp_from<0x111, 0xF>(LO, v));
    v = max(v, dpp_from<0x112, 0xF>(LO, v));
    v = max(v, dpp_from<0x114, 0xF>(LO, v));
    v = max(v, dpp_from<0x118, 0xF>(LO, v));
    v = max(v, dpp_from<0x142, 0xA>(LO, v));
    v = max(v, dpp_from<0x143, 0xC>(LO, v));
    return v;
}
__device__ __forceinline__ int wave_total_sum_int(int v) {
    return __builtin_amdgcn_readlane(wave_incl_scan_int(v), 63);
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
