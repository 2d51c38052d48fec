// kvq_mfma.hpp -- matrix-core operand helpers shared by the decode and the
// scoring kernels (gfx950, wave64): v_mfma_f32_16x16x32_f16 and the exact
// widening of int8 key codes to fp16 k-slots.
//
// Operand layout of v_mfma_f32_16x16x32_f16: A lane l holds row l%16, k-slots
// [8*(l/16), +8); B lane l holds column l%16, the same k-slots; the result
// lane l holds column l%16, rows 4*(l/16) .. +3.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4_t mfma(uint4 a, uint4 b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_f16: A lane l holds row l%16, k-slots [4*(l/16), +4);
// B lane l holds column l%16, the same k-slots; the result as above.
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4_t mfma16(uint2 a, uint2 b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b), c,
                                                 0, 0, 0);
}

// 4 int8 codes -> 2 x fp16 pairs (exact): offset code u = c + 128 under the
// fp16 exponent of 1024 reads as 1024 + u; minus 1152 leaves c.
__device__ __forceinline__ uint2 i8x4_to_h4(uint32_t x) {
    const uint32_t u = x ^ 0x80808080u;
    const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const half2_t lo = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
    const half2_t hi = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// 8 int8 codes (two dwords) -> the 8 fp16 k-slots of one A operand.
__device__ __forceinline__ uint4 i8x8_to_h8(uint32_t x0, uint32_t x1) {
    const uint2 a = i8x4_to_h4(x0), b = i8x4_to_h4(x1);
    return make_uint4(a.x, a.y, b.x, b.y);
}


// Hadamard-rotated query for KVQ_CODEC_ROTATE_K caches, in the B-operand
// layout: lane (n, g) holds q[n][32g + 8s .. +8] in qb[s], s = 0..3.  Returns
// H q / 8 (H the +-1 Sylvester matrix of order 128) as two fp16 parts per
// channel, hi = f16(x) and lo = f16(x - hi), so that two matrix-core products
// reproduce the rotated query to about 2^-22: butterflies at channel
// strides 1 .. 16 inside the lane and 32, 64 across lanes xor 16, 32, in
// fp32.  All 64 lanes take part.
__device__ __forceinline__ void rotate_q(const uint4 (&qb)[4], int lane, uint4 (&hi)[4], uint4 (&lo)[4]) {
    float v[32];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t w[4] = {qb[s].x, qb[s].y, qb[s].z, qb[s].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * s + 2 * i] = h2f(w[i] & 0xFFFFu);
            v[8 * s + 2 * i + 1] = h2f(w[i] >> 16);
        }
    }
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
        for (int j = 0; j < 32; ++j)
            if (!(j & h)) {
                const float x = v[j], y = v[j + h];
                v[j] = x + y;
                v[j + h] = x - y;
            }
    // partners across lanes xor 16 and xor 32 by the row-swap permutes (VALU,
    // no LDS round trip): with both operands the value, the first result
    // holds the partner's value in odd rows (upper half) and the second in
    // even rows (lower half)
    const bool up16 = (lane & 16) != 0, up32 = (lane & 32) != 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[j]), false, false);
        const float o = __uint_as_float(up16 ? r[0] : r[1]);
        v[j] = up16 ? o - v[j] : v[j] + o;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[j]), false, false);
        const float o = __uint_as_float(up32 ? r[0] : r[1]);
        v[j] = up32 ? o - v[j] : v[j] + o;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = v[8 * s + 2 * i] * 0.125f, b = v[8 * s + 2 * i + 1] * 0.125f;
            const uint32_t ha = f2h_rn(a), hb = f2h_rn(b);
            wh[i] = ha | (hb << 16);
            wl[i] = f2h_rn(a - h2f(ha)) | (f2h_rn(b - h2f(hb)) << 16);
        }
        hi[s] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        lo[s] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    }
}

}  // namespace kvq
