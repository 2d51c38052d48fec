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


}  // namespace kvq
