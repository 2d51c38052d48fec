// kvq_decode_common.hpp -- pieces shared by the decode kernels: workgroup
// setup (query rows, query norms, per-block fallback masks) and the
// cross-wave / cross-split log-sum-exp merge.
//
// "Runtime-Certified Bounded-Error Quantized Attention", Methodology 2: both
// bounds are evaluated online from quantities already at hand (block error
// statistics and query norms) without touching the FP16 originals; the masks
// are decided per (batch, KV head, block) before any tile is fetched.
#pragma once

#include "kvq_device.hpp"
#include "kvq_internal.hpp"

namespace kvq {

// Loads the G query rows of (b, kvh) into q_lds (fp16 bits, [16][128], rows
// >= G zeroed) and returns the group query norm (max over the G heads).  Must
// be called by all threads of the workgroup (at least 256); 16-lane group h
// handles head h.  qn_lds: 16 floats.
__device__ __forceinline__ float load_q_and_norm(const uint16_t *__restrict__ q, int64_t qrow0,
                                                 int g, uint16_t (*q_lds)[D], float *qn_lds) {
    const int tid = threadIdx.x;
    const int h = tid >> 4, lane16 = tid & 15;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (h < g) raw = *reinterpret_cast<const uint4 *>(q + (qrow0 + h) * D + 8 * lane16);
    if (h < 16) *reinterpret_cast<uint4 *>(&q_lds[h][8 * lane16]) = raw;
    const float n = qnorm16(raw);  // all 16 lanes of the group participate
    if (lane16 == 0 && h < 16) qn_lds[h] = n;
    __syncthreads();
    float qn = 0.0f;
    for (int i = 0; i < g; ++i) qn = max_keep_nan(qn, qn_lds[i]);
    return qn;
}

// Fallback masks of blocks [blk0, blk1) of one (b, kvh) into mask_lds, and
// into mask_out when given.  Followed by a workgroup barrier.
__device__ __forceinline__ void compute_masks(const DecodeArgs &a, int64_t bh, int64_t blk0,
                                              int64_t blk1, float qn, uint8_t *mask_lds) {
    for (int64_t i = threadIdx.x; i < blk1 - blk0; i += blockDim.x) {
        const int64_t blk = blk0 + i;
        const int64_t si = bh * a.nbc + blk;
        const uint32_t m = block_mask(a.sm, qn, a.c.k_err[si], a.c.v_err[si], a.tau_k, a.tau_v);
        mask_lds[i] = (uint8_t)m;
        if (a.mask_out) a.mask_out[bh * a.nb + blk] = (uint8_t)m;
    }
    __syncthreads();
}

// Online-softmax state of one head on one wave, and its merge with another.
struct Running {
    float m, l;
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Writes this workgroup's partial (running max, running sum, unnormalised
// accumulator) of split `split` for the G heads of (b, kvh).  Running maxima
// are in log2 units (scores scaled by sm * log2(e)).  wm/wl: [nw][16]
// per-wave running max/sum, wacc: [nw][gp][128] per-wave accumulators, all in
// LDS and complete (a barrier has been passed) on entry.
__device__ __forceinline__ void write_partial(const DecodeArgs &a, int64_t bh, int split, int nw,
                                              int gp, const float (*wm)[16], const float (*wl)[16],
                                              const float *wacc) {
    const int g = a.g;
    for (int idx = threadIdx.x; idx < g * D; idx += blockDim.x) {
        const int h = idx / D, j = idx % D;
        float M = -__builtin_huge_valf();
        for (int w = 0; w < nw; ++w) M = fmaxf(M, wm[w][h]);
        float L = 0.0f, A = 0.0f;
        if (M != -__builtin_huge_valf()) {
            for (int w = 0; w < nw; ++w) {
                if (wm[w][h] == -__builtin_huge_valf()) continue;
                const float f = __builtin_amdgcn_exp2f(wm[w][h] - M);
                L += wl[w][h] * f;
                A += wacc[(w * gp + h) * D + j] * f;
            }
        }
        const int64_t p = (bh * a.splits + split) * g + h;
        a.part_acc[p * D + j] = A;
        if (j == 0) a.part_ml[p] = make_float2(M, L);
    }
}

}  // namespace kvq
