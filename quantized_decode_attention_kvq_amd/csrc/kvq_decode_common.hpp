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

constexpr int FOLD_REG = 8;  // split counts the split merge handles in registers

// Device-coherent (agent-scope) stores and loads: values written by one
// workgroup and read by another of the same launch, which may run on another
// XCD with its own L2.
__device__ __forceinline__ void st_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// are in log2 units (scores scaled by sm * log2(e)).  wm/wl: [NWT][16]
// per-wave running max/sum, wacc: [NWT][gp][128] per-wave accumulators, all in
// LDS and complete (a barrier has been passed) on entry.  Each thread reads
// its NWT values of each array before any arithmetic (one LDS round trip),
// then combines them in wave order.
template <int NWT>
__device__ __forceinline__ void write_partial(const DecodeArgs &a, int64_t bh, int split, int gp,
                                              const float (*wm)[16], const float (*wl)[16],
                                              const float *wacc) {
    const int g = a.g;
    for (int idx = threadIdx.x; idx < g * D; idx += blockDim.x) {
        const int h = idx / D, j = idx % D;
        float mw[NWT], lw[NWT], aw[NWT];
#pragma unroll
        for (int w = 0; w < NWT; ++w) {
            mw[w] = wm[w][h];
            lw[w] = wl[w][h];
            aw[w] = wacc[(w * gp + h) * D + j];
        }
        float M = -__builtin_huge_valf();
#pragma unroll
        for (int w = 0; w < NWT; ++w) M = fmaxf(M, mw[w]);
        float L = 0.0f, A = 0.0f;
        if (M != -__builtin_huge_valf()) {
#pragma unroll
            for (int w = 0; w < NWT; ++w) {
                if (mw[w] == -__builtin_huge_valf()) continue;
                const float f = __builtin_amdgcn_exp2f(mw[w] - M);
                L += lw[w] * f;
                A += aw[w] * f;
            }
        }
        const int64_t p = (bh * a.splits + split) * g + h;
        if (a.arrive) {
            // read back in this launch by another workgroup, maybe on another
            // XCD: device-coherent stores
            st_agent(a.part_acc + p * D + j, A);
            if (j == 0) {
                st_agent(reinterpret_cast<float *>(a.part_ml + p), M);
                st_agent(reinterpret_cast<float *>(a.part_ml + p) + 1, L);
            }
        } else {
            a.part_acc[p * D + j] = A;
            if (j == 0) a.part_ml[p] = make_float2(M, L);
        }
    }
}

// The split merge in the decode launch itself: once this workgroup's partial
// stores have completed (device-coherent), it counts itself in; the last of
// the group's a.splits workgroups to arrive loads every partial of the group
// (device-coherent loads) and writes the fp16 output rows of its G heads,
// with the arithmetic of the separate merge kernel:
//   M = max_s m_s, L = sum_s l_s 2^(m_s - M), out = sum_s acc_s 2^(m_s - M) / L
// (0 when no split saw a token).  It then leaves the counter at zero.  lds:
// at least 8 * G * splits + 128 bytes of LDS free for the merge.  Called by
// every thread of the workgroup.
__device__ __forceinline__ void fold_merge(const DecodeArgs &a, int64_t bh, int64_t b, int64_t kvh, uint8_t *lds) {
    __shared__ int last_lds;
    constexpr float NEG_INF = -__builtin_huge_valf();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.arrive + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_lds = prev == (uint32_t)(a.splits - 1);
    }
    __syncthreads();
    if (!last_lds) return;
    const int g = a.g, S = a.splits, nt = blockDim.x;
    const float2 *pml = a.part_ml + bh * S * g;                  // split s, head h at [s * g + h]
    const float *pacc = a.part_acc + bh * S * g * D;             // split s, head h, channel j at [(s g + h) D + j]
    if (S <= FOLD_REG) {
        // up to FOLD_REG splits: each thread loads its head's (m, l) of every
        // split and its channel's accumulators at once (one round of
        // device-coherent loads), then merges in split order
        for (int i = threadIdx.x; i < g * D; i += nt) {
            const int h = i / D, j = i % D;
            float ms[FOLD_REG], ls[FOLD_REG], as[FOLD_REG];
#pragma unroll
            for (int s_ = 0; s_ < FOLD_REG; ++s_) {
                if (s_ < S) {
                    const float *e = reinterpret_cast<const float *>(pml + s_ * g + h);
                    ms[s_] = ld_agent(e);
                    ls[s_] = ld_agent(e + 1);
                    as[s_] = ld_agent(pacc + ((int64_t)s_ * g + h) * D + j);
                }
            }
            float M = NEG_INF;
#pragma unroll
            for (int s_ = 0; s_ < FOLD_REG; ++s_)
                if (s_ < S) M = fmaxf(M, ms[s_]);
            float L = 0.0f;
            if (M != NEG_INF) {
#pragma unroll
                for (int s_ = 0; s_ < FOLD_REG; ++s_)
                    if (s_ < S && ms[s_] != NEG_INF) L += ls[s_] * __builtin_amdgcn_exp2f(ms[s_] - M);
            }
            float o = 0.0f;
#pragma unroll
            for (int s_ = 0; s_ < FOLD_REG; ++s_) {
                if (s_ < S) {
                    const float w = (L > 0.0f && ms[s_] != NEG_INF) ? __builtin_amdgcn_exp2f(ms[s_] - M) / L : 0.0f;
                    o += w * as[s_];
                }
            }
            a.out[(b * a.hq + kvh * g + h) * D + j] = (uint16_t)f2h_rn(o);
        }
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(a.arrive + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    float2 *wml = reinterpret_cast<float2 *>(lds);               // [G][S] (m, l) of every split
    float2 *hml = reinterpret_cast<float2 *>(lds) + g * S;       // [G] (M, L)
    for (int i = threadIdx.x; i < g * S; i += nt) {
        const int h = i / S, s_ = i % S;
        const float *e = reinterpret_cast<const float *>(pml + s_ * g + h);
        wml[i] = make_float2(ld_agent(e), ld_agent(e + 1));
    }
    __syncthreads();
    for (int h = threadIdx.x; h < g; h += nt) {
        float M = NEG_INF;
        for (int s_ = 0; s_ < S; ++s_) M = fmaxf(M, wml[h * S + s_].x);
        float L = 0.0f;
        if (M != NEG_INF)
            for (int s_ = 0; s_ < S; ++s_)
                if (wml[h * S + s_].x != NEG_INF) L += wml[h * S + s_].y * __builtin_amdgcn_exp2f(wml[h * S + s_].x - M);
        hml[h] = make_float2(M, L);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < g * D; i += nt) {
        const int h = i / D, j = i % D;
        const float M = hml[h].x, L = hml[h].y;
        float o = 0.0f;
        for (int s_ = 0; s_ < S; ++s_) {
            const float m_s = wml[h * S + s_].x;
            const float w = (L > 0.0f && m_s != NEG_INF) ? __builtin_amdgcn_exp2f(m_s - M) / L : 0.0f;
            o += w * ld_agent(pacc + ((int64_t)s_ * g + h) * D + j);
        }
        a.out[(b * a.hq + kvh * g + h) * D + j] = (uint16_t)f2h_rn(o);
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.arrive + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kvq
