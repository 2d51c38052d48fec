// kvq_decode_valu.hip -- per-block bounds kernel and the VALU split-K decode
// kernel (gfx950, wave64), for GQA groups too narrow for a matrix-core
// contraction.
//
// "Runtime-Certified Bounded-Error Quantized Attention": Methodology 1 (INT8
// keys / INT4 values served from the compressed tier, FP16 originals on
// fallback), Methodology 2 (bounds evaluated online per block from the block
// statistics and the query norm), Key Contributions "Deterministic Recovery"
// (a block whose bound is not certified is read from the FP16 originals).
//
// Grid (splits, Hkv, B), 256 threads.  A workgroup owns a contiguous range of
// 64-token blocks of one (b, kvh); its four waves take every fourth block.
// Per block a wave maps lane t to token t for Q.K (int8 codes are widened to
// fp16 pairs with a byte permute and dotted against q with v_dot2_f32_f16),
// updates its online softmax (scores in log2 units, exp2), stages the
// weights p*s_v in LDS and then maps
// lane l to channels (2l, 2l+1) for P.V over the block's channel-major int4
// codes.  Waves and splits are merged by log-sum-exp; the last workgroup of a
// (b, kvh) to finish writes the fp16 output.
#include "kvq_decode_common.hpp"

namespace kvq {

// ------------------------------------------------------------ bounds kernel

__global__ __launch_bounds__(256) void bounds_kernel(BoundsArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[16][D];
    __shared__ float qn_lds[16];
    const int64_t b = blockIdx.y, kvh = blockIdx.x;
    const int64_t bh = b * a.hkv + kvh;
    const float qn = load_q_and_norm(a.q, b * a.hq + kvh * a.g, a.g, q_lds, qn_lds);
    for (int64_t blk = threadIdx.x; blk < a.nb; blk += blockDim.x) {
        const float ke = a.k_err[bh * a.nbc + blk], ve = a.v_err[bh * a.nbc + blk];
        const float kbv = key_bound(a.sm, qn, ke);
        const int64_t o = bh * a.nb + blk;
        if (a.kb) a.kb[o] = kbv;
        if (a.vb) a.vb[o] = ve;
        if (a.mask) a.mask[o] = (uint8_t)(falls_back(kbv, a.tau_k) | (falls_back(ve, a.tau_v) << 1));
    }
}

hipError_t launch_bounds(const BoundsArgs &a, int batch, hipStream_t s) {
    hipLaunchKernelGGL(bounds_kernel, dim3((unsigned)a.hkv, (unsigned)batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ------------------------------------------------------------ decode (VALU)

// Four int8 codes (one dword) -> two fp16 pairs holding the exact values.
// x ^ 0x80 gives the offset code u = c + 128 in [1, 255]; placed under the
// fp16 exponent of 1024 (byte 0x64 above it) it reads as 1024 + u, and
// subtracting 1152 leaves c exactly.
__device__ __forceinline__ void i8x4_to_h2x2(uint32_t x, half2_t &lo, half2_t &hi) {
    const uint32_t u = x ^ 0x80808080u;
    const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    lo = __builtin_bit_cast(half2_t, a) + bias;
    hi = __builtin_bit_cast(half2_t, b) + bias;
}

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Signed nibble k (0..7) of a dword, as float.
__device__ __forceinline__ float nib(uint32_t w, int k) {
    return (float)(int)__builtin_amdgcn_sbfe(w, 4 * k, 4);  // the builtin returns unsigned
}

template <int GP>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
    constexpr int NW = 4;
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[16][D];
    __shared__ float qn_lds[16];
    __shared__ uint8_t mask_lds[MAX_BPS];
    // per-wave softmax weights [wave][head][value group][token]; reused for the
    // wave merge afterwards
    __shared__ __attribute__((aligned(16))) float w_lds[NW][GP][4][BLK];
    __shared__ float wm[NW][16], wl[NW][16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept scalar
    const int split = blockIdx.x;
    const int64_t kvh = blockIdx.y, b = blockIdx.z;
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g;
    const int64_t blk0 = (int64_t)split * a.bps;
    const int64_t blk1 = blk0 + a.bps < a.nb ? blk0 + a.bps : a.nb;

    const float qn = load_q_and_norm(a.q, b * a.hq + kvh * g, g, q_lds, qn_lds);
    compute_masks(a, bh, blk0, blk1, qn, mask_lds);

    float m_run[GP], l_run[GP], acc[GP][2];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        m_run[h] = -__builtin_huge_valf();
        l_run[h] = 0.0f;
        acc[h][0] = acc[h][1] = 0.0f;
    }

    const int64_t row_base = bh * a.cap;
    const int vg = lane >> 4;  // value group of channels (2*lane, 2*lane+1)
    const float sml2 = a.sm * 1.4426950408889634f;  // scores in log2 units

    for (int64_t blk = blk0 + wave; blk < blk1; blk += NW) {
        const uint32_t mk = __builtin_amdgcn_readfirstlane(mask_lds[blk - blk0]);
        const int64_t t = blk * BLK + lane;
        const bool valid = t < a.length;

        // ---------------- scores s_h = sm * q_h . k~_t
        float sc[GP];
#pragma unroll
        for (int h = 0; h < GP; ++h) sc[h] = 0.0f;
        if (!(mk & 1u)) {
            const uint4 *kp = reinterpret_cast<const uint4 *>(a.c.k_codes + (row_base + t) * D);
            const float ks = h2f(a.c.k_scales[row_base + t]);
#pragma unroll 2
            for (int c = 0; c < 8; ++c) {  // 16 channels per chunk
                const uint4 kr = kp[c];
                half2_t kh[8];
                i8x4_to_h2x2(kr.x, kh[0], kh[1]);
                i8x4_to_h2x2(kr.y, kh[2], kh[3]);
                i8x4_to_h2x2(kr.z, kh[4], kh[5]);
                i8x4_to_h2x2(kr.w, kh[6], kh[7]);
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    const uint4 qa = *reinterpret_cast<const uint4 *>(&q_lds[h][16 * c]);
                    const uint4 qb = *reinterpret_cast<const uint4 *>(&q_lds[h][16 * c + 8]);
                    float s = sc[h];
                    s = dot2(kh[0], __builtin_bit_cast(half2_t, qa.x), s);
                    s = dot2(kh[1], __builtin_bit_cast(half2_t, qa.y), s);
                    s = dot2(kh[2], __builtin_bit_cast(half2_t, qa.z), s);
                    s = dot2(kh[3], __builtin_bit_cast(half2_t, qa.w), s);
                    s = dot2(kh[4], __builtin_bit_cast(half2_t, qb.x), s);
                    s = dot2(kh[5], __builtin_bit_cast(half2_t, qb.y), s);
                    s = dot2(kh[6], __builtin_bit_cast(half2_t, qb.z), s);
                    s = dot2(kh[7], __builtin_bit_cast(half2_t, qb.w), s);
                    sc[h] = s;
                }
            }
            const float f = ks * sml2;
#pragma unroll
            for (int h = 0; h < GP; ++h) sc[h] *= f;
        } else {
            const uint4 *kp = reinterpret_cast<const uint4 *>(a.c.k16 + (row_base + t) * D);
#pragma unroll 2
            for (int c = 0; c < 16; ++c) {  // 8 channels per chunk
                const uint4 kr = kp[c];
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    const uint4 qa = *reinterpret_cast<const uint4 *>(&q_lds[h][8 * c]);
                    float s = sc[h];
                    s = dot2(__builtin_bit_cast(half2_t, kr.x), __builtin_bit_cast(half2_t, qa.x), s);
                    s = dot2(__builtin_bit_cast(half2_t, kr.y), __builtin_bit_cast(half2_t, qa.y), s);
                    s = dot2(__builtin_bit_cast(half2_t, kr.z), __builtin_bit_cast(half2_t, qa.z), s);
                    s = dot2(__builtin_bit_cast(half2_t, kr.w), __builtin_bit_cast(half2_t, qa.w), s);
                    sc[h] = s;
                }
            }
#pragma unroll
            for (int h = 0; h < GP; ++h) sc[h] *= sml2;
        }

        // ---------------- online softmax over the block (per head)
        float vsc[4];
        if (!(mk & 2u)) {
            const uint2 sv = *reinterpret_cast<const uint2 *>(a.c.v_scales + (row_base + t) * 4);
            vsc[0] = h2f(sv.x & 0xFFFFu);
            vsc[1] = h2f(sv.x >> 16);
            vsc[2] = h2f(sv.y & 0xFFFFu);
            vsc[3] = h2f(sv.y >> 16);
        } else {
            vsc[0] = vsc[1] = vsc[2] = vsc[3] = 1.0f;
        }
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            if (h >= g) break;
            const float s = valid ? sc[h] : -__builtin_huge_valf();
            const float m_new = fmaxf(m_run[h], wave_max(s));
            float p = 0.0f, alpha = 1.0f;
            if (m_new != -__builtin_huge_valf()) {
                p = valid ? __builtin_amdgcn_exp2f(s - m_new) : 0.0f;
                alpha = (m_run[h] == -__builtin_huge_valf()) ? 0.0f : __builtin_amdgcn_exp2f(m_run[h] - m_new);
            }
            l_run[h] = l_run[h] * alpha + wave_sum(p);
            acc[h][0] *= alpha;
            acc[h][1] *= alpha;
            m_run[h] = m_new;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) w_lds[wave][h][gg][lane] = valid ? p * vsc[gg] : 0.0f;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---------------- P.V: lane owns channels 2*lane, 2*lane+1
        if (!(mk & 2u)) {
            const uint4 *vp = reinterpret_cast<const uint4 *>(
                a.c.v_codes + (bh * a.nbc + blk) * (D * BLK / 2) + (2 * lane) * (BLK / 2));
            const uint4 c0a = vp[0], c0b = vp[1], c1a = vp[2], c1b = vp[3];
            const uint32_t w0[8] = {c0a.x, c0a.y, c0a.z, c0a.w, c0b.x, c0b.y, c0b.z, c0b.w};
            const uint32_t w1[8] = {c1a.x, c1a.y, c1a.z, c1a.w, c1b.x, c1b.y, c1b.z, c1b.w};
#pragma unroll
            for (int t8 = 0; t8 < 8; ++t8) {  // 8 tokens per dword
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    float f0[4], f1[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        f0[u] = nib(w0[t8], 4 * half + u);
                        f1[u] = nib(w1[t8], 4 * half + u);
                    }
#pragma unroll
                    for (int h = 0; h < GP; ++h) {
                        if (h >= g) break;
                        const float4 wv = *reinterpret_cast<const float4 *>(&w_lds[wave][h][vg][8 * t8 + 4 * half]);
                        acc[h][0] += wv.x * f0[0] + wv.y * f0[1] + wv.z * f0[2] + wv.w * f0[3];
                        acc[h][1] += wv.x * f1[0] + wv.y * f1[1] + wv.z * f1[2] + wv.w * f1[3];
                    }
                }
            }
        } else {
            const int64_t nvalid = a.length - blk * BLK < BLK ? a.length - blk * BLK : BLK;
            const uint32_t *vp = reinterpret_cast<const uint32_t *>(a.c.v16 + (row_base + blk * BLK) * D) + lane;
            for (int tk = 0; tk < nvalid; ++tk) {
                const uint32_t pair = vp[tk * (D / 2)];
                const float f0 = h2f(pair & 0xFFFFu), f1 = h2f(pair >> 16);
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    if (h >= g) break;
                    const float wv = w_lds[wave][h][0][tk];
                    acc[h][0] += wv * f0;
                    acc[h][1] += wv * f1;
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---------------- merge waves, then splits
    __syncthreads();  // every wave is done with w_lds: reuse it as [wave][head][channel]
    float *wacc = &w_lds[0][0][0][0];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        if (h >= g) break;
        wacc[(wave * GP + h) * D + 2 * lane] = acc[h][0];
        wacc[(wave * GP + h) * D + 2 * lane + 1] = acc[h][1];
        if (lane == 0) {
            wm[wave][h] = m_run[h];
            wl[wave][h] = l_run[h];
        }
    }
    __syncthreads();
    write_partial<NW>(a, bh, split, GP, wm, wl, wacc);
}

// ------------------------------------------------------------ split merge

static_assert(MAX_SPLITS <= 128, "the split merge covers at most 128 splits (two per lane)");

// Split merge of head h of (b, kvh): with M = max_s m_s and
// L = sum_s l_s 2^(m_s - M), out = sum_s 2^(m_s - M) acc_s / L.  One
// workgroup per head; wave w sums the splits w, w + 4, ..., lane l holds
// channels 2l and 2l + 1, and the four waves' sums meet in LDS.  With no
// valid token in any split (length 0) the output is 0.
__global__ __launch_bounds__(256) void merge_splits_kernel(DecodeArgs a) {
    __shared__ float2 red[4][64];
    const int h = blockIdx.x;
    const int64_t kvh = blockIdx.y, b = blockIdx.z;
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g, S = a.splits;
    const int64_t head = b * a.hq + kvh * g + h;
    if (a.gate && !a.gate[head]) return;  // recompute pass: only the recomputed heads
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float2 *pml = a.part_ml + bh * S * g + h;  // split s at pml[s * g]
    const float *pacc = a.part_acc + (bh * S * g + h) * D + 2 * lane;  // split s at pacc[s * g * D]
    constexpr float NEG_INF = -__builtin_huge_valf();
    // the first split's partial of this wave is loaded with (m, l), before
    // the maxima are known
    const float2 v0 = wave < S ? *reinterpret_cast<const float2 *>(pacc + (int64_t)wave * g * D)
                               : make_float2(0.0f, 0.0f);
    // M and L over the splits (at most 128: lanes l and l + 64), on DPP moves
    const float2 e0 = lane < S ? pml[lane * g] : make_float2(NEG_INF, 0.0f);
    const float2 e1 = lane + 64 < S ? pml[(lane + 64) * g] : make_float2(NEG_INF, 0.0f);
    const float M = wave_total_max(fmaxf(e0.x, e1.x));
    float L = 0.0f;
    if (e0.x != NEG_INF) L += e0.y * __builtin_amdgcn_exp2f(e0.x - M);
    if (e1.x != NEG_INF) L += e1.y * __builtin_amdgcn_exp2f(e1.x - M);
    L = wave_total_sum(L);
    float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll 8
    for (int s = wave; s < S; s += 4) {
        const float m_s = pml[s * g].x;
        const float w = (L > 0.0f && m_s != NEG_INF) ? __builtin_amdgcn_exp2f(m_s - M) / L : 0.0f;
        const float2 v = s == wave ? v0 : *reinterpret_cast<const float2 *>(pacc + (int64_t)s * g * D);
        acc.x += w * v.x;
        acc.y += w * v.y;
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        float2 o = red[0][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            o.x += red[w][lane].x;
            o.y += red[w][lane].y;
        }
        const uint32_t pair = (uint32_t)f2h_rn(o.x) | ((uint32_t)f2h_rn(o.y) << 16);
        *reinterpret_cast<uint32_t *>(a.out + head * D + 2 * lane) = pair;
    }
}

hipError_t launch_merge(const DecodeArgs &a, int batch, hipStream_t s) {
    hipLaunchKernelGGL(merge_splits_kernel, dim3((unsigned)a.g, (unsigned)a.hkv, (unsigned)batch), dim3(256), 0, s,
                       a);
    return hipGetLastError();
}

hipError_t launch_decode_valu(const DecodeArgs &a, int batch, hipStream_t s) {
    dim3 grid((unsigned)a.splits, (unsigned)a.hkv, (unsigned)batch);
    const int g = a.g;
    if (g <= 1)
        hipLaunchKernelGGL(decode_valu_kernel<1>, grid, dim3(256), 0, s, a);
    else if (g <= 2)
        hipLaunchKernelGGL(decode_valu_kernel<2>, grid, dim3(256), 0, s, a);
    else if (g <= 4)
        hipLaunchKernelGGL(decode_valu_kernel<4>, grid, dim3(256), 0, s, a);
    else if (g <= 8)
        hipLaunchKernelGGL(decode_valu_kernel<8>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(decode_valu_kernel<16>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
