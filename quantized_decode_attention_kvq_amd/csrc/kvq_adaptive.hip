// kvq_adaptive.hip -- adaptive precision: the INT8 scoring pass, top-K*
// coverage selection with value promotion, and the ranking-consistency check.
//
// "Runtime-Certified Bounded-Error Quantized Attention", technical summary,
// Methodology 3: "Adaptive Top-K Selection" (a light scoring pass over the
// INT8 keys estimates each block's attention mass; the top-K* blocks covering
// tau_cov of it are promoted to FP16 keys), the "Ranking-Consistency Check"
// (the INT8 and FP16 rankings of the promoted blocks are compared; an
// inconsistent head falls back to dense attention) and rungs 1-3 of the
// fallback ladder (coverage, value promotion, per-head fallback).  Readings,
// for query head h of (b, kvh):
//   scoring     lhat_i = log2 sum_{t in block i, t < length} exp2(sm*log2(e) *
//               s_t * q_h . c_t) over the dequantized keys of every block;
//               masses m_i = exp2(lhat_i - max) / S, S their sum.
//   rung 1      the blocks whose mass is at least the K*-th largest, K* the
//               smallest count whose largest masses sum to tau_cov (none
//               when tau_cov <= 0; all when the sum never gets there); a key
//               tile is promoted when any head of its group promotes it.
//   rung 2      a value tile is promoted when m_i * v_err_i > tau_vc for some
//               head of the group.
//   check       over the head's own promoted blocks, the share of pairs the
//               INT8 and FP16 block log-masses order oppositely; above
//               tau_rank the head is flagged for the FP16 recompute.
// The FP16 block log-masses come from the certifying decode, which writes
// each FP16 key step's per-head largest score and exp2-sum (no second read of
// the keys).
#include "kvq_decode_common.hpp"
#include "kvq_mfma.hpp"

namespace kvq {

namespace {

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr int BPW = 4;  // blocks per wave of the scoring pass

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// Scoring pass.  Grid (ceil(nb / (4 * BPW)), Hkv, B), 4 waves; wave w of
// workgroup x scores blocks (4x + w) * BPW .. +BPW - 1.  Per 16-token tile,
// Q.K^T on v_mfma_f32_16x16x32_f16 with the tokens on M and the heads on N:
// lane (row m, k-group g4) holds channels 32 g4 + 8 kc .. +8 of token m for
// instruction kc (32 contiguous code bytes per lane), and the q operand uses
// the same channel order.  Result lane (head m, g4): tokens 4 g4 .. +3.
__global__ __launch_bounds__(256) void score_int8_kernel(AdaptArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g4 = lane >> 4;
    const int64_t kvh = blockIdx.y, b = blockIdx.z;
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g;
    uint4 qb[4];
    {
        const uint16_t *qh = a.q + ((b * a.hq) + kvh * g + (m < g ? m : 0)) * D + 32 * g4;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
            qb[kc] = m < g ? *reinterpret_cast<const uint4 *>(qh + 8 * kc) : make_uint4(0u, 0u, 0u, 0u);
    }
    const float sml2 = a.sm * 1.4426950408889634f;
    for (int r = 0; r < BPW; ++r) {
        const int64_t i = ((int64_t)blockIdx.x * 4 + wave) * BPW + r;
        if (i >= a.nb) break;
        const int64_t t0 = i * BLK;
        float sc[4][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int8_t *row = a.c.k_codes + (bh * a.cap + t0 + 16 * tt + m) * D + 32 * g4;
            const uint4 c0 = *reinterpret_cast<const uint4 *>(row);
            const uint4 c1 = *reinterpret_cast<const uint4 *>(row + 16);
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma(i8x8_to_h8(c0.x, c0.y), qb[0], acc);
            acc = mfma(i8x8_to_h8(c0.z, c0.w), qb[1], acc);
            acc = mfma(i8x8_to_h8(c1.x, c1.y), qb[2], acc);
            acc = mfma(i8x8_to_h8(c1.z, c1.w), qb[3], acc);
            const uint2 ks = *reinterpret_cast<const uint2 *>(a.c.k_scales + bh * a.cap + t0 + 16 * tt + 4 * g4);
            const uint32_t kw[4] = {ks.x & 0xFFFFu, ks.x >> 16, ks.y & 0xFFFFu, ks.y >> 16};
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int64_t t = t0 + 16 * tt + 4 * g4 + rr;
                // rows past `length` hold stale codes and scales: never used
                sc[tt][rr] = t < a.length ? acc[rr] * (h2f(kw[rr]) * sml2) : NEG_INF;
            }
        }
        float mx = NEG_INF;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, sc[tt][rr]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        float sum = 0.0f;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sum += sc[tt][rr] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(sc[tt][rr] - mx);
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        if (g4 == 0 && m < g) a.lhat[((b * a.hq) + kvh * g + m) * a.nbc + i] = mx + __log2f(sum);
    }
}

// Selection.  Grid (Hkv, B), 4 waves; wave w takes heads w, w + 4, ... of the
// group, with its masses in LDS.  The promoted set {i : m_i >= theta} uses the
// largest theta with sum_{m_i >= theta} m_i >= tau_cov * S, found by a binary
// search over the bit patterns of non-negative floats (which order like the
// values); that theta is the K*-th largest mass.
__global__ __launch_bounds__(256) void select_kernel(AdaptArgs a) {
    __shared__ float mass[4][ADAPT_MAX_NB];
    __shared__ uint32_t uni[ADAPT_MAX_NB / 4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t kvh = blockIdx.x, b = blockIdx.y;
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g, nb = (int)a.nb;
    for (int i = threadIdx.x; i < (nb + 3) / 4; i += 256) uni[i] = 0u;
    __syncthreads();
    float *ms = mass[wave];
    for (int hl = wave; hl < g; hl += 4) {
        const int64_t head = b * a.hq + kvh * g + hl;
        const float *lh = a.lhat + head * a.nbc;
        float mx = NEG_INF;
        for (int i = lane; i < nb; i += 64) mx = fmaxf(mx, lh[i]);
        mx = wave_max(mx);
        float tot = 0.0f;
        for (int i = lane; i < nb; i += 64) {
            const float v = __builtin_amdgcn_exp2f(lh[i] - mx);
            ms[i] = v;
            tot += v;
        }
        tot = wave_sum(tot);
        const float target = a.tau_cov * tot;
        const bool none = !(a.tau_cov > 0.0f);
        const bool all = !none && !(target <= tot);  // out of reach (or NaN): every block
        uint32_t lo = 0u, hi = 0x7F800000u;            // F(lo) >= target > F(hi)
        if (!none && !all) {
            while (hi - lo > 1u) {
                const uint32_t mid = lo + (hi - lo) / 2u;
                float f = 0.0f;
                for (int i = lane; i < nb; i += 64)
                    if (__float_as_uint(ms[i]) >= mid) f += ms[i];
                f = wave_sum(f);
                if (f >= target)
                    lo = mid;
                else
                    hi = mid;
            }
        }
        int cnt = 0;
        for (int i = lane; i < nb; i += 64) {
            const bool pk = !none && (all || __float_as_uint(ms[i]) >= lo);
            const bool pv = (ms[i] / tot) * a.c.v_err[bh * a.nbc + i] > a.tau_vc;
            a.phead[head * a.nbc + i] = pk ? 1 : 0;
            cnt += pk ? 1 : 0;
            const uint32_t bits = (pk ? 1u : 0u) | (pv ? 2u : 0u);
            if (bits) atomicOr(&uni[i >> 2], bits << (8 * (i & 3)));
        }
        cnt = wave_sum_int(cnt);
        if (lane == 0 && a.kstar) a.kstar[head] = cnt;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += 256) a.promote[bh * a.nbc + i] = (uint8_t)(uni[i >> 2] >> (8 * (i & 3)));
}

// FP16 block log-mass (log2 units) of block i for head hl of (b, kvh), from
// the decode's per-step statistics of the block's valid 8-token steps.
__device__ float fp16_block_logmass(const AdaptArgs &a, int64_t bh, int64_t i, int hl) {
    const int64_t left = a.length - i * BLK;
    const int nst = left >= BLK ? 8 : (int)((left + 7) / 8);
    const float2 *st = a.step_ml + (bh * a.nbc + i) * 8 * a.g + hl;
    float L[8], M = NEG_INF;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        L[k] = NEG_INF;
        if (k < nst) {
            const float2 p = st[k * a.g];
            if (p.y > 0.0f) L[k] = p.x + __log2f(p.y);
        }
        M = fmaxf(M, L[k]);
    }
    if (M == NEG_INF) return NEG_INF;
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (L[k] != NEG_INF) s += __builtin_amdgcn_exp2f(L[k] - M);
    return M + __log2f(s);
}

// Ranking check.  Grid (Hq, B), 4 waves: the head's promoted blocks are
// compacted into LDS (INT8 and FP16 log-masses), then every pair is compared.
__global__ __launch_bounds__(256) void check_kernel(AdaptArgs a) {
    __shared__ float pa[ADAPT_MAX_NB], pf[ADAPT_MAX_NB];
    __shared__ int wcnt[4];
    __shared__ unsigned wred[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t h = blockIdx.x, b = blockIdx.y;
    const int g = a.g;
    const int64_t kvh = h / g, hl = h % g;
    const int64_t bh = b * a.hkv + kvh, head = b * a.hq + h;
    const uint8_t *ph = a.phead + head * a.nbc;
    const float *lh = a.lhat + head * a.nbc;
    int n = 0;
    for (int64_t c0 = 0; c0 < a.nb; c0 += 256) {
        const int64_t i = c0 + tid;
        const bool f = i < a.nb && ph[i] != 0;
        const uint64_t bal = __ballot(f);
        if (lane == 0) wcnt[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int v = wcnt[w];
            before += w < wave ? v : 0;
            tot += v;
        }
        if (f) {
            const int pos = n + before + __popcll(bal & ((1ull << lane) - 1ull));
            pa[pos] = lh[i];
            pf[pos] = fp16_block_logmass(a, bh, i, (int)hl);
        }
        n += tot;
        __syncthreads();
    }
    unsigned cnt = 0u;
    for (int i = tid; i < n; i += 256) {
        const float ai = pa[i], fi = pf[i];
        for (int j = i + 1; j < n; ++j) cnt += ((ai - pa[j]) * (fi - pf[j]) < 0.0f) ? 1u : 0u;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) cnt += (unsigned)__shfl_xor((int)cnt, o);
    if (lane == 0) wred[wave] = cnt;
    __syncthreads();
    if (tid == 0) {
        const unsigned nd = wred[0] + wred[1] + wred[2] + wred[3];
        const double np = (double)n * (double)(n - 1) / 2.0;
        if (a.ndisc) a.ndisc[head] = (int32_t)nd;
        if (np > 0.0 && (double)nd > (double)a.tau_rank * np) a.flags[head] = 1;
    }
}

}  // namespace

hipError_t launch_score(const AdaptArgs &a, int batch, hipStream_t s) {
    const unsigned gx = (unsigned)((a.nb + 4 * BPW - 1) / (4 * BPW));
    hipLaunchKernelGGL(score_int8_kernel, dim3(gx, (unsigned)a.hkv, (unsigned)batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_select(const AdaptArgs &a, int batch, hipStream_t s) {
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)a.hkv, (unsigned)batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_check(const AdaptArgs &a, int batch, hipStream_t s) {
    hipLaunchKernelGGL(check_kernel, dim3((unsigned)a.hq, (unsigned)batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
