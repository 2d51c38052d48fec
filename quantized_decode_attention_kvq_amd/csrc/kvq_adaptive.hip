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
// The ranking check itself runs in the certificate merge (kvq_certify.hip),
// on the FP16 block log-masses from the certifying decode, which writes each
// FP16 key step's per-head largest score and exp2-sum (no second read of the
// keys).
#include "kvq_decode_common.hpp"
#include "kvq_mfma.hpp"
#include "kvq_quant_row.hpp"

namespace kvq {

namespace {

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr int BPW = 1;        // blocks per wave of the scoring pass (more waves in flight beat fewer, longer ones)

// Rotated query of the Hadamard-rotated key codec, once per call: grid
// (Hkv, B), one wave; lane (head m, k-group g4) rotates as in the decode and
// stores hi and lo at qrot[head][0 / 1][32 g4 .. +32].
__global__ __launch_bounds__(64) void rotate_query_kernel(AdaptArgs a) {
    const int lane = threadIdx.x;
    const int m = lane & 15, g4 = lane >> 4;
    const int64_t kvh = blockIdx.x, b = blockIdx.y;
    const int g = a.g;
    const int64_t head = (b * a.hq) + kvh * g + (m < g ? m : 0);
    uint4 qb[4], hi[4], lo[4];
    const uint16_t *qh = a.q + head * D + 32 * g4;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
        qb[kc] = m < g ? *reinterpret_cast<const uint4 *>(qh + 8 * kc) : make_uint4(0u, 0u, 0u, 0u);
    rotate_q(qb, lane, hi, lo);
    if (m < g) {
        uint16_t *dst = a.qrot + head * 2 * D + 32 * g4;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            *reinterpret_cast<uint4 *>(dst + 8 * kc) = hi[kc];
            *reinterpret_cast<uint4 *>(dst + D + 8 * kc) = lo[kc];
        }
    }
}

// Scoring pass.  Grid (ceil(nb / (4 * BPW)), Hkv, B), 4 waves; wave w of
// workgroup x scores blocks (4x + w) * BPW .. +BPW - 1.  Per 16-token tile,
// Q.K^T on v_mfma_f32_16x16x32_f16 with the tokens on M and the heads on N:
// lane (row m, k-group g4) holds channels 32 g4 + 8 kc .. +8 of token m for
// instruction kc (32 contiguous code bytes per lane), and the q operand uses
// the same channel order.  Result lane (head m, g4): tokens 4 g4 .. +3.
// With a.t_new >= 0 the wave of that token's block first appends it (the
// fused append's arithmetic: the row quantized by lanes 0-15, its tier-1
// bytes and its block's statistics written as the append kernel would) and
// scores the block with the token's fresh codes and scale.
template <bool ROT>
__global__ __launch_bounds__(256) void score_int8_kernel(AdaptArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t nk_lds[4][D], nv_lds[4][D];  // the appended token's codes
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g4 = lane >> 4;
    const int64_t kvh = blockIdx.y, b = blockIdx.z;
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g;
    // the query (plain codec) or the rotated query's hi and lo parts
    uint4 qb[4], qrl[4];
    {
        const int64_t head = (b * a.hq) + kvh * g + (m < g ? m : 0);
        const uint16_t *qh = ROT ? a.qrot + head * 2 * D + 32 * g4 : a.q + head * D + 32 * g4;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            qb[kc] = m < g ? *reinterpret_cast<const uint4 *>(qh + 8 * kc) : make_uint4(0u, 0u, 0u, 0u);
            if (ROT) qrl[kc] = m < g ? *reinterpret_cast<const uint4 *>(qh + D + 8 * kc) : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    const float sml2 = a.sm * 1.4426950408889634f;
    for (int r = 0; r < BPW; ++r) {
        const int64_t i = ((int64_t)blockIdx.x * 4 + wave) * BPW + r;
        if (i >= a.nb) break;
        const int64_t t0 = i * BLK;
        // the appended token, when it lies in this block (wave-uniform)
        const bool app = a.t_new >= 0 && a.t_new / BLK == i;
        const int p_new = app ? (int)(a.t_new % BLK) : -1;
        uint32_t nks = 0u;
        if (app) {
            const int64_t row = bh * a.cap + a.t_new;
            RowQuant rq = {};
            if (lane < 16) {
                rq = quant_row16(load_row16(a.c.k16 + row * D, a.c.v16 + row * D, lane), ROT, lane);
                *reinterpret_cast<uint2 *>(&nk_lds[wave][8 * lane]) = make_uint2(rq.kc[0], rq.kc[1]);
                *reinterpret_cast<uint2 *>(&nv_lds[wave][8 * lane]) = make_uint2(rq.vc[0], rq.vc[1]);
                // tier-1 bytes: key codes, key scale, value scales
                *reinterpret_cast<uint2 *>(a.c.k_codes + row * D + 8 * lane) = make_uint2(rq.kc[0], rq.kc[1]);
                if (lane == 0) a.c.k_scales[row] = (uint16_t)rq.ksb;
                if ((lane & 3) == 0) a.c.v_scales[row * 4 + (lane >> 2)] = (uint16_t)rq.vsb;
            }
            nks = __builtin_amdgcn_readfirstlane(rq.ksb);
            const uint32_t kerr = __builtin_amdgcn_readfirstlane(__float_as_uint(rq.kerr));
            const uint32_t verr = __builtin_amdgcn_readfirstlane(__float_as_uint(rq.verr));
            // value nibbles: a new block starts with the token's nibble in
            // byte (c, 0) and zeros elsewhere; else the token's nibble is
            // replaced in its byte (clear, then set: same address, in order)
            uint8_t *vblk = a.c.v_codes + (bh * a.nbc + i) * (D * BLK / 2);
            if (p_new == 0) {
                for (int k = lane; k < D * 2; k += 64)
                    *reinterpret_cast<uint4 *>(vblk + 16 * k) =
                        make_uint4((k & 1) ? 0u : (uint32_t)(nv_lds[wave][k >> 1] & 0x0Fu), 0u, 0u, 0u);
            } else {
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int ch = lane + 64 * k;
                    const int byte = ch * (BLK / 2) + (p_new >> 1);
                    const int sh = 8 * (byte & 3) + 4 * (p_new & 1);
                    unsigned int *word = reinterpret_cast<unsigned int *>(vblk + (byte & ~3));
                    atomicAnd(word, ~(0x0Fu << sh));
                    atomicOr(word, (uint32_t)(nv_lds[wave][ch] & 0x0Fu) << sh);
                }
            }
            // block statistics: max with the earlier tokens' (non-negative
            // floats and +Inf order like their bit patterns), or the token's
            // own for a new block
            if (lane == 0) {
                const int64_t si = bh * a.nbc + i;
                if (p_new > 0) {
                    atomicMax(reinterpret_cast<unsigned int *>(a.c.k_err + si), kerr);
                    atomicMax(reinterpret_cast<unsigned int *>(a.c.v_err + si), verr);
                } else {
                    a.c.k_err[si] = __uint_as_float(kerr);
                    a.c.v_err[si] = __uint_as_float(verr);
                }
            }
        }
        float sc[4][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int8_t *row = a.c.k_codes + (bh * a.cap + t0 + 16 * tt + m) * D + 32 * g4;
            uint4 c0 = *reinterpret_cast<const uint4 *>(row);
            uint4 c1 = *reinterpret_cast<const uint4 *>(row + 16);
            if (app && 16 * tt + m == p_new) {
                // the appended row, from this launch's quantization
                c0 = *reinterpret_cast<const uint4 *>(&nk_lds[wave][32 * g4]);
                c1 = *reinterpret_cast<const uint4 *>(&nk_lds[wave][32 * g4 + 16]);
            }
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
            const uint4 a0 = i8x8_to_h8(c0.x, c0.y), a1 = i8x8_to_h8(c0.z, c0.w);
            const uint4 a2 = i8x8_to_h8(c1.x, c1.y), a3 = i8x8_to_h8(c1.z, c1.w);
            acc = mfma(a0, qb[0], acc);
            acc = mfma(a1, qb[1], acc);
            acc = mfma(a2, qb[2], acc);
            acc = mfma(a3, qb[3], acc);
            if (ROT) {
                acc = mfma(a0, qrl[0], acc);
                acc = mfma(a1, qrl[1], acc);
                acc = mfma(a2, qrl[2], acc);
                acc = mfma(a3, qrl[3], acc);
            }
            const uint2 ks = *reinterpret_cast<const uint2 *>(a.c.k_scales + bh * a.cap + t0 + 16 * tt + 4 * g4);
            uint32_t kw[4] = {ks.x & 0xFFFFu, ks.x >> 16, ks.y & 0xFFFFu, ks.y >> 16};
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                if (app && 16 * tt + 4 * g4 + rr == p_new) kw[rr] = nks;
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
// SEL_REGS: masses per lane held in registers (64 * SEL_REGS blocks per head;
// the launcher takes the smallest that holds the sequence, 16 or 32).
template <int SEL_REGS>
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
        const bool in_regs = nb <= 64 * SEL_REGS;
        // the lane's masses in registers when they fit (every load issued
        // before the first is used; 0 past nb, never counted as every probe
        // is above 0), else in LDS
        float mr[SEL_REGS], ve[SEL_REGS];
        float mx = NEG_INF, tot = 0.0f;
        if (in_regs) {
            // the value errors (for value promotion) are loaded with the masses
#pragma unroll
            for (int k = 0; k < SEL_REGS; ++k) {
                mr[k] = lane + 64 * k < nb ? lh[lane + 64 * k] : NEG_INF;
                ve[k] = lane + 64 * k < nb ? a.c.v_err[bh * a.nbc + lane + 64 * k] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < SEL_REGS; ++k) mx = fmaxf(mx, mr[k]);
            mx = wave_total_max(mx);
#pragma unroll
            for (int k = 0; k < SEL_REGS; ++k) {
                mr[k] = mr[k] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(mr[k] - mx);
                tot += mr[k];
            }
        } else {
#pragma unroll 8
            for (int i = lane; i < nb; i += 64) mx = fmaxf(mx, lh[i]);
            mx = wave_total_max(mx);
#pragma unroll 8
            for (int i = lane; i < nb; i += 64) {
                const float v = __builtin_amdgcn_exp2f(lh[i] - mx);
                ms[i] = v;
                tot += v;
            }
        }
        tot = wave_total_sum(tot);
        const float target = a.tau_cov * tot;
        const bool none = !(a.tau_cov > 0.0f);
        const bool all = !none && !(target <= tot);  // out of reach (or NaN): every block
        uint32_t lo = 0u, hi = 0x3F800001u;            // F(lo) >= target > F(hi); masses are at most 1
        if (!none && !all && in_regs) {
            while (hi - lo > 1u) {
                const uint32_t mid = lo + (hi - lo) / 2u;
                float f = 0.0f;
#pragma unroll
                for (int k = 0; k < SEL_REGS; ++k) f += __float_as_uint(mr[k]) >= mid ? mr[k] : 0.0f;
                f = wave_total_sum(f);
                if (f >= target)
                    lo = mid;
                else
                    hi = mid;
            }
        } else if (!none && !all) {
            while (hi - lo > 1u) {
                const uint32_t mid = lo + (hi - lo) / 2u;
                float f = 0.0f;
#pragma unroll 8
                for (int i = lane; i < nb; i += 64)
                    if (__float_as_uint(ms[i]) >= mid) f += ms[i];
                f = wave_total_sum(f);
                if (f >= target)
                    lo = mid;
                else
                    hi = mid;
            }
        }
        int cnt = 0;
        auto mark = [&](int i, float mi, float ve) {
            const bool pk = !none && (all || __float_as_uint(mi) >= lo);
            const bool pv = (mi / tot) * ve > a.tau_vc;
            a.phead[head * a.nbc + i] = pk ? 1 : 0;
            cnt += pk ? 1 : 0;
            const uint32_t bits = (pk ? 1u : 0u) | (pv ? 2u : 0u);
            if (bits) atomicOr(&uni[i >> 2], bits << (8 * (i & 3)));
        };
        if (in_regs) {
#pragma unroll
            for (int k = 0; k < SEL_REGS; ++k)
                if (lane + 64 * k < nb) mark(lane + 64 * k, mr[k], ve[k]);
        } else {
#pragma unroll 8
            for (int i = lane; i < nb; i += 64) mark(i, ms[i], a.c.v_err[bh * a.nbc + i]);
        }
        cnt = wave_total_sum_int(cnt);
        if (lane == 0 && a.kstar) a.kstar[head] = cnt;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += 256) a.promote[bh * a.nbc + i] = (uint8_t)(uni[i >> 2] >> (8 * (i & 3)));
}

}  // namespace

hipError_t launch_score(const AdaptArgs &a, int batch, hipStream_t s) {
    const unsigned gx = (unsigned)((a.nb + 4 * BPW - 1) / (4 * BPW));
    const dim3 grid(gx, (unsigned)a.hkv, (unsigned)batch);
    if (a.key_rot) {
        hipLaunchKernelGGL(rotate_query_kernel, dim3((unsigned)a.hkv, (unsigned)batch), dim3(64), 0, s, a);
        hipLaunchKernelGGL(score_int8_kernel<true>, grid, dim3(256), 0, s, a);
    } else
        hipLaunchKernelGGL(score_int8_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_select(const AdaptArgs &a, int batch, hipStream_t s) {
    if (a.nb <= 64 * 16)
        hipLaunchKernelGGL(select_kernel<16>, dim3((unsigned)a.hkv, (unsigned)batch), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(select_kernel<32>, dim3((unsigned)a.hkv, (unsigned)batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
