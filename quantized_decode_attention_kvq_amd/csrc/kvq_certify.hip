// kvq_certify.hip -- the merge of a certified decode: the split merge of the
// outputs plus, per query head, the output certificate and the decision to
// recompute the head on FP16.
//
// "Runtime-Certified Bounded-Error Quantized Attention", Methodology 2 ("Two-
// Term Error Decomposition": a key term from the per-token score
// perturbation through the total variation of the softmax, a value term from
// the per-block value reconstruction errors weighted by attention mass, both
// from quantities the decode already tracks) and Methodology 3 (rung 3 of the
// fallback ladder: per-head FP16 recompute).  For head h of (b, kvh):
//   Delta  = sm * ||q_h|| * (largest key error of a key-certified block), as
//            the key bound of the masks (fp32 products, inflated by 2^-16);
//   R      = 2 * max(7 * S + eta, A): S the largest value scale of a value-
//            certified token, eta the largest value error of a value-
//            certified block, A the largest |v| of a value-fallback token;
//   E_key  = tanh(Delta / 2) * R;
//   E_val  = sum over value-certified blocks of (attention mass) * (value
//            error), merged across splits like the softmax sums;
//   cert   = E_key + E_val, rounded up to fp32.
// Every output channel's distance from dense FP16 attention is at most cert
// in exact arithmetic (the kernel's own fp16/fp32 rounding comes on top).
// Heads with cert > tau_out are flagged for recompute.
#include "kvq_decode_common.hpp"

namespace kvq {

namespace {

// FP16 block log-mass (log2 units) of block i < nb for head hl of group bh,
// from the decode's statistics of the block's valid 8-token slots (a
// 16-token step fills its first slot and empties the second).  The loads
// are unconditional (slots past the valid ones re-read the last valid one)
// so that they issue together.
__device__ __forceinline__ float fp16_block_logmass(const DecodeArgs &a, int64_t bh, int64_t i, int hl) {
    constexpr float NEG_INF = -__builtin_huge_valf();
    const int64_t left = a.length - i * BLK;
    const int nst = left >= BLK ? 8 : (int)((left + 7) / 8);
    const float2 *st = a.step_ml + (bh * a.nbc + i) * 8 * a.g + hl;
    float2 p[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = st[(k < nst ? k : nst - 1) * a.g];
    float L[8], M = NEG_INF;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        L[k] = (k < nst && p[k].y > 0.0f) ? p[k].x + __log2f(p[k].y) : NEG_INF;
        M = fmaxf(M, L[k]);
    }
    if (M == NEG_INF) return NEG_INF;
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (L[k] != NEG_INF) s += __builtin_amdgcn_exp2f(L[k] - M);
    return M + __log2f(s);
}

// Promoted blocks per head up to which the ranking check counts every pair.
constexpr int PAIRWISE_MAX = 1024;

// First index in [lo, hi) of an ascending run whose key is >= k (lower) or
// > k (upper); keys (x, y) compare lexicographically, or by y alone when x
// is null.
template <bool UPPER>
__device__ __forceinline__ int run_bound(const float *x, const float *y, int lo, int hi, float kx, float ky) {
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const float xm = x ? x[mid] : 0.0f, ym = y[mid];
        const float kxx = x ? kx : 0.0f;
        const bool before = UPPER ? (xm < kxx || (xm == kxx && ym <= ky)) : (xm < kxx || (xm == kxx && ym < ky));
        if (before)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// One bottom-up pass of a stable merge sort over n keys in LDS (run width w
// to 2w): an element of a left run moves past the right run's smaller keys,
// one of a right run past the left run's smaller or equal keys (binary
// searches, so every element is placed independently).  With x null the key
// is y alone, and the return value counts, over this thread's right-run
// elements, the left-run keys strictly above them: summed over the passes,
// the inversions of the sequence.
__device__ __forceinline__ int merge_pass(const float *x, const float *y, float *nx, float *ny, int n, int w) {
    int inv = 0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int r0 = i / (2 * w) * (2 * w);
        const int le = r0 + w < n ? r0 + w : n, re = r0 + 2 * w < n ? r0 + 2 * w : n;
        const float kx = x ? x[i] : 0.0f, ky = y[i];
        int dst;
        if (i < le) {
            dst = i + (run_bound<false>(x, y, le, re, kx, ky) - le);
        } else {
            const int ub = run_bound<true>(x, y, r0, le, kx, ky);
            dst = r0 + (i - le) + (ub - r0);
            inv += le - ub;
        }
        if (x) nx[dst] = kx;
        ny[dst] = ky;
    }
    return inv;
}

// Ranking-consistency check of one head (Methodology 3): its promoted blocks
// are compacted into LDS with their INT8 and FP16 log-masses, the pairs
// ordered oppositely are counted (every pair up to PAIRWISE_MAX blocks, by
// merge sorts above), and the head is inconsistent when they exceed tau_rank
// of all pairs.  All 256 threads take part; every thread returns the result.
__device__ bool ranking_inconsistent(const DecodeArgs &a, int64_t bh, int64_t head, int hl, float *pa, float *pf,
                                     float *qa, float *qf, int *wcnt, int *bcast) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (a.nb == 0) {  // uniform: no barrier is skipped by part of the workgroup
        if (tid == 0 && a.ndisc) a.ndisc[head] = 0;
        return false;
    }
    const uint8_t *ph = a.phead + head * a.nbc;
    const float *lh = a.lhat + head * a.nbc;
    // thread t takes blocks [t*K, t*K + K): count its promoted blocks, scan
    // the counts over the workgroup, then write the entries (pair order is
    // irrelevant to the count)
    const int nb = (int)a.nb, K = (nb + 255) / 256;
    const int i0 = tid * K < nb ? tid * K : nb, i1 = i0 + K < nb ? i0 + K : nb;
    // up to KR blocks per thread: every load issued at once (the log-masses
    // of blocks that turn out not promoted are simply unused)
    constexpr int KR = 4;
    bool fr[KR];
    float ar[KR], fpr[KR];
    int mine = 0;
    if (K <= KR) {
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            // unconditional loads at a clamped, in-range block
            const int i = i0 + k < nb ? i0 + k : nb - 1;
            fr[k] = i0 + k < i1 && ph[i] != 0;
            ar[k] = lh[i];
            fpr[k] = fp16_block_logmass(a, bh, i, hl);
        }
#pragma unroll
        for (int k = 0; k < KR; ++k) mine += fr[k] ? 1 : 0;
    } else {
        for (int i = i0; i < i1; ++i) mine += ph[i] != 0;
    }
    const int incl = wave_incl_scan_int(mine);
    if (lane == 63) wcnt[wave] = incl;
    __syncthreads();
    int pos = incl - mine, n = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        pos += w < wave ? wcnt[w] : 0;
        n += wcnt[w];
    }
    if (K <= KR) {
#pragma unroll
        for (int k = 0; k < KR; ++k)
            if (fr[k]) {
                pa[pos] = ar[k];
                pf[pos] = fpr[k];
                ++pos;
            }
    } else {
        for (int i = i0; i < i1; ++i)
            if (ph[i] != 0) {
                pa[pos] = lh[i];
                pf[pos] = fp16_block_logmass(a, bh, i, hl);
                ++pos;
            }
    }
    __syncthreads();
    // Discordant pairs: (a_i - a_j)(f_i - f_j) < 0.
    int cnt = 0;
    if (n <= PAIRWISE_MAX) {
        // every pair, 8 at a time (independent LDS reads)
        for (int i = tid; i < n; i += 256) {
            const float ai = pa[i], fi = pf[i];
            int j = i + 1;
            for (; j + 8 <= n; j += 8) {
                float aj[8], fj[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    aj[u] = pa[j + u];
                    fj[u] = pf[j + u];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) cnt += ((ai - aj[u]) * (fi - fj[u]) < 0.0f) ? 1 : 0;
            }
            for (; j < n; ++j) cnt += ((ai - pa[j]) * (fi - pf[j]) < 0.0f) ? 1 : 0;
        }
    } else {
        // Sorted by (a, f), a pair tied in a has f ascending and a pair tied
        // in f is never strictly inverted, so the count is the number of
        // strict inversions of the f sequence in that order: a merge sort by
        // (a, f), then a merge sort by f counting, per pass, the left-run keys
        // above each right-run key.  O(n log n) in log2(n) barrier-separated
        // passes each (the binary searches are dependent LDS reads, so below
        // PAIRWISE_MAX promoted blocks the pairs are cheaper).
        float *ca = pa, *cf = pf, *na = qa, *nf = qf;
        for (int w = 1; w < n; w *= 2) {
            merge_pass(ca, cf, na, nf, n, w);
            __syncthreads();
            float *t = ca;
            ca = na;
            na = t;
            t = cf;
            cf = nf;
            nf = t;
        }
        for (int w = 1; w < n; w *= 2) {  // ca and na are free: na takes the f keys of the next pass
            cnt += merge_pass(nullptr, cf, nullptr, na, n, w);
            __syncthreads();
            float *t = cf;
            cf = na;
            na = t;
        }
    }
    cnt = wave_total_sum_int(cnt);
    __syncthreads();  // every thread has read wcnt
    if (lane == 0) wcnt[wave] = cnt;
    __syncthreads();
    if (tid == 0) {
        const int nd = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
        const double np = (double)n * (double)(n - 1) / 2.0;
        if (a.ndisc) a.ndisc[head] = nd;
        *bcast = np > 0.0 && (double)nd > (double)a.tau_rank * np ? 1 : 0;
    }
    __syncthreads();
    return *bcast != 0;
}

// One workgroup per query head h of (b, kvh).  The output merge is the
// split merge's (every wave forms M and L; wave w sums the splits w, w + 4,
// ..., lane l holds channels 2l and 2l + 1); wave 1 then gathers the
// certificate's parts of the splits (two per lane, summed in double).  RANK
// (adaptive decode): the head's ranking check runs first, and an
// inconsistent head is flagged for the recompute like one whose certificate
// exceeds tau_out.
template <bool RANK>
__global__ __launch_bounds__(256) void merge_cert_kernel(DecodeArgs a) {
    __shared__ float2 red[4][64];
    __shared__ float qn_lds;
    __shared__ float pa[RANK ? ADAPT_MAX_NB : 1], pf[RANK ? ADAPT_MAX_NB : 1];
    __shared__ float qa[RANK ? ADAPT_MAX_NB : 1], qf[RANK ? ADAPT_MAX_NB : 1];  // merge-sort buffers
    __shared__ int wcnt[4], bcast;
    const int h = blockIdx.x;
    const int64_t kvh = blockIdx.y, b = blockIdx.z;
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g, S = a.splits;
    const int64_t head = b * a.hq + kvh * g + h;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr float NEG_INF = -__builtin_huge_valf();
    if (wave == 0) {
        // query norm of head h: lanes 0-15 hold its 128 channels (the other
        // lane groups take part with zeros)
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (lane < 16) raw = *reinterpret_cast<const uint4 *>(a.q + head * D + 8 * lane);
        const float n = qnorm16(raw);
        if (lane == 0) qn_lds = n;
    }
    const float2 *pml = a.part_ml + bh * S * g + h;  // split s at pml[s * g]
    const float2 e0 = lane < S ? pml[lane * g] : make_float2(NEG_INF, 0.0f);
    const float2 e1 = lane + 64 < S ? pml[(lane + 64) * g] : make_float2(NEG_INF, 0.0f);
    const float M = wave_total_max(fmaxf(e0.x, e1.x));  // DPP moves
    float L = 0.0f;
    if (e0.x != NEG_INF) L += e0.y * __builtin_amdgcn_exp2f(e0.x - M);
    if (e1.x != NEG_INF) L += e1.y * __builtin_amdgcn_exp2f(e1.x - M);
    L = wave_total_sum(L);
    const float *pacc = a.part_acc + (bh * S * g + h) * D + 2 * lane;  // split s at pacc[s * g * D]
    float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll 8
    for (int s = wave; s < S; s += 4) {
        const float m_s = pml[s * g].x;
        const float w = (L > 0.0f && m_s != NEG_INF) ? __builtin_amdgcn_exp2f(m_s - M) / L : 0.0f;
        const float2 v = *reinterpret_cast<const float2 *>(pacc + (int64_t)s * g * D);
        acc.x += w * v.x;
        acc.y += w * v.y;
    }
    red[wave][lane] = acc;
    __syncthreads();
    const bool inconsistent = RANK && ranking_inconsistent(a, bh, head, h, pa, pf, qa, qf, wcnt, &bcast);
    if (wave == 0) {
        float2 o = red[0][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            o.x += red[w][lane].x;
            o.y += red[w][lane].y;
        }
        const uint32_t pair = (uint32_t)f2h_rn(o.x) | ((uint32_t)f2h_rn(o.y) << 16);
        *reinterpret_cast<uint32_t *>(a.out + head * D + 2 * lane) = pair;
    } else if (wave == 1) {
        // L and E in double over the splits with a valid token, the
        // largest value scale and fallback |v| over all splits
        double Ld = 0.0, E = 0.0;
        float smax = 0.0f, amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = lane + 64 * k;
            if (r < S) {
                const float2 e = k ? e1 : e0;
                if (e.x != NEG_INF) {
                    const double f = (double)__builtin_amdgcn_exp2f(e.x - M);
                    Ld += (double)e.y * f;
                    E += (double)a.part_e[(bh * S + r) * g + h] * f;
                }
                const float2 sa = a.part_sa[bh * S + r];
                smax = fmaxf(smax, sa.x);
                amax = max_keep_nan(amax, sa.y);  // a NaN value keeps the certificate NaN
            }
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            Ld += __shfl_xor(Ld, o);
            E += __shfl_xor(E, o);
            smax = fmaxf(smax, __shfl_xor(smax, o));
            amax = max_keep_nan(amax, __shfl_xor(amax, o));
        }
        if (lane == 0) {
            const float2 kv = a.part_kv[bh];
            const double e_val = Ld > 0.0 ? E / Ld : 0.0;
            const double delta = (double)key_bound(a.sm, qn_lds, kv.x);
            const double r1 = 7.0 * (double)smax + (double)kv.y;
            const double range = 2.0 * ((double)amax != (double)amax || (double)amax > r1 ? (double)amax : r1);
            const double c = tanh(0.5 * delta) * range + e_val;
            float cf = (float)c;
            if ((double)cf < c) cf = __uint_as_float(__float_as_uint(cf) + 1u);  // c >= 0: the next float up
            a.cert[head] = cf;
            a.flags[head] = (cf > a.tau_out || inconsistent) ? 1 : 0;
        }
    }
}

}  // namespace

hipError_t launch_merge_cert(const DecodeArgs &a, int batch, hipStream_t s) {
    const dim3 grid((unsigned)a.g, (unsigned)a.hkv, (unsigned)batch);
    if (a.step_ml)
        hipLaunchKernelGGL(merge_cert_kernel<true>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(merge_cert_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
