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

// FP16 block log-mass (log2 units) of one block of one head: the log2 of
// the sum over the block's valid 8-token slots of l * 2^m, from the
// decode's statistics (m, l) of those slots (a 16-token step fills its first
// slot and empties the second).  A head's slots are contiguous, 8 per block.
__device__ __forceinline__ int block_slots(const DecodeArgs &a, int64_t i) {
    const int64_t left = a.length - i * BLK;
    return left >= BLK ? 8 : (int)((left + 7) / 8);
}

__device__ __forceinline__ float block_logmass(const float4 (&p)[4], int nst) {
    constexpr float NEG_INF = -__builtin_huge_valf();
    float m[8], l[8], L[8], M = NEG_INF;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        m[2 * k] = p[k].x;
        l[2 * k] = p[k].y;
        m[2 * k + 1] = p[k].z;
        l[2 * k + 1] = p[k].w;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        L[k] = (k < nst && l[k] > 0.0f) ? m[k] + __log2f(l[k]) : NEG_INF;
        M = fmaxf(M, L[k]);
    }
    if (M == NEG_INF) return NEG_INF;
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (L[k] != NEG_INF) s += __builtin_amdgcn_exp2f(L[k] - M);
    return M + __log2f(s);
}

// Order-preserving image of a float as an unsigned integer (-0 as +0):
// for non-NaN a, b, a < b exactly when ord_key(a) < ord_key(b).
__device__ __forceinline__ uint32_t ord_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Thread t's blocks are t, t + 256, t + 512, ...  The promoted flag, INT8
// log-mass and FP16 log-mass of its blocks c, c + 256, ..., c + 256 (KR - 1),
// every load issued before any is used; blocks at or past nb re-read block
// nb - 1 and come back unpromoted.
template <int KR>
__device__ __forceinline__ void load_blocks(const DecodeArgs &a, const uint8_t *ph, const float *lh, const float4 *sth,
                                            int c, int nb, bool *fr, float *ar, float *fpr) {
    uint8_t f[KR];
    float4 p[KR][4];
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const int i = c + 256 * k < nb ? c + 256 * k : nb - 1;
        f[k] = ph[i];
        ar[k] = lh[i];
#pragma unroll
        for (int u = 0; u < 4; ++u) p[k][u] = sth[4 * i + u];
    }
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const int i = c + 256 * k < nb ? c + 256 * k : nb - 1;
        fr[k] = (c + 256 * k < nb) & (f[k] != 0);
        fpr[k] = block_logmass(p[k], block_slots(a, i));
    }
}

// Promoted blocks per head up to which the ranking check counts every pair.
constexpr int PAIRWISE_MAX = 256;

// One pass (runs of w to 2w, w a power of two) of a bottom-up stable merge
// sort of n keys in LDS, held in arrays padded from n up to the next power
// of two with keys above every real one.  Each element counts, by binary
// lifting over the whole sibling run (log2(w) + 1 steps, one LDS read
// each), the sibling keys that go before it -- smaller ones for an element
// of a left run, smaller or equal ones for an element of a right run -- and
// moves past them.  E elements per thread (c + tid + 256 e) search together.
// Returns, over this thread's right-run elements, the left-run keys strictly
// above them: summed over the passes, the strict inversions of the sequence.
template <typename Key, int E>
__device__ __forceinline__ int merge_pass(const Key *src, Key *dst, int n, int w) {
    constexpr uint32_t KB = sizeof(Key);
    const char *sb = reinterpret_cast<const char *>(src);
    int inv = 0;
    for (int c = 0; c < n; c += 256 * E) {
        uint32_t off[E];  // byte offset of the sibling run's start plus the count so far
        Key key[E], kk[E];
        bool right[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = c + (int)threadIdx.x + 256 * e;
            const int ii = i < n ? i : n - 1;  // past the end: a copy of the last key, never written
            const int r0 = ii & ~(2 * w - 1);
            right[e] = ii - r0 >= w;
            off[e] = (uint32_t)(right[e] ? r0 : r0 + w) * KB;  // the sibling run
            key[e] = src[ii];
            // "smaller or equal" as "smaller than key + 1" (no real key is the
            // largest value of the type)
            kk[e] = right[e] ? key[e] + 1 : key[e];
        }
        for (int s = w >> 1; s >= 1; s >>= 1) {
            const uint32_t step = (uint32_t)s * KB;
            Key v[E];
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = *reinterpret_cast<const Key *>(sb + off[e] + step - KB);
#pragma unroll
            for (int e = 0; e < E; ++e) off[e] += v[e] < kk[e] ? step : 0u;
        }
        {
            Key v[E];
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = *reinterpret_cast<const Key *>(sb + off[e]);
#pragma unroll
            for (int e = 0; e < E; ++e) off[e] += v[e] < kk[e] ? KB : 0u;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = c + (int)threadIdx.x + 256 * e;
            if (i < n) {
                const int r0 = i & ~(2 * w - 1);
                const int pos = (int)(off[e] / KB) - (right[e] ? r0 : r0 + w);
                dst[right[e] ? i - w + pos : i + pos] = key[e];
                if (right[e]) inv += w - pos;
            }
        }
    }
    return inv;
}

// Both merge sorts of the ranking check with E elements per thread and
// search: the (INT8, FP16) key pairs kp[0 .. n) by their 64-bit keys, then
// their FP16 halves, counting strict inversions.  kp and kq are the pair
// buffers (padded to np2); the FP16 halves use kq's memory.
template <int E>
__device__ __forceinline__ int sort_and_count(uint64_t *kp, uint64_t *kq, int n) {
    uint64_t *src = kp, *dst = kq;
    for (int w = 1; w < n; w *= 2) {
        merge_pass<uint64_t, E>(src, dst, n, w);
        __syncthreads();
        uint64_t *t = src;
        src = dst;
        dst = t;
    }
    // src holds the pairs sorted by (INT8, FP16); dst's memory takes the two
    // 32-bit buffers of the second sort (their padding written here too)
    uint32_t *fs = reinterpret_cast<uint32_t *>(dst), *fd = fs + ADAPT_MAX_NB;
    const int np2 = n > 1 ? 1 << (32 - __builtin_clz(n - 1)) : 1;
    for (int i = threadIdx.x; i < np2; i += 256) {
        fs[i] = i < n ? (uint32_t)src[i] : 0xFFFFFFFFu;
        fd[i] = 0xFFFFFFFFu;
    }
    __syncthreads();
    int cnt = 0;
    for (int w = 1; w < n; w *= 2) {
        cnt += merge_pass<uint32_t, E>(fs, fd, n, w);
        __syncthreads();
        uint32_t *t = fs;
        fs = fd;
        fd = t;
    }
    return cnt;
}

// The promoted blocks of one head, compacted into kp[0 .. n) as keys pairing
// the order-preserving images of their INT8 and FP16 log-masses; returns n.
// Thread t takes blocks t, t + 256, ...: it counts its promoted blocks, the
// counts are scanned over the workgroup, and each thread writes its keys at
// its offset (pair order is irrelevant to the count).  A head of at most
// 256 KR blocks keeps each thread's blocks in registers between the count
// and the writes; a longer one is counted from its flags, then loaded KR
// blocks at a time.  All 256 threads take part.
template <int KR>
__device__ __forceinline__ int compact_keys(const DecodeArgs &a, const uint8_t *ph, const float *lh,
                                            const float4 *sth, int nb, uint64_t *kp, int *wcnt) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = (nb + 255) / 256;
    bool fr[KR];
    float ar[KR], fpr[KR];
    int mine = 0;
    if (K <= KR) {
        load_blocks<KR>(a, ph, lh, sth, tid, nb, fr, ar, fpr);
#pragma unroll
        for (int k = 0; k < KR; ++k) mine += fr[k] ? 1 : 0;
    } else {
        for (int c = tid; c < nb; c += 256 * 16) {
            uint8_t f[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) f[u] = ph[c + 256 * u < nb ? c + 256 * u : nb - 1];
#pragma unroll
            for (int u = 0; u < 16; ++u) mine += (c + 256 * u < nb && f[u] != 0) ? 1 : 0;
        }
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
    auto put = [&](float aa, float ff) {
        kp[pos++] = ((uint64_t)ord_key(aa) << 32) | ord_key(ff);
    };
    if (K > KR) {
        for (int c = tid; c < nb; c += 256 * KR) {
            load_blocks<KR>(a, ph, lh, sth, c, nb, fr, ar, fpr);
#pragma unroll
            for (int k = 0; k < KR; ++k)
                if (fr[k]) put(ar[k], fpr[k]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < KR; ++k)
            if (fr[k]) put(ar[k], fpr[k]);
    }
    return n;
}

// Ranking-consistency check of one head (Methodology 3): its promoted blocks
// are compacted into LDS as keys pairing the order-preserving images of
// their INT8 and FP16 log-masses, the pairs ordered oppositely by the two
// are counted (every pair up to PAIRWISE_MAX blocks, by merge sorts above),
// and the head is inconsistent when they exceed tau_rank of all pairs.  The
// integer images compare exactly like the log-masses, so a pair is
// discordant when one log-mass is strictly lower and the other strictly
// higher (log-masses are finite or -inf here; a NaN, from non-finite
// inputs, leaves the count unspecified).  All 256 threads take part; every
// thread returns the result.
__device__ bool ranking_inconsistent(const DecodeArgs &a, int64_t bh, int64_t head, int hl, uint64_t *kp,
                                     uint64_t *kq, int *wcnt, int *bcast) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (a.nb == 0) {  // uniform: no barrier is skipped by part of the workgroup
        if (tid == 0 && a.ndisc) a.ndisc[head] = 0;
        return false;
    }
    const uint8_t *ph = a.phead + head * a.nbc;
    const float *lh = a.lhat + head * a.nbc;
    const float4 *sth = reinterpret_cast<const float4 *>(a.step_ml + (bh * a.g + hl) * a.nbc * 8);
    // up to 8 blocks per thread are held in registers between the count and
    // the writes, as many as the head has (one load round and one log-mass
    // each); longer heads are counted from their flags, then loaded 8 blocks
    // at a time
    const int nb = (int)a.nb, K = (nb + 255) / 256;
    const int n = K <= 1   ? compact_keys<1>(a, ph, lh, sth, nb, kp, wcnt)
                  : K <= 2 ? compact_keys<2>(a, ph, lh, sth, nb, kp, wcnt)
                  : K <= 4 ? compact_keys<4>(a, ph, lh, sth, nb, kp, wcnt)
                           : compact_keys<8>(a, ph, lh, sth, nb, kp, wcnt);
    // the merge sorts' padding: keys above every real one up to the next
    // power of two, in both pair buffers
    const int np2 = n > 1 ? 1 << (32 - __builtin_clz(n - 1)) : 1;
    if (n > PAIRWISE_MAX)
        for (int i = n + tid; i < np2; i += 256) kp[i] = kq[i] = ~0ull;
    __syncthreads();
    int cnt = 0;
    if (n <= PAIRWISE_MAX) {
        // Discordant pairs one by one, 8 partners at a time: thread i takes
        // the partners i + 1, ..., i + (n - 1) / 2 (mod n), and for even n
        // the opposite one i + n / 2 when i < n / 2 -- every pair once, and
        // about n / 2 of them per thread.
        static_assert(PAIRWISE_MAX <= 256, "one row per thread");
        const int i = tid;
        if (i < n) {
            const uint64_t ki = kp[i];
            const uint32_t ai = (uint32_t)(ki >> 32), fi = (uint32_t)ki;
            const int nd = (n - 1) / 2 + ((n % 2 == 0 && i < n / 2) ? 1 : 0);
            auto disc = [&](uint64_t kj) {
                const uint32_t aj = (uint32_t)(kj >> 32), fj = (uint32_t)kj;
                return ((ai < aj && fi > fj) || (ai > aj && fi < fj)) ? 1 : 0;
            };
            int d = 1;
            for (; d + 8 <= nd + 1; d += 8) {
                uint64_t kj[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = i + d + u;
                    kj[u] = kp[j < n ? j : j - n];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) cnt += disc(kj[u]);
            }
            for (; d <= nd; ++d) {
                const int j = i + d;
                cnt += disc(kp[j < n ? j : j - n]);
            }
        }
    } else {
        // Sorted by (INT8, FP16), a pair tied in INT8 has FP16 ascending and
        // a pair tied in FP16 is never strictly inverted, so the count is the
        // number of strict inversions of the FP16 sequence in that order.
        if (n <= 512)
            cnt = sort_and_count<2>(kp, kq, n);
        else if (n <= 1024)
            cnt = sort_and_count<4>(kp, kq, n);
        else
            cnt = sort_and_count<8>(kp, kq, n);
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
// ..., lane l holds channels 2l and 2l + 1); wave 1 then combines the
// certificate's parts of the splits, loaded at the start with the split
// statistics (two per lane, summed in double).  RANK
// (adaptive decode): the head's ranking check runs first, and an
// inconsistent head is flagged for the recompute like one whose certificate
// exceeds tau_out.
template <bool RANK>
__global__ __launch_bounds__(256) void merge_cert_kernel(DecodeArgs a) {
    __shared__ float2 red[4][64];
    __shared__ float qn_lds;
    __shared__ uint64_t kp[RANK ? ADAPT_MAX_NB : 1], kq[RANK ? ADAPT_MAX_NB : 1];  // ranking keys, merge-sort buffers
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
    // wave 1's certificate parts of the splits (two per lane), loaded with
    // the split statistics: used only at the end
    float pe[2] = {0.0f, 0.0f};
    float2 psa[2] = {make_float2(0.0f, 0.0f), make_float2(0.0f, 0.0f)}, pkv = make_float2(0.0f, 0.0f);
    if (wave == 1) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = lane + 64 * k;
            if (r < S) {
                pe[k] = a.part_e[(bh * S + r) * g + h];
                psa[k] = a.part_sa[bh * S + r];
            }
        }
        pkv = a.part_kv[bh];
    }
    const float M = wave_total_max(fmaxf(e0.x, e1.x));  // DPP moves
    float L = 0.0f;
    if (e0.x != NEG_INF) L += e0.y * __builtin_amdgcn_exp2f(e0.x - M);
    if (e1.x != NEG_INF) L += e1.y * __builtin_amdgcn_exp2f(e1.x - M);
    L = wave_total_sum(L);
    const float *pacc = a.part_acc + (bh * S * g + h) * D + 2 * lane;  // split s at pacc[s * g * D]
    // wave w sums the splits w, w + 4, ... in order, 8 of them loaded at once
    float2 acc = make_float2(0.0f, 0.0f);
    for (int s0 = wave; s0 < S; s0 += 32) {
        float ms[8];
        float2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int s = s0 + 4 * u < S ? s0 + 4 * u : S - 1;  // past the end: a re-read, not added
            ms[u] = pml[s * g].x;
            v[u] = *reinterpret_cast<const float2 *>(pacc + (int64_t)s * g * D);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (s0 + 4 * u < S) {
                const float w = (L > 0.0f && ms[u] != NEG_INF) ? __builtin_amdgcn_exp2f(ms[u] - M) / L : 0.0f;
                acc.x += w * v[u].x;
                acc.y += w * v[u].y;
            }
        }
    }
    red[wave][lane] = acc;
    __syncthreads();
    const bool inconsistent = RANK && ranking_inconsistent(a, bh, head, h, kp, kq, wcnt, &bcast);
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
                    E += (double)pe[k] * f;
                }
                const float2 sa = psa[k];
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
            const float2 kv = pkv;
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
