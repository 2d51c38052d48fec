// kvq_decode_mfma.hip -- matrix-core split-K decode kernel (gfx950, wave64).
//
// "Runtime-Certified Bounded-Error Quantized Attention": Methodology 1 (INT8
// keys / INT4 values served from the compressed tier, FP16 originals on
// fallback), Methodology 2 (per-block bounds evaluated online from the block
// statistics and the query norm, before any tile is fetched), Key
// Contributions "Deterministic Recovery" (uncertified blocks read FP16).
//
// The G query heads of a KV group share every K/V tile, so per 64-token
// block Q.K^T is a (64 tokens x 128) x (128 x G) contraction and P.V a
// (128 x 64 tokens) x (64 x G) one.  Both run on v_mfma_f32_16x16x32_f16 with
// the heads on the N side (padded to 16); int8/int4 codes are widened to
// exact fp16 integers in registers and their scales are applied to the fp32
// scores (keys) and folded into the fp16 P operand per 32-channel group
// (values).  Only the widening, the online softmax and the operand packing
// run on the VALU, which keeps a G >= 2 group from being ALU-bound.
//
// Operand layout (A lane l: row l%16, k-slots [8*(l/16), +8); B lane l: column
// l%16, same k-slots; C lane l: column l%16, rows 4*(l/16) .. +3).  The
// contraction order inside one instruction is free, so the slots are chosen
// to make loads contiguous and to let the P operand of P.V come straight out
// of the Q.K^T accumulators without any cross-lane traffic:
//   Q.K^T subtile st = 2u+e (u, e in {0,1}) holds tokens
//       sigma(st, m) = 16*(m/4) + 8u + 4e + (m%4),  m = 0..15,
//   and its A lane (m, dg) holds key channels [32dg + 8s, +8) at step s, so
//   one lane reads 32 contiguous code bytes of one token row.
//   P.V step u of m-tile mt (channels 16mt..16mt+15) has A lane (m, kg)
//   holding the 8 tokens 16kg + 8u + [0, 8) of channel 16mt + m -- four bytes
//   of the channel-major nibble layout -- in the slot order (0,4),(1,5),(2,6),
//   (3,7) that the C registers of subtiles 2u and 2u+1 provide.
//
// Grid (splits, Hkv, B), 256 threads; each wave streams every fourth block of
// its workgroup's range with its own online softmax, prefetching the next
// block's quantized tiles into registers while it computes the current one;
// two such waves share each SIMD.
// Blocks with a fallback bit take a slower path that loads the FP16 tile
// (keys: contiguous 64 B per lane; values: per-token gathers).  Waves and
// splits are merged by log-sum-exp; the last workgroup of a (b, kvh) writes
// the fp16 output.
#include "kvq_decode_common.hpp"

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

namespace {

constexpr int NW = 4;  // waves per workgroup
constexpr float NEG_INF = -__builtin_huge_valf();

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

// 8 int4 codes (one dword, nibble k = token k) -> fp16 pairs (n_p, n_{p+4}),
// p = 0..3.  A two's-complement nibble n with bit 3 flipped is the offset code
// c + 8.  Masking the low nibbles of bytes 0 and 2 and xor-ing with
// 0x64086408 both flips that bit and sets the fp16 exponent of 1024, giving
// 1024 + (c + 8); minus 1032 leaves c.  The high nibbles, masked in place and
// xor-ed with 0x64806480, read 1024 + 16 (c + 8), which one packed FMA
// (x/16 - 72) turns into c.  Every step is exact in fp16.
__device__ __forceinline__ uint4 i4x8_to_h8(uint32_t x) {
    const uint32_t x8 = x >> 8;
    const half2_t lo_bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2_t hi_bias = {(_Float16)-72.0f, (_Float16)-72.0f};
    const half2_t a = __builtin_bit_cast(half2_t, (x & 0x000F000Fu) ^ 0x64086408u) + lo_bias;
    const half2_t b = __builtin_bit_cast(half2_t, (x & 0x00F000F0u) ^ 0x64806480u) * sixteenth + hi_bias;
    const half2_t c = __builtin_bit_cast(half2_t, (x8 & 0x000F000Fu) ^ 0x64086408u) + lo_bias;
    const half2_t d = __builtin_bit_cast(half2_t, (x8 & 0x00F000F0u) ^ 0x64806480u) * sixteenth + hi_bias;
    return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                      __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    const float2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Registers of one block's quantized tiles for one lane.
struct QTile {
    uint4 k[4][2];  // [subtile][half]: 16 code bytes of row sigma(st, m), channels 32dg + 16h ..
    uint2 v[8];     // [m-tile]: 8 nibble bytes, channel 16mt + m, tokens 16kg .. 16kg+15
    uint32_t ks;    // k_scale of token `lane` (fp16 bits)
    uint2 vs;       // 4 v_scales of token `lane`
};

__device__ __forceinline__ int sigma(int st, int m) {
    return 16 * (m >> 2) + 8 * (st >> 1) + 4 * (st & 1) + (m & 3);
}

// Per-lane byte offsets of the quantized tiles inside one block, computed once:
// keys: row sigma(0, m), channels 32dg (the other subtiles and halves add
// constants); values: channel m, tokens 16kg (m-tiles add 512 B).
struct LaneOffsets {
    uint32_t k, v;
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
    const int m = lane & 15, g4 = lane >> 4;
    return LaneOffsets{(uint32_t)(sigma(0, m) * D + 32 * g4), (uint32_t)(m * (BLK / 2) + 8 * g4)};
}

// Loads block `blk` of (b, kvh) into `t`: wave-uniform block bases plus the
// lane offsets plus compile-time constants (sigma(st, m) - sigma(0, m) =
// 8*(st/2) + 4*(st%2) rows).
__device__ __forceinline__ void load_qtile(QTile &t, const DecodeArgs &a, int64_t bh, int64_t blk,
                                           LaneOffsets lo, int lane) {
    const int64_t row0 = bh * a.cap + blk * BLK;
    const int8_t *kc = a.c.k_codes + row0 * D + lo.k;
    const uint8_t *vc = a.c.v_codes + (bh * a.nbc + blk) * (D * BLK / 2) + lo.v;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int rows = 8 * (st >> 1) + 4 * (st & 1);
        t.k[st][0] = *reinterpret_cast<const uint4 *>(kc + rows * D);
        t.k[st][1] = *reinterpret_cast<const uint4 *>(kc + rows * D + 16);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) t.v[mt] = *reinterpret_cast<const uint2 *>(vc + mt * 16 * (BLK / 2));
    t.ks = a.c.k_scales[row0 + lane];
    t.vs = *reinterpret_cast<const uint2 *>(a.c.v_scales + (row0 + lane) * 4);
}

}  // namespace

// Scores, online softmax and P.V of one block for one wave, from the block's
// quantized tiles in `t` (already in registers) or, for fallback parts, from
// the FP16 originals.  Scores are kept in log2 units (sm * log2(e) folded into
// the per-token key factor) so the softmax uses exp2.  State: m_run / l_run of
// head m (this lane's column; l as this lane's share of the 16-token groups)
// and the P.V accumulators.
struct WaveState {
    float m_run, l_run;
    float4_t acc[8];
};

__device__ __forceinline__ void process_block(const DecodeArgs &a, const QTile &t, int64_t bh,
                                              int64_t blk, uint32_t mk, const uint4 (&qb)[4],
                                              float sml2, float *ks_w, uint16_t (*vs_w)[BLK],
                                              WaveState &w, int lane) {
    const int m = lane & 15, g4 = lane >> 4;
    const int64_t row0 = bh * a.cap + blk * BLK;
    const int nvalid = (int)(a.length - blk * BLK < BLK ? a.length - blk * BLK : BLK);
    const bool lane_valid = lane < nvalid;  // token `lane` of the block

    // ---------------- Q.K^T: S^T[token][head] for the 4 subtiles
    float4_t sc[4];
    if (!(mk & 1u)) {
        ks_w[lane] = h2f(t.ks) * sml2;  // per-token factor k_scale * sm * log2(e)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            float4_t c = {0.f, 0.f, 0.f, 0.f};
            c = mfma(i8x8_to_h8(t.k[st][0].x, t.k[st][0].y), qb[0], c);
            c = mfma(i8x8_to_h8(t.k[st][0].z, t.k[st][0].w), qb[1], c);
            c = mfma(i8x8_to_h8(t.k[st][1].x, t.k[st][1].y), qb[2], c);
            c = mfma(i8x8_to_h8(t.k[st][1].z, t.k[st][1].w), qb[3], c);
            sc[st] = c;
        }
        wave_sync();
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const float4 f = *reinterpret_cast<const float4 *>(&ks_w[16 * g4 + 4 * st]);
            sc[st][0] *= f.x;
            sc[st][1] *= f.y;
            sc[st][2] *= f.z;
            sc[st][3] *= f.w;
        }
    } else {
        const uint16_t *kr = a.c.k16 + row0 * D + 32 * g4;  // channels [32dg, 32dg+32)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint4 *p = reinterpret_cast<const uint4 *>(kr + sigma(st, m) * D);
            float4_t c = {0.f, 0.f, 0.f, 0.f};
            c = mfma(p[0], qb[0], c);
            c = mfma(p[1], qb[1], c);
            c = mfma(p[2], qb[2], c);
            c = mfma(p[3], qb[3], c);
            sc[st] = c * sml2;
        }
    }

    // ---------------- online softmax of head m over this block
    const int tk0 = 16 * g4;  // this lane's 16 tokens: tk0 + 4st + i of the block
    float bmax = NEG_INF;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (tk0 + 4 * st + i >= nvalid) sc[st][i] = NEG_INF;
            bmax = fmaxf(bmax, sc[st][i]);
        }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(w.m_run, bmax);  // finite: the block holds a valid token
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_new);  // 0 on the first block
    float pv[4][4];
    float psum = 0.0f;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[st][i] = __builtin_amdgcn_exp2f(sc[st][i] - m_new);  // exp2(-inf) = 0
            psum += pv[st][i];
        }
    w.m_run = m_new;
    w.l_run = w.l_run * alpha + psum;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) w.acc[mt] *= alpha;
    }

    // ---------------- P.V
    // B operand (k-slot pairs): p of tokens (8u + q, 8u + 4 + q) of this lane's 16
    half2_t pp[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            pp[u][q] = __builtin_bit_cast(half2_t, pack_h2(pv[2 * u][q], pv[2 * u + 1][q]));
    if (!(mk & 2u)) {
        // value scales staged as [group][token], the tokens of each 8-run in
        // the slot order 0,4,1,5,2,6,3,7, so one 16-byte read yields the
        // (token q, token q+4) scale pairs; scales of tokens past `length`
        // are zeroed (their p is 0, and a stale scale must not make it NaN)
        {
            const uint2 sv = lane_valid ? t.vs : make_uint2(0u, 0u);
            const int r = lane & 7, slot = (lane & ~7) + ((r & 3) << 1) + (r >> 2);
            vs_w[0][slot] = (uint16_t)(sv.x & 0xFFFFu);
            vs_w[1][slot] = (uint16_t)(sv.x >> 16);
            vs_w[2][slot] = (uint16_t)(sv.y & 0xFFFFu);
            vs_w[3][slot] = (uint16_t)(sv.y >> 16);
        }
        wave_sync();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const uint4 sp = *reinterpret_cast<const uint4 *>(&vs_w[gg][16 * g4 + 8 * u]);
                uint4 bop;  // p * s_v in fp16: one rounding of p, one of the product
                bop.x = __builtin_bit_cast(uint32_t, pp[u][0] * __builtin_bit_cast(half2_t, sp.x));
                bop.y = __builtin_bit_cast(uint32_t, pp[u][1] * __builtin_bit_cast(half2_t, sp.y));
                bop.z = __builtin_bit_cast(uint32_t, pp[u][2] * __builtin_bit_cast(half2_t, sp.z));
                bop.w = __builtin_bit_cast(uint32_t, pp[u][3] * __builtin_bit_cast(half2_t, sp.w));
                w.acc[2 * gg] = mfma(i4x8_to_h8(u ? t.v[2 * gg].y : t.v[2 * gg].x), bop, w.acc[2 * gg]);
                w.acc[2 * gg + 1] =
                    mfma(i4x8_to_h8(u ? t.v[2 * gg + 1].y : t.v[2 * gg + 1].x), bop, w.acc[2 * gg + 1]);
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint4 bop = make_uint4(__builtin_bit_cast(uint32_t, pp[u][0]), __builtin_bit_cast(uint32_t, pp[u][1]),
                                         __builtin_bit_cast(uint32_t, pp[u][2]), __builtin_bit_cast(uint32_t, pp[u][3]));
            const int tb = 16 * g4 + 8 * u;  // tokens tb + q and tb + 4 + q
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const uint16_t *vcol = a.c.v16 + row0 * D + 16 * mt + m;
                uint32_t r[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // rows past `length` are still inside the block's storage:
                    // load them unconditionally, then zero them (a stale value
                    // could be NaN, and 0 * NaN would reach the accumulator)
                    const int ta = tb + q, tb2 = tb + 4 + q;
                    const uint32_t lo = vcol[ta * D], hi = vcol[tb2 * D];
                    r[q] = ((ta < nvalid) ? lo : 0u) | (((tb2 < nvalid) ? hi : 0u) << 16);
                }
                w.acc[mt] = mfma(make_uint4(r[0], r[1], r[2], r[3]), bop, w.acc[mt]);
            }
        }
    }
}

// Two waves per SIMD (at most 256 registers each): one wave's VALU and matrix
// work overlaps the other's memory latency.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_mfma_kernel(
    DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[16][D];
    __shared__ float qn_lds[16];
    __shared__ uint8_t mask_lds[MAX_BPS];
    __shared__ __attribute__((aligned(16))) float ks_lds[NW][BLK];
    __shared__ __attribute__((aligned(16))) uint16_t vs_lds[NW][4][BLK];
    __shared__ __attribute__((aligned(16))) float wacc[NW * 16 * D];
    __shared__ float wm[NW][16], wl[NW][16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept scalar
    const int m = lane & 15, g4 = lane >> 4;  // MFMA row/column index and k-group
    const int split = blockIdx.x;
    const int64_t kvh = blockIdx.y, b = blockIdx.z;
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g;
    const int64_t blk0 = (int64_t)split * a.bps;
    const int64_t blk1 = blk0 + a.bps < a.nb ? blk0 + a.bps : a.nb;

    const float qn = load_q_and_norm(a.q, b * a.hq + kvh * g, g, q_lds, qn_lds);
    compute_masks(a, bh, blk0, blk1, qn, mask_lds);

    // B operands of Q.K^T: lane (n = head, dg) holds q[n][32dg + 8s .. +8] at step s
    uint4 qb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = *reinterpret_cast<const uint4 *>(&q_lds[m][32 * g4 + 8 * s]);

    const float sml2 = a.sm * 1.4426950408889634f;  // scores in log2 units
    WaveState ws;
    ws.m_run = NEG_INF;
    ws.l_run = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) ws.acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};

    // Two register tiles in ping-pong: while one block is processed from one
    // tile, the loads of the wave's next block land in the other.  The next
    // block index is clamped to a valid block at the end of the range so the
    // load sequence stays uniform and the compiler can count it exactly.
    QTile t0, t1;
    const LaneOffsets lo = lane_offsets(lane);
    int64_t blk = blk0 + wave;
    if (blk < blk1) {
        load_qtile(t0, a, bh, blk, lo, lane);
        for (;;) {
            int64_t nb = blk + NW < blk1 ? blk + NW : blk;
            load_qtile(t1, a, bh, nb, lo, lane);
            process_block(a, t0, bh, blk, __builtin_amdgcn_readfirstlane(mask_lds[blk - blk0]), qb, sml2,
                          ks_lds[wave], vs_lds[wave], ws, lane);
            blk += NW;
            if (blk >= blk1) break;
            nb = blk + NW < blk1 ? blk + NW : blk;
            load_qtile(t0, a, bh, nb, lo, lane);
            process_block(a, t1, bh, blk, __builtin_amdgcn_readfirstlane(mask_lds[blk - blk0]), qb, sml2,
                          ks_lds[wave], vs_lds[wave], ws, lane);
            blk += NW;
            if (blk >= blk1) break;
        }
    }

    // ---------------- merge waves, then splits
    // lane (n = m, r = g4) holds O^T[16mt + 4r + i][n] and a share of l
    float l_run = ws.l_run;
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (m < g) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) wacc[(wave * 16 + m) * D + 16 * mt + 4 * g4 + i] = ws.acc[mt][i];
        if (g4 == 0) {
            wm[wave][m] = ws.m_run;
            wl[wave][m] = l_run;
        }
    }
    __syncthreads();
    write_partial(a, bh, split, NW, 16, wm, wl, wacc);
}

bool mfma_supports(int g) { return g >= 1 && g <= 16; }

hipError_t launch_decode_mfma(const DecodeArgs &a, int batch, hipStream_t s) {
    dim3 grid((unsigned)a.splits, (unsigned)a.hkv, (unsigned)batch);
    hipLaunchKernelGGL(decode_mfma_kernel, grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_merge(a, batch, s);
}

}  // namespace kvq
