// kvq_decode_mfma.hip -- matrix-core split-K decode kernel (gfx950, wave64).
//
// "Runtime-Certified Bounded-Error Quantized Attention": Methodology 1 (INT8
// keys / INT4 values served from the compressed tier, FP16 originals on
// fallback), Methodology 2 (per-block bounds evaluated online from the block
// statistics and the query norm, before any tile is fetched), Key
// Contributions "Deterministic Recovery" (uncertified blocks read FP16).
//
// The G query heads of a KV group share every K/V tile, so Q.K^T over a tile
// is a (tokens x 128) x (128 x G) contraction and P.V a (128 x tokens) x
// (tokens x G) one.  Both run on v_mfma_f32_16x16x32_f16 with the heads on the
// N side (padded to 16); int8/int4 codes are widened to exact fp16 integers in
// registers and their scales are applied to the fp32 scores (keys) and folded
// into the fp16 P operand per 32-channel group (values).  Only the widening,
// the online softmax and the operand packing run on the VALU.
//
// Operand layout (A lane l: row l%16, k-slots [8*(l/16), +8); B lane l: column
// l%16, same k-slots; C lane l: column l%16, rows 4*(l/16) .. +3).  The
// contraction order inside one instruction is free, so the slots are chosen
// to make loads contiguous and to let the P operand of P.V come straight out
// of the Q.K^T accumulators without any cross-lane traffic.  A 64-token block
// is streamed as two 32-token halves u; in half u,
//   Q.K^T subtile e (e in {0,1}) holds tokens
//       32u + 8*(m/4) + 4e + (m%4),  m = 0..15,
//   and its A lane (m, dg) holds key channels [32dg + 8s, +8) at step s (32
//   contiguous code bytes of one token row);
//   P.V m-tile mt (channels 16mt..16mt+15) has A lane (m, kg) holding the 8
//   tokens 32u + 8kg + [0, 8) of channel 16mt + m -- four bytes of the
//   channel-major nibble layout -- in the slot order (0,4),(1,5),(2,6),(3,7)
//   that the C registers of subtiles 0 and 1 provide.
//
// Grid (splits, Hkv, B), NW = 8 waves, one workgroup per CU (two waves per
// SIMD: one wave's VALU and matrix work hides the other's latencies).  Two
// variants.  The general one (decode_group): after the fallback masks of its
// (b, kvh) are known, a workgroup takes an equal share of the group's work in
// steps, in block order, lists the blocks the share touches, and its waves
// claim the share's steps one at a time from an LDS counter at issue time, so
// that the waves of a workgroup finish together however the fallback blocks
// fall.  The streaming one (decode_group_stream, up to STREAM_MAX_NB blocks,
// no certificate or promotions): the first half-blocks of each split's home
// range are copied before the masks are known, the rest of the group's work
// is cut into equal ranges of a step pool, and blocks are found from 64-block
// windows instead of a table.  Each wave streams its steps
// through its own 3-stage LDS ring: the quantized data of a half (4 KB key
// codes, 2 KB value codes, key and value scales) is copied HBM -> LDS by
// global_load_lds (no registers held while in flight), so two halves are in
// flight while the wave computes a third.  The copy places every chunk where
// the MFMA lane that consumes it reads it back with a lane-linear ds_read.
// A block with a fallback bit is streamed through the same ring as 16-token
// steps (keys or values alone falling back) or 8-token steps (both), whose
// FP16 rows fit a stage; the step's tokens sit in the rows of the MFMA tiles
// that a 32-token half gives to them, and the other rows are masked.  Every
// step, of either kind, issues exactly 8 copy instructions, so the waits
// stay compile-time constants, and no global load is ever waited on while
// later steps are in flight.
// Waves are merged by log-sum-exp in LDS; the splits of a group are merged
// by the last of its workgroups to finish, in the same launch (the
// certificate path merges in a second kernel).
#include "kvq_decode_common.hpp"
#include "kvq_mfma.hpp"
#include "kvq_quant_row.hpp"

namespace kvq {

namespace {

constexpr int NW = 8;  // waves per workgroup (one workgroup per CU, NW/4 waves per SIMD)
constexpr float NEG_INF = -__builtin_huge_valf();

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

// 4 int4 codes (the low 16 bits, nibble k = token k) -> fp16 (n0, n1),
// (n2, n3): each nibble moved under the low half or the high half of a dword
// and widened as the low nibbles are above.  Exact.
__device__ __forceinline__ uint2 i4x4_to_h4(uint32_t x) {
    const half2_t lo_bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const uint32_t a = (x & 0xFu) | ((x & 0xF0u) << 12), b = ((x >> 8) & 0xFu) | ((x & 0xF000u) << 4);
    const half2_t ha = __builtin_bit_cast(half2_t, a ^ 0x64086408u) + lo_bias;
    const half2_t hb = __builtin_bit_cast(half2_t, b ^ 0x64086408u) + lo_bias;
    return make_uint2(__builtin_bit_cast(uint32_t, ha), __builtin_bit_cast(uint32_t, hb));
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    const float2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
}

// Max over the four 16-lane rows (lanes l, l^16, l^32, l^48), with the
// row-swap permutes (no LDS round trip): after a swap of a value with itself
// the two results hold, in every lane, the lane's value and its partner's.
__device__ __forceinline__ float max_across_rows(float v) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Sum over the four 16-lane rows, with the same row-swap permutes.
__device__ __forceinline__ float sum_across_rows(float v) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// The sum of a double with its value in lane l ^ 32 (X32) or l ^ 16, by the
// row-swap permutes: the swap of each half with itself returns the lane's own
// word and its partner's, and addition is commutative.
template <bool X32>
__device__ __forceinline__ double add_partner_d(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
    const auto rl = X32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                        : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto rh = X32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                        : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const double d0 = __longlong_as_double((long long)(((uint64_t)rh[0] << 32) | rl[0]));
    const double d1 = __longlong_as_double((long long)(((uint64_t)rh[1] << 32) | rl[1]));
    return d0 + d1;
}

// Unsigned max over the wave, in every lane (DPP within the rows, then the
// row-swap permutes).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = row16_max_u32(v);
    const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = umax(r16[0], r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return umax(r32[0], r32[1]);
}

// Row (token) of the half held by MFMA row m of Q.K^T subtile e.
__device__ __forceinline__ int half_row(int e, int m) { return 8 * (m >> 2) + 4 * e + (m & 3); }

// One stage of a wave's LDS ring: the quantized data of one 32-token half u
// of a block.
//   [0, 4096)     key codes, 4 chunks of 1 KB; chunk 2e+h, lane l (m, dg):
//                 row half_row(e, m), code bytes [32dg + 16h, +16)
//   [4096, 6144)  value codes, 2 chunks of 1 KB; chunk j, lane l: channel
//                 64j + l, bytes [16u, +16) (tokens 32u .. 32u+31)
//   [6144, 6400)  key scales, one dword per token of the half (fp16 in the
//                 low half; lanes 32..63 repeat tokens 0..31)
//   [6400, 6656)  value scales: dword t < 32 = groups (0,1) of token t,
//                 dword 32 + t = groups (2,3)
constexpr int ST_K = 0, ST_V = 4096, ST_KS = 6144, ST_VS = 6400, ST_BYTES = 6656;
// A fallback step uses the same stage.  Keys alone falling back: tokens
// 16j .. 16j+15 of the block (half u = j/2, positions 16(j%2) .. +15), with
//   keys   [0, 4096): chunk c (1 KB), lane (s, dg, r) = lane 16s + 4dg + r:
//          token 4c + r of the step, channels [32dg + 8s, +8);
// and the value codes and scales of half u as for a certified half.  Values
// alone falling back: the same 16 tokens, with
//   keys   [0, 2048): the code bytes of the MFMA rows m of the step
//          (8(j%2) <= m < 8(j%2) + 8) packed: chunk k (1 KB), slot
//          32h' + 8dg + (m & 7) holds what a certified half keeps in chunk
//          2k + h', lane m + 16dg;
//   key scales as for a certified half (all 32 of half u);
//   values [2048, 6144): the step's 16 rows, row-major [16][128].
// Both falling back: tokens 8j .. 8j+7 (half u = j/4, positions 8(j%4) ..
// +7), with
//   keys   [0, 2048): chunk e as for keys alone, token 4e + r of the step;
//   values [2048, 4096): the step's 8 rows, row-major [8][128].
// The copies are padded up to 8 with dwords of the block's statistics into a
// region the step leaves unused.
constexpr int FB_K16 = 0, FB_V16 = 2048;
constexpr int NSTAGE = 3;  // LDS stages per wave
// the split merge in the launch reuses the ring for its (m, l) tables
static_assert(8 * 16 * (MAX_SPLITS + 1) <= NW * NSTAGE * ST_BYTES, "fold_merge needs 8 (S + 1) G bytes of LDS");
// With three stages the copies of step k+2 are issued in the middle of step k;
// with two, those of step k+1 at the start of step k.
constexpr bool EARLY_ISSUE = NSTAGE == 2;
constexpr int DMA_PER_STEP = 8;  // copy instructions of every step (half or fallback step)

// Copies of global memory into LDS that bypass the registers.  M0 holds the
// wave-uniform LDS destination; lane l writes its bytes at M0 + l*size (16 B
// per lane for dwordx4; a zero-extended dword per lane for dword and ushort).
// The source is a wave-uniform base address (scalar registers) plus this
// lane's 32-bit byte offset.  The copy is issued in inline assembly so that
// its completion is tracked here, with s_waitcnt vmcnt, rather than by the
// compiler's conservative wait before every LDS read.  The preceding
// lgkmcnt(0) retires any LDS read of the stage being refilled.
__device__ __forceinline__ void dma16(uint32_t lds, const void *base, uint32_t off) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds), "v"(off), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, const void *base, uint32_t off) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(lds), "v"(off), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma2(uint32_t lds, const void *base, uint32_t off) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, %2"
                 :: "s"(lds), "v"(off), "s"(base) : "memory", "m0");
}

// Waits until at most N of this wave's memory loads are outstanding (loads
// complete in issue order).  The "memory" clobber keeps LDS reads of the
// stage below the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// The lane index, opaque to the optimizer: the per-lane copy offsets derived
// from it are recomputed at each issue (a few VALU operations) instead of
// being hoisted out of the stream loop, where they would hold registers.
__device__ __forceinline__ int opaque_lane(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}

// Copies of the code parts of half u: keys (4 chunks + scales, 5 copies) and
// values (2 chunks + scales, 3 copies).  row0: first token of the block.
__device__ __forceinline__ void issue_keys(const DecodeArgs &a, int64_t row0, int u, uint32_t stage, int lane) {
    const int m = lane & 15, dg = lane >> 4, l32 = lane & 31;
    const int8_t *kc = a.c.k_codes + (row0 + 32 * u) * D;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            dma16(stage + ST_K + (2 * e + h) * 1024, kc, (uint32_t)(half_row(e, m) * D + 32 * dg + 16 * h));
    dma2(stage + ST_KS, a.c.k_scales + row0 + 32 * u, (uint32_t)(2 * l32));
}
__device__ __forceinline__ void issue_values(const DecodeArgs &a, int64_t bh, int64_t blk, int64_t row0, int u,
                                             uint32_t stage, int lane) {
    const int l32 = lane & 31;
    const uint8_t *vc = a.c.v_codes + (bh * a.nbc + blk) * (D * BLK / 2) + 16 * u;
    dma16(stage + ST_V, vc, (uint32_t)(lane * (BLK / 2)));
    dma16(stage + ST_V + 1024, vc, (uint32_t)((64 + lane) * (BLK / 2)));
    dma4(stage + ST_VS, a.c.v_scales + (row0 + 32 * u) * 4, (uint32_t)(2 * (4 * l32 + 2 * (lane >> 5))));
}

// Issues the copies of half u of block `blk` of (b, kvh) into the stage at
// LDS byte address `stage` (wave-uniform).  Every source address lies inside
// the block.
__device__ __forceinline__ void issue_half(const DecodeArgs &a, int64_t bh, int64_t blk, int u,
                                           uint32_t stage, int lane_) {
    const int lane = opaque_lane(lane_);
    const int64_t row0 = bh * a.cap + blk * BLK;
    issue_keys(a, row0, u, stage, lane);
    issue_values(a, bh, blk, row0, u, stage, lane);
}

// Steps of a block by its fallback mask: two certified halves, four 16-token
// steps when only the keys or only the values fall back, eight 8-token steps
// when both do.
__device__ __forceinline__ int steps_of(uint32_t mk) { return mk == 0u ? 2 : (mk == 3u ? 8 : 4); }

// Issues the 8 copies of fallback step j of block `blk` with fallback mask
// mk (nonzero): tokens 16j .. 16j+15 when only the keys fall back (FP16 key
// rows in the four 1 KB chunks: chunk c, lane (r, dg, st) holds token 4c + r,
// channels 32dg + 8st .. +8; the value codes and scales of half j >> 1) or
// only the values (the packed key codes and the key scales of half j >> 1,
// FP16 value rows), tokens 8j .. 8j+7 otherwise.  Every source address lies
// inside the block.
__device__ __forceinline__ void issue_fb(const DecodeArgs &a, int64_t bh, int64_t blk, int j,
                                         uint32_t mk, uint32_t stage, int lane_) {
    const int lane = opaque_lane(lane_);
    const int64_t row0 = bh * a.cap + blk * BLK;  // first token of the block
    const float *pad = a.c.k_err + bh * a.nbc + blk;
    if (mk == 1u) {
        const int64_t rk = row0 + 16 * j;
        const int r = lane & 3, dg = (lane >> 2) & 3, st = lane >> 4;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            dma16(stage + FB_K16 + 1024 * c, a.c.k16 + rk * D, (uint32_t)(2 * ((4 * c + r) * D + 32 * dg + 8 * st)));
        issue_values(a, bh, blk, row0, j >> 1, stage, lane);
        dma4(stage + ST_KS, pad, 0u);  // padding into the unused key-scale region
        return;
    }
    if (mk == 2u) {
        const int u = j >> 1, hh = j & 1;
        const int8_t *kc = a.c.k_codes + (row0 + 32 * u) * D;
        const int ci = lane & 31, dg = ci >> 3, mm = 8 * hh + (ci & 7);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int jj = 2 * k + (lane >> 5), e = jj >> 1, h = jj & 1;
            dma16(stage + ST_K + 1024 * k, kc, (uint32_t)(half_row(e, mm) * D + 32 * dg + 16 * h));
        }
        dma2(stage + ST_KS, a.c.k_scales + row0 + 32 * u, (uint32_t)(2 * (lane & 31)));
        const int64_t rv = row0 + 16 * j;
#pragma unroll
        for (int d = 0; d < 4; ++d)
            dma16(stage + FB_V16 + 1024 * d, a.c.v16 + rv * D,
                  (uint32_t)(2 * ((4 * d + (lane >> 4)) * D + 8 * (lane & 15))));
        dma4(stage + ST_VS, pad, 0u);  // padding into the unused value-scale region
        return;
    }
    // both parts fall back: 8 tokens of FP16 keys and values
    const int64_t rs = row0 + 8 * j;  // first token of the step
    const int r = lane & 3, dg = (lane >> 2) & 3, st = lane >> 4;
#pragma unroll
    for (int e = 0; e < 2; ++e)
        dma16(stage + FB_K16 + 1024 * e, a.c.k16 + rs * D, (uint32_t)(2 * ((4 * e + r) * D + 32 * dg + 8 * st)));
#pragma unroll
    for (int d = 0; d < 2; ++d)
        dma16(stage + FB_V16 + 1024 * d, a.c.v16 + rs * D,
              (uint32_t)(2 * ((4 * d + (lane >> 4)) * D + 8 * (lane & 15))));
    // padding: 4 copies into the unused region past the values
#pragma unroll
    for (int i = 0; i < 4; ++i) dma4(stage + 4096 + 256 * i, pad, 0u);
}

// Scores, online softmax and P.V of one step for one wave, from its stage in
// LDS.  The step covers positions [p_lo, p_hi) of a 32-token half: a whole
// certified half (mk = 0, [0, valid tokens)), or the 8 positions of a fallback
// step, whose parts with a bit in mk come as FP16 rows.  Scores are kept in
// log2 units (sm * log2(e) folded into the per-token key factor) so the
// softmax uses exp2.  State: m_run / l_run of head m (this lane's column; l as
// this lane's share of the 8-position groups) and the P.V accumulators.
// RANK: a step of FP16 keys also writes, per head, its largest score and the
// sum of exp2(score - that) over its valid tokens to rank_out[head * rank_hs]
// (the FP16 block masses of the ranking check; each head's statistics slots
// are contiguous, rank_hs apart).
struct WaveState {
    float m_run, l_run;
    float4_t acc[8];
    // certificate only: the attention mass times the block's value error
    // (online, like l_run), the largest value scale of a value-certified
    // token and the largest |v| of a value-fallback token (fp16 bits)
    float e_run;
    uint32_t smax, amax;
};

// A 16-token step whose keys alone fall back (mask 1), compact: tokens
// p_lo .. p_hi-1 of the half (p_lo = 0 or 16) are rows 0 .. 15 of one Q.K^T
// subtile (token r from chunk r/4, lane slot 16st + 4dg + r%4 of the stage),
// so result lane (head m, g4) holds tokens 4 g4 .. +3 of the step, and those
// same 4 tokens are that lane's k-slots of a v_mfma_f32_16x16x16_f16 P.V:
// A = the value codes of channel 16mt + m for them (4 nibbles at byte
// p_lo/2 + 2 g4 of the channel's 16), B = p * s_v in fp16 (one rounding of p,
// one of the product, as for a certified half).  Same online softmax,
// certificate parts and ranking statistics as process_step.
template <bool CERT, bool RANK, typename Mid>
__device__ __forceinline__ void process_key16(const uint8_t *stage, int p_lo, int p_hi, const uint4 (&qb)[4],
                                              float sml2, WaveState &w, int lane, float eta, float2 *rank_out,
                                              int64_t rank_hs, int g, Mid &&mid) {
    const int m = lane & 15, g4 = lane >> 4;
    float4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
        c = mfma(*reinterpret_cast<const uint4 *>(stage + FB_K16 + 1024 * (m >> 2) + 16 * (16 * st + 4 * g4 + (m & 3))),
                 qb[st], c);
    mid();
    const int nv = p_hi - p_lo;  // valid tokens of the step
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = (4 * g4 + i < nv) ? c[i] * sml2 : NEG_INF;
    float bmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bmax = max_across_rows(bmax);
    if (RANK && rank_out) {
        float es = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) es += (sc[i] == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(sc[i] - bmax);
        es = sum_across_rows(es);
        if (g4 == 0 && m < g) {
            rank_out[m * rank_hs] = make_float2(bmax, es);
            rank_out[m * rank_hs + 1] = make_float2(NEG_INF, 0.0f);  // a 16-token step fills two 8-token slots
        }
    }
    const float m_new = fmaxf(w.m_run, bmax);
    const float m_use = (m_new == NEG_INF) ? 0.0f : m_new;  // as in process_step
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_use);
    float pv[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sc[i] - m_use);
        psum += pv[i];
    }
    w.m_run = m_new;
    w.l_run = w.l_run * alpha + psum;
    if (CERT) w.e_run = w.e_run * alpha + psum * eta;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) w.acc[mt] *= alpha;
    }
    // P.V over the lane's 4 tokens
    const half2_t p01 = __builtin_bit_cast(half2_t, pack_h2(pv[0], pv[1]));
    const half2_t p23 = __builtin_bit_cast(half2_t, pack_h2(pv[2], pv[3]));
    const int tp = p_lo + 4 * g4;  // the lane's first token, as a position of the half
    uint16_t vn[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
        vn[mt] = *reinterpret_cast<const uint16_t *>(stage + ST_V + (mt >> 2) * 1024 + 16 * (16 * (mt & 3) + m) +
                                                     (tp >> 1));
    // value scales of the 4 tokens: dwords of groups (0,1) and (2,3); tokens
    // outside the step carry other tokens' scales (stale past `length`): 0
    const uint4 s01 = *reinterpret_cast<const uint4 *>(stage + ST_VS + 4 * tp);
    const uint4 s23 = *reinterpret_cast<const uint4 *>(stage + ST_VS + 128 + 4 * tp);
    uint32_t a01[4] = {s01.x, s01.y, s01.z, s01.w}, a23[4] = {s23.x, s23.y, s23.z, s23.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (4 * g4 + i >= nv) a01[i] = a23[i] = 0u;
    if (CERT) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w.smax = umax(w.smax, umax(umax(a01[i] & 0xFFFFu, a01[i] >> 16), umax(a23[i] & 0xFFFFu, a23[i] >> 16)));
    }
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
        // (s of token 0, token 1) and (token 2, token 3) for group gg
        const uint32_t *sg = gg < 2 ? a01 : a23;
        const uint32_t sel = (gg & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t s01g = __builtin_amdgcn_perm(sg[1], sg[0], sel), s23g = __builtin_amdgcn_perm(sg[3], sg[2], sel);
        const uint2 bop = make_uint2(__builtin_bit_cast(uint32_t, p01 * __builtin_bit_cast(half2_t, s01g)),
                                     __builtin_bit_cast(uint32_t, p23 * __builtin_bit_cast(half2_t, s23g)));
        w.acc[2 * gg] = mfma16(i4x4_to_h4(vn[2 * gg]), bop, w.acc[2 * gg]);
        w.acc[2 * gg + 1] = mfma16(i4x4_to_h4(vn[2 * gg + 1]), bop, w.acc[2 * gg + 1]);
    }
}

// ROT: the key codes are those of Hadamard-rotated keys, scored against the
// rotated query (qrh + qrl, its fp16 high and low parts); FP16 key rows use
// the query itself.  K16: key-only fallback steps take the compact path
// (process_key16).
template <bool CERT, bool RANK, bool ROT, bool K16, typename Mid>
__device__ __forceinline__ void process_step(const uint8_t *stage, uint32_t mk, int p_lo, int p_hi,
                                             const uint4 (&qb)[4], const uint4 (&qrh)[4], const uint4 (&qrl)[4],
                                             float sml2, WaveState &w, int lane, float eta, float2 *rank_out,
                                             int64_t rank_hs,
                                             int g, Mid &&mid) {
    if (K16 && mk == 1u) {
        process_key16<CERT, RANK>(stage, p_lo, p_hi, qb, sml2, w, lane, eta, rank_out, rank_hs, g, mid);
        return;
    }
    const int m = lane & 15, g4 = lane >> 4;
    const bool partial = p_lo > 0 || p_hi < 32;  // wave-uniform

    // ---------------- Q.K^T: S^T[position][head] for the 2 subtiles
    float4_t sc[2];
    if (mk & 1u) {
        // FP16 key rows.  8-token step (both parts FP16): subtile e row r
        // holds token 4e + (r & 3) of the step (the rows of group p_lo/8 are
        // the step's positions; others masked).  16-token step (keys only):
        // row r of subtile e holds token 8((r >> 2) & 1) + 4e + (r & 3), from
        // chunk 2((r >> 2) & 1) + e, so that result row 4g + i is position
        // 8g + 4e + i of the half for g = p_lo/8, p_lo/8 + 1.
        const int hsel = (mk & 2u) ? 0 : ((m >> 2) & 1);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                c = mfma(*reinterpret_cast<const uint4 *>(stage + FB_K16 + 1024 * (2 * hsel + e) +
                                                          16 * (16 * st + 4 * g4 + (m & 3))),
                         qb[st], c);
            sc[e] = c * sml2;
        }
    } else {
        // a value-fallback step keeps the code bytes of its 8 MFMA rows packed
        // (the other rows read a copy of them and are masked below)
        uint4 kt[4];
        const bool packed = mk == 2u;
        const int koff = packed ? 16 * ((m & 7) + 8 * g4) : 16 * lane;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            kt[j] = *reinterpret_cast<const uint4 *>(stage + ST_K + (packed ? 1024 * (j >> 1) + 512 * (j & 1) : 1024 * j) +
                                                     koff);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float4_t c = {0.f, 0.f, 0.f, 0.f};
            const uint4 a0 = i8x8_to_h8(kt[2 * e].x, kt[2 * e].y), a1 = i8x8_to_h8(kt[2 * e].z, kt[2 * e].w);
            const uint4 a2 = i8x8_to_h8(kt[2 * e + 1].x, kt[2 * e + 1].y);
            const uint4 a3 = i8x8_to_h8(kt[2 * e + 1].z, kt[2 * e + 1].w);
            if (ROT) {
                c = mfma(a0, qrh[0], c);
                c = mfma(a1, qrh[1], c);
                c = mfma(a2, qrh[2], c);
                c = mfma(a3, qrh[3], c);
                c = mfma(a0, qrl[0], c);
                c = mfma(a1, qrl[1], c);
                c = mfma(a2, qrl[2], c);
                c = mfma(a3, qrl[3], c);
            } else {
                c = mfma(a0, qb[0], c);
                c = mfma(a1, qb[1], c);
                c = mfma(a2, qb[2], c);
                c = mfma(a3, qb[3], c);
            }
            sc[e] = c;
        }
        // key scales of positions 8*g4 + 4e + i (one dword per token)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint4 f = *reinterpret_cast<const uint4 *>(stage + ST_KS + 4 * (8 * g4 + 4 * e));
            sc[e][0] *= h2f(f.x & 0xFFFFu) * sml2;
            sc[e][1] *= h2f(f.y & 0xFFFFu) * sml2;
            sc[e][2] *= h2f(f.z & 0xFFFFu) * sml2;
            sc[e][3] *= h2f(f.w & 0xFFFFu) * sml2;
        }
    }

    mid();

    // ---------------- online softmax of head m over this step
    const int tk0 = 8 * g4;  // this lane's 8 positions: tk0 + 4e + i
    if (partial) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tk0 + 4 * e + i < p_lo || tk0 + 4 * e + i >= p_hi) sc[e][i] = NEG_INF;
    }
    float bmax = NEG_INF;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, sc[e][i]);
    bmax = max_across_rows(bmax);
    if (RANK && (mk & 1u) && rank_out) {
        float es = 0.0f;
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) es += (sc[e][i] == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(sc[e][i] - bmax);
        es = sum_across_rows(es);
        if (g4 == 0 && m < g) {
            rank_out[m * rank_hs] = make_float2(bmax, es);
            // a 16-token step fills two 8-token statistics slots
            if (!(mk & 2u)) rank_out[m * rank_hs + 1] = make_float2(NEG_INF, 0.0f);
        }
    }
    const float m_new = fmaxf(w.m_run, bmax);
    // exp2(-inf) is 0: against a finite reference a -inf score weighs 0, and
    // a -inf running max scales its sum and accumulators (still 0) by 0.  A
    // step with no finite score so far leaves m_new at -inf; 0 stands in.
    const float m_use = (m_new == NEG_INF) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_use);
    float pv[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[e][i] = __builtin_amdgcn_exp2f(sc[e][i] - m_use);
            psum += pv[e][i];
        }
    w.m_run = m_new;
    w.l_run = w.l_run * alpha + psum;
    if (CERT) w.e_run = w.e_run * alpha + psum * eta;  // eta: the block's value error, 0 on value fallback
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) w.acc[mt] *= alpha;
    }

    // ---------------- P.V
    // B operand (k-slot pairs): p of positions (8kg + q, 8kg + 4 + q)
    half2_t pp[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pp[q] = __builtin_bit_cast(half2_t, pack_h2(pv[0][q], pv[1][q]));
    if (mk & 2u) {
        // FP16 value rows: lane (m, kg) with its 8 positions 8kg .. 8kg+7
        // inside the step gathers channel 16mt + m of them (rows from
        // 8kg - p_lo); other lanes and tokens past p_hi give 0 (a stale row
        // could hold NaN, and 0 * NaN would reach the accumulator).  All 64
        // reads first, then the selects, so that the reads share one wait.
        const uint4 bop = make_uint4(__builtin_bit_cast(uint32_t, pp[0]), __builtin_bit_cast(uint32_t, pp[1]),
                                     __builtin_bit_cast(uint32_t, pp[2]), __builtin_bit_cast(uint32_t, pp[3]));
        const bool act = tk0 >= p_lo && tk0 < p_hi;
        const int rb = act ? tk0 - p_lo : 0;
        uint32_t v[8][8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const uint16_t *col = reinterpret_cast<const uint16_t *>(stage + FB_V16) + rb * D + 16 * mt + m;
#pragma unroll
            for (int t = 0; t < 8; ++t) v[mt][t] = col[t * D];
        }
        uint32_t keep = 0;  // bit t: token t of the step is valid in this lane
#pragma unroll
        for (int t = 0; t < 8; ++t) keep |= (act && tk0 + t < p_hi) ? (1u << t) : 0u;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            uint32_t r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                r[q] = ((keep >> q) & 1u ? v[mt][q] : 0u) | (((keep >> (q + 4)) & 1u ? v[mt][q + 4] : 0u) << 16);
            w.acc[mt] = mfma(make_uint4(r[0], r[1], r[2], r[3]), bop, w.acc[mt]);
            if (CERT) {
                // |v| of the step's valid values (fp16 bits without the sign
                // order like the magnitudes; NaN above +Inf)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w.amax = umax(w.amax, umax(r[q] & 0x7FFFu, (r[q] >> 16) & 0x7FFFu));
            }
        }
    } else {
        // value codes of channel 16mt + m, positions 8kg .. 8kg+7
        uint32_t vt[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            vt[mt] = *reinterpret_cast<const uint32_t *>(stage + ST_V + (mt >> 2) * 1024 + 16 * (16 * (mt & 3) + m) +
                                                         4 * g4);
        // scales of positions 8kg + [0, 8): dwords of groups (0,1) and (2,3)
        const uint4 a01 = *reinterpret_cast<const uint4 *>(stage + ST_VS + 4 * tk0);
        const uint4 b01 = *reinterpret_cast<const uint4 *>(stage + ST_VS + 4 * (tk0 + 4));
        const uint4 a23 = *reinterpret_cast<const uint4 *>(stage + ST_VS + 128 + 4 * tk0);
        const uint4 b23 = *reinterpret_cast<const uint4 *>(stage + ST_VS + 128 + 4 * (tk0 + 4));
        uint32_t lo_a[4] = {a01.x, a01.y, a01.z, a01.w}, lo_b[4] = {b01.x, b01.y, b01.z, b01.w};
        uint32_t hi_a[4] = {a23.x, a23.y, a23.z, a23.w}, hi_b[4] = {b23.x, b23.y, b23.z, b23.w};
        if (partial) {
            // positions outside the step carry scales of other tokens (stale
            // past `length`): zero them (their p is 0, and 0 * NaN would
            // reach the accumulator)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (tk0 + q < p_lo || tk0 + q >= p_hi) lo_a[q] = hi_a[q] = 0u;
                if (tk0 + 4 + q < p_lo || tk0 + 4 + q >= p_hi) lo_b[q] = hi_b[q] = 0u;
            }
        }
        if (CERT) {
            // largest value scale of the step's valid tokens (non-negative
            // fp16: bit patterns order like the values)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                w.smax = umax(w.smax, umax(umax(lo_a[q] & 0xFFFFu, lo_a[q] >> 16), umax(hi_a[q] & 0xFFFFu, hi_a[q] >> 16)));
                w.smax = umax(w.smax, umax(umax(lo_b[q] & 0xFFFFu, lo_b[q] >> 16), umax(hi_b[q] & 0xFFFFu, hi_b[q] >> 16)));
            }
        }
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            uint32_t r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t wa = (gg < 2) ? lo_a[q] : hi_a[q], wb = (gg < 2) ? lo_b[q] : hi_b[q];
                // (scale of position q, scale of position q+4) for group gg
                const uint32_t sp = (gg & 1) ? __builtin_amdgcn_perm(wb, wa, 0x07060302u)
                                             : __builtin_amdgcn_perm(wb, wa, 0x05040100u);
                // p * s_v in fp16: one rounding of p, one of the product
                r[q] = __builtin_bit_cast(uint32_t, pp[q] * __builtin_bit_cast(half2_t, sp));
            }
            const uint4 bop = make_uint4(r[0], r[1], r[2], r[3]);
            w.acc[2 * gg] = mfma(i4x8_to_h8(vt[2 * gg]), bop, w.acc[2 * gg]);
            w.acc[2 * gg + 1] = mfma(i4x8_to_h8(vt[2 * gg + 1]), bop, w.acc[2 * gg + 1]);
        }
    }
}

}  // namespace

// Writes the appended token (position q of a half) into a stage whose code
// parts were copied from HBM before workgroup 0 of (b, kvh) wrote the token:
// its 128 key codes (8 slots of 16 B in the key chunks), its key scale
// dwords, the nibble of each channel's byte and its value-scale dwords.
// Parts served as FP16 rows (bits of mk) are read from the caller's rows and
// need nothing.  Called by the whole wave after the stage is resident.
__device__ __forceinline__ void patch_new_token(uint8_t *stage, uint32_t mk, int q, const uint8_t *nk,
                                                const uint8_t *nv, uint16_t nks, const uint16_t *nvs,
                                                int lane) {
    if (!(mk & 1u)) {
        const int e = (q >> 2) & 1, mrow = 4 * (q >> 3) + (q & 3);
        if (lane < 8) {
            const int dg = lane >> 1, h = lane & 1;
            // a value-fallback step holds its rows' code bytes packed
            const int off = mk == 2u ? 1024 * e + 512 * h + 16 * ((mrow & 7) + 8 * dg)
                                     : (2 * e + h) * 1024 + 16 * (mrow + 16 * dg);
            *reinterpret_cast<uint4 *>(stage + ST_K + off) = *reinterpret_cast<const uint4 *>(nk + 32 * dg + 16 * h);
        }
        if (lane == 8) *reinterpret_cast<uint32_t *>(stage + ST_KS + 4 * q) = nks;
        if (lane == 9) *reinterpret_cast<uint32_t *>(stage + ST_KS + 4 * (q + 32)) = nks;
    }
    if (!(mk & 2u)) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int c = lane + 64 * k;
            uint8_t *bp = stage + ST_V + (c >> 6) * 1024 + 16 * (c & 63) + (q >> 1);
            const uint32_t nib = nv[c] & 0x0Fu;
            *bp = (q & 1) ? (uint8_t)((*bp & 0x0Fu) | (nib << 4)) : (uint8_t)((*bp & 0xF0u) | nib);
        }
        if (lane == 10) *reinterpret_cast<uint32_t *>(stage + ST_VS + 4 * q) = (uint32_t)nvs[0] | ((uint32_t)nvs[1] << 16);
        if (lane == 11)
            *reinterpret_cast<uint32_t *>(stage + ST_VS + 128 + 4 * q) = (uint32_t)nvs[2] | ((uint32_t)nvs[3] << 16);
    }
}

// Entries of the table of blocks that one workgroup's share of steps touches:
// at most half its steps (every block has two or more) plus the two blocks
// cut by its range ends.
constexpr int TBL = 4 * MFMA_MAX_BPS + 8;

// Round a non-negative float up to an fp16 value (a bound stays a bound).
__device__ __forceinline__ uint16_t f16_up(float x) {
    uint32_t h = f2h_rn(x);
    if (h2f(h) < x) h += 1;
    return (uint16_t)h;
}

// CERT: also the per-head output certificate's per-split parts (the
// mass-weighted value error, the largest certified value scale and
// fallback |v|, and the largest certified block errors).
template <bool CERT, bool RANK, bool ROT, bool K16>
__device__ __forceinline__ void decode_group(const DecodeArgs &a, const int split, const int64_t kvh,
                                             const int64_t b) {
    // NW waves x NSTAGE stages x 6656 B of ring.  Before the stream starts, the
    // ring from wave 1 on holds the masks of every block of (b, kvh); after it
    // ends, the ring holds the wave merge.
    __shared__ __attribute__((aligned(16))) uint8_t ring[NW][NSTAGE][ST_BYTES];
    __shared__ int16_t toff_lds[TBL];  // share-local index of each listed block's first step
    __shared__ uint8_t tmk_lds[TBL];   // its fallback mask
    __shared__ float wm[NW][16], wl[NW][16];
    __shared__ int wsum_lds[NW];
    __shared__ int blo_lds, ntbl_lds;
    __shared__ int next_lds;  // next unclaimed step of the share
    __shared__ uint16_t teta_lds[CERT ? TBL : 1];  // certificate: value error of each listed block (fp16, rounded up; 0 on value fallback)
    uint8_t *maskb = &ring[1][0][0];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept scalar
    const int m = lane & 15, g4 = lane >> 4;                    // MFMA row/column index and k-group
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g;
    const int nb = (int)a.nb;
    constexpr int NT = NW * 64;

    // fused append: token t_new of (b, kvh) is quantized by every workgroup
    // of (b, kvh), in the 16-lane group holding the mask thread of its block
    // (block i has thread i % NT), with the same arithmetic as the append
    // kernel; that thread puts the token's statistics into its block's mask,
    // workgroup 0 of (b, kvh) writes the token's tier-1 bytes, and the wave
    // whose step holds the token patches it into its stage.  Its rows are
    // loaded first, with the block statistics and the query rows.
    const int64_t t_new = a.t_new;
    const int64_t blk_new = t_new >= 0 ? t_new / BLK : -1;
    const int p_new = t_new >= 0 ? (int)(t_new % BLK) : 0;
    const bool qgroup = t_new >= 0 && (tid >> 4) == (int)((blk_new % NT) >> 4);
    RowIn rin;
    if (qgroup) {
        const int64_t row = bh * a.cap + t_new;
        rin = load_row16(a.c.k16 + row * D, a.c.v16 + row * D, tid & 15);
    }

    // block statistics of the first PF * NT blocks, fetched while the query
    // rows load
    constexpr int PF = 4;
    float ke[PF], ve[PF];
#pragma unroll
    for (int r = 0; r < PF; ++r) {
        const int i = tid + r * NT;
        ke[r] = i < nb ? a.c.k_err[bh * a.nbc + i] : 0.0f;
        ve[r] = i < nb ? a.c.v_err[bh * a.nbc + i] : 0.0f;
    }
    // B operands of Q.K^T, loaded by every wave straight from HBM: lane
    // (n = head, dg) holds q[n][32dg + 8s .. +8] at step s (heads >= G: 0).
    // The same registers give the query norms: run 4dg + s of head n is its
    // 8 channels at step s, so the pinned tree's run pairs (r, r+8), (r, r+4)
    // are lanes dg, dg^2 and dg, dg^1, and (r, r+2), (r, r+1) are in-lane.
    uint4 qb[4];
    float qn;
    {
        const bool live = m < g;
        const uint16_t *qr = a.q + (b * a.hq + kvh * g + (live ? m : 0)) * D + 32 * g4;
        double run[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 v = *reinterpret_cast<const uint4 *>(qr + 8 * s);
            qb[s] = live ? v : make_uint4(0u, 0u, 0u, 0u);
            const uint32_t w4[4] = {qb[s].x, qb[s].y, qb[s].z, qb[s].w};
            double t[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t[2 * i] = sq64(h2f(w4[i] & 0xFFFFu));
                t[2 * i + 1] = sq64(h2f(w4[i] >> 16));
            }
            run[s] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) run[s] = add_partner_d<true>(run[s]);
#pragma unroll
        for (int s = 0; s < 4; ++s) run[s] = add_partner_d<false>(run[s]);
        const float qh = (float)__dsqrt_rn((run[0] + run[2]) + (run[1] + run[3]));
        // group norm: max over the heads (lanes m; heads >= G have norm 0),
        // keeping NaN: non-negative floats, +Inf and NaN order like their
        // bit patterns
        qn = __uint_as_float(row16_max_u32(__float_as_uint(qh)));
    }
    // rotated key codec: the query rotated the same way, for the code tiles
    uint4 qrh[4], qrl[4];
    if (ROT) rotate_q(qb, lane, qrh, qrl);

    __shared__ __attribute__((aligned(16))) uint8_t nk_lds[D];  // key codes of the new token
    __shared__ __attribute__((aligned(16))) uint8_t nv_lds[D];  // its value codes (low nibbles)
    __shared__ uint16_t nks_lds, nvs_lds[4];                     // its key and value scales
    __shared__ float nerr_lds[2];                                // its key and value errors
    RowQuant rq = {};
    if (qgroup) {
        rq = quant_row16(rin, ROT, tid & 15);
        const int l16 = tid & 15;
        *reinterpret_cast<uint2 *>(&nk_lds[8 * l16]) = make_uint2(rq.kc[0], rq.kc[1]);
        *reinterpret_cast<uint2 *>(&nv_lds[8 * l16]) = make_uint2(rq.vc[0], rq.vc[1]);
        if ((l16 & 3) == 0) nvs_lds[l16 >> 2] = (uint16_t)rq.vsb;
        if (l16 == 0) {
            nks_lds = (uint16_t)rq.ksb;
            nerr_lds[0] = rq.kerr;
            nerr_lds[1] = rq.verr;
        }
    }

    // masks of every block of (b, kvh); mask_out receives this workgroup's
    // home range of bps blocks.  Certificate: each block's value error
    // (etab, 0 on value fallback) and, per wave, the largest key and value
    // errors of the certified blocks (kvw), both in the ring until the
    // stream starts.
    float *etab = reinterpret_cast<float *>(&ring[0][0][0] + 40960);  // past maskb's 16 KB
    float *kvw = etab + MFMA_MAX_BPS * MAX_SPLITS;
    float kmx = 0.0f, vmx = 0.0f;
    {
        const int64_t h0 = (int64_t)split * a.bps, h1 = h0 + a.bps;
        auto put = [&](int i, float kerr, float verr) {
            if (i == blk_new) {
                // the block holding the appended token (this thread is in the
                // lane group that quantized it): its statistics after the
                // append (max with the earlier tokens of the block)
                kerr = p_new > 0 ? fmaxf(rq.kerr, kerr) : rq.kerr;
                verr = p_new > 0 ? fmaxf(rq.verr, verr) : rq.verr;
            }
            uint32_t mk = block_mask(a.sm, qn, kerr, verr, a.tau_k, a.tau_v);
            if (a.promote) mk |= a.promote[bh * a.nbc + i];  // adaptive precision: promoted tiles
            maskb[i] = (uint8_t)mk;
            if (a.mask_out && i >= h0 && i < h1) a.mask_out[bh * a.nb + i] = (uint8_t)mk;
            if (CERT) {
                if (!(mk & 1u)) kmx = fmaxf(kmx, kerr);
                if (!(mk & 2u)) vmx = fmaxf(vmx, verr);
                etab[i] = (mk & 2u) ? 0.0f : verr;
            }
        };
#pragma unroll
        for (int r = 0; r < PF; ++r)
            if (tid + r * NT < nb) put(tid + r * NT, ke[r], ve[r]);
        for (int i = tid + PF * NT; i < nb; i += NT) put(i, a.c.k_err[bh * a.nbc + i], a.c.v_err[bh * a.nbc + i]);
        if (CERT) {
            // non-negative errors (+Inf included): max of the bit patterns
            kmx = __uint_as_float(wave_max_u32(__float_as_uint(kmx)));
            vmx = __uint_as_float(wave_max_u32(__float_as_uint(vmx)));
            if (lane == 0) {
                kvw[wave] = kmx;
                kvw[NW + wave] = vmx;
            }
        }
    }
    __syncthreads();
    if (CERT) {
        // the largest key and value errors of the certified blocks of (b, kvh)
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            kmx = fmaxf(kmx, kvw[w]);
            vmx = fmaxf(vmx, kvw[NW + w]);
        }
    }

    // workgroup 0 of (b, kvh) writes the appended token's tier-1 bytes and
    // its block's statistics (as the append kernel would); no other
    // workgroup reads them in this launch except through a stage, which the
    // patch below corrects
    if (t_new >= 0 && split == 0) {
        const int64_t row = bh * a.cap + t_new;
        if (tid < 8) *reinterpret_cast<uint4 *>(a.c.k_codes + row * D + 16 * tid) =
            *reinterpret_cast<const uint4 *>(&nk_lds[16 * tid]);
        if (tid == 8) a.c.k_scales[row] = nks_lds;
        if (tid >= 12 && tid < 16) a.c.v_scales[row * 4 + (tid - 12)] = nvs_lds[tid - 12];
        uint8_t *vblk = a.c.v_codes + (bh * a.nbc + blk_new) * (D * BLK / 2);
        if (p_new == 0) {
            // a new block: byte (c, 0) holds the token's nibble, every other
            // nibble of the block is 0
            for (int i = tid; i < D * 2; i += NT)
                *reinterpret_cast<uint4 *>(vblk + 16 * i) =
                    make_uint4((i & 1) ? 0u : (uint32_t)(nv_lds[i >> 1] & 0x0Fu), 0u, 0u, 0u);
        } else if (tid < D) {
            // replace the token's nibble in its byte with two atomics (clear,
            // then set; same address, so in order) rather than a read-back
            // that would hold this wave until the load returns
            const int byte = tid * (BLK / 2) + (p_new >> 1);
            const int sh = 8 * (byte & 3) + 4 * (p_new & 1);
            unsigned int *word = reinterpret_cast<unsigned int *>(vblk + (byte & ~3));
            atomicAnd(word, ~(0x0Fu << sh));
            atomicOr(word, (uint32_t)(nv_lds[tid] & 0x0Fu) << sh);
        }
        if (tid == 0) {
            // block statistics: max with the earlier tokens' (non-negative
            // floats and +Inf order like their bit patterns), or the token's
            // own for a new block
            const int64_t si = bh * a.nbc + blk_new;
            if (p_new > 0) {
                atomicMax(reinterpret_cast<unsigned int *>(a.c.k_err + si), __float_as_uint(nerr_lds[0]));
                atomicMax(reinterpret_cast<unsigned int *>(a.c.v_err + si), __float_as_uint(nerr_lds[1]));
            } else {
                a.c.k_err[si] = nerr_lds[0];
                a.c.v_err[si] = nerr_lds[1];
            }
        }
    }

    // Work of (b, kvh) in steps: 2 per certified block (its halves), 4 per
    // block whose keys alone fall back (16-token steps), 8 per other fallback
    // block (8-token steps).  Split s takes steps [r0, r1) of the
    // sequence in block order, so splits carry equal work however the
    // fallback blocks fall.  Thread t sums the contiguous blocks [t*c, t*c+c).
    const int c = (nb + NT - 1) / NT;
    const int i0 = tid * c < nb ? tid * c : nb, i1 = i0 + c < nb ? i0 + c : nb;
    int mysum = 0;
    for (int i = i0; i < i1; ++i) mysum += steps_of(maskb[i]);
    const int incl = wave_incl_scan_int(mysum);
    if (lane == 63) wsum_lds[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int v = wsum_lds[w];
        before += w < wave ? v : 0;
        total += v;
    }
    const int excl = before + incl - mysum;  // steps before block i0
    const int r0 = (int)((int64_t)split * total / a.splits);
    const int r1 = (int)((int64_t)(split + 1) * total / a.splits);
    // first and last block of the share, then the table
    {
        int p = excl;
        for (int i = i0; i < i1; ++i) {
            const int w = steps_of(maskb[i]);
            if (p <= r0 && r0 < p + w) blo_lds = i;
            if (p <= r1 - 1 && r1 - 1 < p + w) ntbl_lds = i;  // last block, made a count below
            p += w;
        }
    }
    __syncthreads();
    const int blo = blo_lds;
    if (tid == 0) next_lds = 0;
    {
        int p = excl;
        for (int i = i0; i < i1; ++i) {
            const uint32_t mk = maskb[i];
            const int w = steps_of(mk);
            if (p < r1 && p + w > r0) {
                toff_lds[i - blo] = (int16_t)(p - r0);
                tmk_lds[i - blo] = (uint8_t)mk;
                if (CERT) teta_lds[i - blo] = (mk & 2u) ? (uint16_t)0 : f16_up(etab[i]);
            }
            p += w;
        }
    }
    __syncthreads();
    const int ntbl = r1 > r0 ? ntbl_lds - blo + 1 : 0;

    // The share's steps are claimed by the waves one at a time, at issue
    // time, from a counter in LDS, so that a wave that runs ahead (the SIMD
    // issues the older of its two waves first) takes more steps and the waves
    // of the workgroup finish together.  A wave's claims increase, so a step
    // is found in the table with a 64-entry window that only moves forward,
    // held one entry per lane: the listed block is the last one whose first
    // step is at or before it.
    const int nshare = r1 - r0;
    struct Window {
        int jb;        // table index of lane 0
        int off;       // this lane's entry: first step, mask
        uint32_t mk;
    };
    auto load_window = [&](Window &wn, int jb) {
        wn.jb = jb;
        const int j = jb + lane;
        wn.off = j < ntbl ? toff_lds[j] : 0x7fffffff;
        wn.mk = j < ntbl ? tmk_lds[j] : 0u;
    };
    // share step t -> block, sub-step (half or fallback step), mask
    auto find = [&](Window &wn, int t, int64_t &blk, int &sub, uint32_t &mk) {
        uint64_t bal = __builtin_amdgcn_ballot_w64(wn.off <= t);
        while ((bal >> 63) && wn.jb + 64 < ntbl) {
            load_window(wn, wn.jb + 63);
            bal = __builtin_amdgcn_ballot_w64(wn.off <= t);
        }
        const int idx = 63 - __builtin_clzll(bal);
        blk = blo + wn.jb + idx;
        sub = t - __builtin_amdgcn_readlane(wn.off, idx);
        mk = __builtin_amdgcn_readlane(wn.mk, idx);
    };
    Window iwin, pwin;  // issue and process cursors
    load_window(iwin, 0);
    pwin = iwin;
    auto claim = [&]() -> int {
        int t = 0;
        if (lane == 0) t = atomicAdd(&next_lds, 1);
        return __builtin_amdgcn_readfirstlane(t);
    };
    const uint32_t ring0 = (uint32_t)(uintptr_t)&ring[wave][0][0];
    // claims of the steps in the stages (>= nshare: none)
    int tq[NSTAGE];
    auto claim_issue = [&](int st) {
        const int t = claim();
        tq[st] = t;
        if (t < nshare) {
            int64_t blk;
            int sub;
            uint32_t mk;
            find(iwin, t, blk, sub, mk);
            const uint32_t sa = ring0 + st * ST_BYTES;
            if (mk)
                issue_fb(a, bh, blk, sub, mk, sa, lane);
            else
                issue_half(a, bh, blk, sub, sa, lane);
        }
    };
    // all stages but the last (the masks in the ring are no longer needed)
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st) claim_issue(st);

    const float sml2 = a.sm * 1.4426950408889634f;  // scores in log2 units
    WaveState ws;
    ws.m_run = NEG_INF;
    ws.l_run = 0.0f;
    ws.e_run = 0.0f;
    ws.smax = 0u;
    ws.amax = 0u;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) ws.acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};

    // Stage s holds claim tq[s].  When the step in stage s starts, the step in
    // the next stage has been claimed and issued too if it exists (with two
    // stages, just now); waiting until at most its 8 copies are outstanding
    // makes stage s resident.  Any other load issued in between only makes
    // the wait stronger.  With three stages the stage after that is claimed
    // and issued once this step's key part is in the matrix cores.  Returns
    // false once the wave has no step left.
    auto step = [&](int s) -> bool {
        const int t = tq[s];
        if (t >= nshare) return false;
        const int s1 = s + 1 == NSTAGE ? 0 : s + 1;
        const int s2 = s1 + 1 == NSTAGE ? 0 : s1 + 1;
        if (EARLY_ISSUE) claim_issue(s1);
        if (tq[s1] < nshare)
            wait_vmcnt<DMA_PER_STEP>();
        else
            wait_vmcnt<0>();
        auto mid = [&]() {
            if (!EARLY_ISSUE) claim_issue(s2);
        };
        int64_t blk;
        int sub;
        uint32_t mk;
        find(pwin, t, blk, sub, mk);
        uint8_t *stage = &ring[wave][s][0];
        // tokens of the step: 32 (certified half), 16 (keys only) or 8
        const int step_len = BLK / steps_of(mk);
        if (blk == blk_new && p_new / step_len == sub)
            patch_new_token(stage, mk, p_new & 31, nk_lds, nv_lds, nks_lds, nvs_lds, lane);
        // positions [p_lo, p_hi) of the half: the valid tokens of the step
        const int p_lo = (step_len * sub) & 31;
        const int64_t left = a.length - (blk * BLK + step_len * sub);
        const int nvalid = (int)(left < step_len ? (left > 0 ? left : 0) : step_len);
        if (nvalid > 0)
            process_step<CERT, RANK, ROT, K16>(stage, mk, p_lo, p_lo + nvalid, qb, qrh, qrl, sml2, ws, lane,
                                     CERT ? h2f(teta_lds[blk - blo]) : 0.0f,
                                     RANK ? a.step_ml + (bh * g * a.nbc + blk) * 8 + sub * (8 / steps_of(mk)) : nullptr,
                                     a.nbc * 8, g, mid);
        else
            mid();
        return true;
    };
    for (bool more = true; more;) {
#pragma unroll
        for (int s = 0; s < NSTAGE; ++s)
            if (more) more = step(s);
    }

    // ---------------- merge waves, then splits
    // lane (n = m, r = g4) holds O^T[16mt + 4r + i][n] and a share of l
    const float l_run = sum_across_rows(ws.l_run);
    __syncthreads();  // every wave is done with the ring: reuse it for the wave merge
    float *wacc = reinterpret_cast<float *>(&ring[0][0][0]);
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
    float *we = reinterpret_cast<float *>(&ring[0][0][0] + NW * 16 * D * 4);  // [NW][16]
    uint32_t *wsa = reinterpret_cast<uint32_t *>(we + NW * 16);                // [NW][2]
    if (CERT) {
        const float e_run = sum_across_rows(ws.e_run);
        const uint32_t sm_ = wave_max_u32(ws.smax), am_ = wave_max_u32(ws.amax);
        if (m < g && g4 == 0) we[wave * 16 + m] = e_run;
        if (lane == 0) {
            wsa[2 * wave] = sm_;
            wsa[2 * wave + 1] = am_;
        }
    }
    __syncthreads();
    write_partial<NW>(a, bh, split, 16, wm, wl, wacc);
    if (!CERT && a.arrive) {
        __syncthreads();  // the wave merge's LDS is read; the ring is free for the split merge
        fold_merge(a, bh, b, kvh, &ring[0][0][0]);
    }
    if (CERT) {
        // per head: the split's mass-weighted value error on the scale of its
        // running maximum (as write_partial scales the running sum)
        for (int h = tid; h < g; h += NT) {
            float M = -__builtin_huge_valf();
            for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w][h]);
            float E = 0.0f;
            if (M != -__builtin_huge_valf())
                for (int w = 0; w < NW; ++w)
                    if (wm[w][h] != -__builtin_huge_valf()) E += we[w * 16 + h] * __builtin_amdgcn_exp2f(wm[w][h] - M);
            a.part_e[(bh * a.splits + split) * g + h] = E;
        }
        if (tid == 0) {
            uint32_t sm_ = 0u, am_ = 0u;
            for (int w = 0; w < NW; ++w) {
                sm_ = umax(sm_, wsa[2 * w]);
                am_ = umax(am_, wsa[2 * w + 1]);
            }
            a.part_sa[bh * a.splits + split] = make_float2(h2f(sm_), h2f(am_));
            if (split == 0) a.part_kv[bh] = make_float2(kmx, vmx);
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming split-K decode with its set-up overlapped: the plain and rotated
// key codecs, up to STREAM_MAX_NB blocks per sequence, no certificate.
//
// The bounds of Methodology 2 need the query norm and the block statistics
// before a tile can be chosen, and the first memory accesses of a launch take
// several microseconds.  The tiles of most blocks are certified, so each
// workgroup streams the quantized halves of the first NSPEC blocks of its
// home range before it knows their masks: wave w issues half w of them right
// behind its set-up loads (query operand, the statistics of its blocks of
// the mask pass, and in one lane group the appended token's rows) and half
// w + NW once those loads are in.  It then forms the group norm and the masks
// of its blocks, with each 64-block chunk's pool steps, and after the one
// workgroup barrier every wave knows every mask.  A first block whose tile is
// certified keeps its speculative halves (MK_SPEC); a speculative half whose
// block falls back is dropped when it lands.  Every other block joins the
// group's pool in block order, with two halves, four 16-token steps (keys or
// values alone falling back) or eight 8-token steps (both).  The pool is cut
// so that every workgroup of the group carries the same work, its
// speculative halves included, and the waves claim the steps of their range
// from an LDS counter.  A wave finds a step's block through a window over 64
// consecutive blocks of the group (mask byte and first pool step, one per
// lane) that only moves forward, with the pool steps before each 64-block
// chunk held one per lane.  The appended token (fused append) lies in the
// last block, which stays out of the pool: after the barrier, the first
// split quantizes it and writes its tier-1 bytes, and the last split
// quantizes it, forms the block's mask and takes its steps after its range,
// so that no wave waits for that work at the barrier.
constexpr int STREAM_MAX_NB = 2048;  // blocks per sequence: four rounds of statistics per wave
constexpr int NSPEC = 8;             // first blocks of a split streamed before their masks are known
constexpr uint32_t MK_SPEC = 4u;     // mask byte of such a block whose tile is certified
constexpr uint32_t MK_LATE = 5u;     // the appended token's block (its mask is formed after the barrier)
constexpr int NO_STEP = 0x7fffffff;
static_assert(2 * NSPEC == NW * (NSTAGE - 1), "one speculative half per wave in each stage but the last");

// Steps a block adds to the pool, from its mask byte.
__device__ __forceinline__ int pool_steps(uint32_t code) {
    return code == 0u ? 2 : (code == 3u ? 8 : (code >= MK_SPEC ? 0 : 4));
}

template <bool ROT>
__device__ __forceinline__ void decode_group_stream(const DecodeArgs &a, const int split, const int64_t kvh,
                                                    const int64_t b) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[NW][NSTAGE][ST_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t maskb[STREAM_MAX_NB];
    __shared__ int csteps_lds[STREAM_MAX_NB / 64];  // pool steps per 64-block chunk
    __shared__ float wm[NW][16], wl[NW][16];
    __shared__ int next_lds;
    __shared__ int late_lds;  // mask of the appended token's block | LATE_READY, once formed
    __shared__ __attribute__((aligned(16))) uint8_t nk_lds[D];  // key codes of the new token
    __shared__ __attribute__((aligned(16))) uint8_t nv_lds[D];  // its value codes (low nibbles)
    __shared__ uint16_t nks_lds, nvs_lds[4];                     // its key and value scales
    __shared__ float nerr_lds[2];                                // its key and value errors

    constexpr int NT = NW * 64;
    constexpr int MAXR = STREAM_MAX_NB / NT;  // blocks per thread in the mask pass
    constexpr int LATE_READY = 0x100;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, g4 = lane >> 4;
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g;
    const int nb = (int)a.nb;
    const int bps = a.bps;
    const int nsplit = a.splits;
    const int a0 = split * bps;  // first block of the home range
    const uint32_t ring0 = (uint32_t)(uintptr_t)&ring[wave][0][0];

    // fused append: token t_new lies in the last block.  The workgroups that
    // need it quantize it after the mask barrier, in the 16-lane group of the
    // thread holding that block in the mask pass (block i: thread i % NT):
    // the first split writes its tier-1 bytes, the last split attends over it
    // and takes the block after its share of the pool.
    const int64_t t_new = a.t_new;
    const bool late = t_new >= 0;
    const int blk_new = late ? (int)(t_new / BLK) : -1;
    const int p_new = late ? (int)(t_new % BLK) : 0;
    const bool take_late = late && split == nsplit - 1;
    const bool qgroup = late && (split == 0 || take_late) && (tid >> 4) == ((blk_new % NT) >> 4);

    if (tid == 0) {
        next_lds = 0;  // both read after the mask barrier
        late_lds = 0;
    }

    // ---------------- set-up loads: query operand, block statistics (thread
    // t: blocks t + NT r), the appended token's rows
    const int rounds = (nb + NT - 1) / NT;
    uint4 qraw[4];
    {
        const uint16_t *qr = a.q + (b * a.hq + kvh * g + (m < g ? m : 0)) * D + 32 * g4;
#pragma unroll
        for (int s = 0; s < 4; ++s) qraw[s] = *reinterpret_cast<const uint4 *>(qr + 8 * s);
    }
    float ke[MAXR], ve[MAXR];
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
        const int i = r * NT + tid;
        ke[r] = (r < rounds && i < nb) ? a.c.k_err[bh * a.nbc + i] : 0.0f;
        ve[r] = (r < rounds && i < nb) ? a.c.v_err[bh * a.nbc + i] : 0.0f;
    }
    RowIn rin;
    if (qgroup) {
        const int64_t row = bh * a.cap + t_new;
        rin = load_row16(a.c.k16 + row * D, a.c.v16 + row * D, tid & 15);
    }

    // ---------------- speculative halves: half j = wave + NW * st of the home
    // range's first NSPEC blocks into stage st (the appended token's block is
    // never speculative).  Stage 0's copies go right behind the set-up loads:
    // the first accesses of a launch take microseconds, and these land with
    // them.  Stage 1's follow once the set-up loads are used (more copies
    // ahead of them would delay them).  `live` bit st: stage st holds copies
    // not yet consumed.
    int tq[NSTAGE];
    uint32_t live = 0u;
    const int na = min(NSPEC, min(bps, nb - a0));
    auto spec_issue = [&](int st) {
        const int j = wave + NW * st;
        const int blk = a0 + (j >> 1);
        tq[st] = NO_STEP;
        if ((j >> 1) < na && blk != blk_new && (int64_t)blk * BLK + 32 * (j & 1) < a.length) {
            issue_half(a, bh, blk, j & 1, ring0 + st * ST_BYTES, lane);
            tq[st] = -1 - j;
            live |= 1u << st;
        }
    };
    spec_issue(0);
    tq[NSTAGE - 1] = NO_STEP;

    // ---------------- query operand and group norm (as decode_group); the
    // first use of the set-up loads waits for everything issued so far
    uint4 qb[4];
    float qn;
    {
        double run[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            qb[s] = m < g ? qraw[s] : make_uint4(0u, 0u, 0u, 0u);
            const uint32_t w4[4] = {qb[s].x, qb[s].y, qb[s].z, qb[s].w};
            double t[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t[2 * i] = sq64(h2f(w4[i] & 0xFFFFu));
                t[2 * i + 1] = sq64(h2f(w4[i] >> 16));
            }
            run[s] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) run[s] = add_partner_d<true>(run[s]);
#pragma unroll
        for (int s = 0; s < 4; ++s) run[s] = add_partner_d<false>(run[s]);
        const float qh = (float)__dsqrt_rn((run[0] + run[2]) + (run[1] + run[3]));
        qn = __uint_as_float(row16_max_u32(__float_as_uint(qh)));
    }
    spec_issue(1);
    uint4 qrh[4], qrl[4];
    if (ROT) rotate_q(qb, lane, qrh, qrl);

    // ---------------- masks of every block of (b, kvh) but the appended
    // token's (MK_LATE); mask_out receives the home range.  Bytes past the
    // last block (to the end of its 64-block chunk) are MK_SPEC: no steps.
    const int nch = (nb + 63) / 64;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
        if (r >= rounds) break;
        const int i = r * NT + tid;  // the wave's 64 lanes hold chunk r * NW + wave
        uint32_t code = MK_SPEC;
        if (i == blk_new) {
            code = MK_LATE;
        } else if (i < nb) {
            const uint32_t mk = block_mask(a.sm, qn, ke[r], ve[r], a.tau_k, a.tau_v);
            if (a.mask_out && i >= a0 && i < a0 + bps) a.mask_out[bh * a.nb + i] = (uint8_t)mk;
            code = (mk == 0u && (uint32_t)i % (uint32_t)bps < (uint32_t)NSPEC) ? MK_SPEC : mk;
        }
        const int c = r * NW + wave;
        if (c < nch) {
            maskb[i] = (uint8_t)code;
            const int cs = wave_total_sum_int(pool_steps(code));
            if (lane == 0) csteps_lds[c] = cs;
        }
    }
    __syncthreads();

    // ---------------- the appended token (quantizing group only): its codes,
    // its block's statistics and mask, then (first split) its tier-1 bytes,
    // written by the whole wave from what its lanes put in LDS
    if (qgroup) {
        const int l16 = tid & 15;
        const RowQuant rq = quant_row16(rin, ROT, l16);
        *reinterpret_cast<uint2 *>(&nk_lds[8 * l16]) = make_uint2(rq.kc[0], rq.kc[1]);
        *reinterpret_cast<uint2 *>(&nv_lds[8 * l16]) = make_uint2(rq.vc[0], rq.vc[1]);
        if ((l16 & 3) == 0) nvs_lds[l16 >> 2] = (uint16_t)rq.vsb;
        if (l16 == 0) {
            nks_lds = (uint16_t)rq.ksb;
            nerr_lds[0] = rq.kerr;
            nerr_lds[1] = rq.verr;
        }
        if (tid == blk_new % NT) {
            // statistics after the append: max with the block's earlier tokens
            const int rb = blk_new / NT;
            float ko = ke[0], vo = ve[0];
#pragma unroll
            for (int r = 1; r < MAXR; ++r)
                if (rb == r) {
                    ko = ke[r];
                    vo = ve[r];
                }
            const float kerr = p_new > 0 ? fmaxf(rq.kerr, ko) : rq.kerr;
            const float verr = p_new > 0 ? fmaxf(rq.verr, vo) : rq.verr;
            const uint32_t mk = block_mask(a.sm, qn, kerr, verr, a.tau_k, a.tau_v);
            if (a.mask_out && blk_new >= a0 && blk_new < a0 + bps) a.mask_out[bh * a.nb + blk_new] = (uint8_t)mk;
            // the codes and scales above are in LDS before the flag (this
            // lane's LDS writes complete in order)
            __hip_atomic_store(&late_lds, (int)mk | LATE_READY, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    if (late && split == 0 && wave == ((blk_new % NT) >> 6)) {
        // the quantizing wave (the same lanes wrote the LDS values read here)
        const int64_t row = bh * a.cap + t_new;
        if (lane < 8)
            *reinterpret_cast<uint4 *>(a.c.k_codes + row * D + 16 * lane) =
                *reinterpret_cast<const uint4 *>(&nk_lds[16 * lane]);
        if (lane == 8) a.c.k_scales[row] = nks_lds;
        if (lane >= 12 && lane < 16) a.c.v_scales[row * 4 + (lane - 12)] = nvs_lds[lane - 12];
        uint8_t *vblk = a.c.v_codes + (bh * a.nbc + blk_new) * (D * BLK / 2);
        if (p_new == 0) {
            // a new block: byte (c, 0) holds the token's nibble, every other
            // nibble of the block is 0
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = lane + 64 * k;
                *reinterpret_cast<uint4 *>(vblk + 16 * i) =
                    make_uint4((i & 1) ? 0u : (uint32_t)(nv_lds[i >> 1] & 0x0Fu), 0u, 0u, 0u);
            }
        } else {
            // the token's nibble replaced in its byte by two atomics (clear,
            // then set; same address, so in order)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int c = lane + 64 * k;
                const int byte = c * (BLK / 2) + (p_new >> 1);
                const int sh = 8 * (byte & 3) + 4 * (p_new & 1);
                unsigned int *word = reinterpret_cast<unsigned int *>(vblk + (byte & ~3));
                atomicAnd(word, ~(0x0Fu << sh));
                atomicOr(word, (uint32_t)(nv_lds[c] & 0x0Fu) << sh);
            }
        }
        if (lane == 0) {
            const int64_t si = bh * a.nbc + blk_new;
            if (p_new > 0) {
                atomicMax(reinterpret_cast<unsigned int *>(a.c.k_err + si), __float_as_uint(nerr_lds[0]));
                atomicMax(reinterpret_cast<unsigned int *>(a.c.v_err + si), __float_as_uint(nerr_lds[1]));
            } else {
                a.c.k_err[si] = nerr_lds[0];
                a.c.v_err[si] = nerr_lds[1];
            }
        }
    }

    // ---------------- the pool: the steps before each 64-block chunk (lane
    // c) and this workgroup's equal share; the last split then takes the
    // appended token's block
    const int csteps = lane < nch ? csteps_lds[lane] : 0;
    const int cincl = wave_incl_scan_int(csteps);
    const int ptotal = __builtin_amdgcn_readlane(cincl, 63);
    const int cpre = lane < nch ? cincl - csteps : NO_STEP;
    // Each split's pool range: the work before split s (its speculative
    // halves and pool steps) is s/S of the whole, the halves being those of
    // the certified first blocks of every split (lane s and s + 64 count
    // split s's); a running max keeps the ranges ordered when a split's
    // halves exceed its fair share.  s * work < 2^31: at most 128 splits of
    // 2048 blocks of 8 steps.
    int p0, nshare;
    {
        auto spec_count = [&](int sp) -> int {
            int c = 0;
            if (sp < nsplit) {
                const int b0 = sp * bps, n = min(NSPEC, min(bps, nb - b0));
                for (int k = 0; k < n; ++k) c += maskb[b0 + k] == MK_SPEC ? 1 : 0;
            }
            return c;
        };
        const int sc0 = spec_count(lane), sc1 = spec_count(lane + 64);
        const int in0 = wave_incl_scan_int(sc0);
        const int in1 = wave_incl_scan_int(sc1) + __builtin_amdgcn_readlane(in0, 63);
        const int work = ptotal + 2 * __builtin_amdgcn_readlane(in1, 63);
        auto raw = [&](int sp, int before) -> int {
            return sp < nsplit ? (int)((uint32_t)(sp * work) / (uint32_t)nsplit) - 2 * before : NO_STEP;
        };
        const int r0 = wave_incl_scan_max_int(raw(lane, in0 - sc0));
        const int r1 = max(wave_incl_scan_max_int(raw(lane + 64, in1 - sc1)), __builtin_amdgcn_readlane(r0, 63));
        auto start = [&](int sp) -> int {
            const int v = sp >= nsplit ? ptotal
                                       : (sp < 64 ? __builtin_amdgcn_readlane(r0, sp) : __builtin_amdgcn_readlane(r1, sp - 64));
            return min(max(v, 0), ptotal);
        };
        p0 = start(split);
        nshare = start(split + 1) - p0;
    }

    // window over chunk c: lane j holds block 64c + j, its first pool step
    // (off) and mask byte (0xFF: no steps); cursors only move forward
    struct Window {
        int c, off;
        uint32_t code;
    };
    auto load_window = [&](Window &wn, int c) {
        wn.c = c;
        const uint32_t code = maskb[64 * c + lane];
        const int st = pool_steps(code);
        const int incl = wave_incl_scan_int(st);
        wn.off = __builtin_amdgcn_readlane(cpre, c) + incl - st;
        wn.code = st > 0 ? code : 0xFFu;
    };
    // share step t (>= 0) -> block, sub-step (half or fallback step), mask
    // bits; false past the last step
    auto resolve = [&](Window &wn, int t, int &blk, int &sub, uint32_t &mk) -> bool {
        if (t < nshare) {
            const int pt = p0 + t;
            if (wn.c < 0 || pt >= __builtin_amdgcn_readlane(cpre, wn.c + 1)) {
                const uint64_t cb = __builtin_amdgcn_ballot_w64(cpre <= pt);
                load_window(wn, 63 - __builtin_clzll(cb));
            }
            const uint64_t bal = __builtin_amdgcn_ballot_w64(wn.code != 0xFFu && wn.off <= pt);
            const int idx = 63 - __builtin_clzll(bal);
            blk = 64 * wn.c + idx;
            sub = pt - __builtin_amdgcn_readlane(wn.off, idx);
            mk = (uint32_t)__builtin_amdgcn_readlane((int)wn.code, idx) & 3u;
            return true;
        }
        if (!take_late) return false;
        // the appended token's block: wait until its mask is formed (by the
        // time a share is used up it nearly always is)
        int v;
        while (((v = __hip_atomic_load(&late_lds, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) & LATE_READY) == 0)
            __builtin_amdgcn_s_sleep(2);
        mk = (uint32_t)v & 3u;
        blk = blk_new;
        sub = t - nshare;
        return sub < steps_of(mk);
    };
    Window iwin = {-1, 0, 0xFFu}, pwin = {-1, 0, 0xFFu};  // issue and process cursors
    auto claim_issue = [&](int st) {
        int t = 0;
        if (lane == 0) t = atomicAdd(&next_lds, 1);
        t = __builtin_amdgcn_readfirstlane(t);
        tq[st] = t;
        int blk, sub;
        uint32_t mk;
        if (resolve(iwin, t, blk, sub, mk)) {
            const uint32_t sa = ring0 + st * ST_BYTES;
            if (mk)
                issue_fb(a, bh, blk, sub, mk, sa, lane);
            else
                issue_half(a, bh, blk, sub, sa, lane);
            live |= 1u << st;
        }
    };
    // stages without a speculative half take the first claims, in stage
    // order (the last stage is claimed during the first step)
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st)
        if (!((live >> st) & 1u)) claim_issue(st);

    const float sml2 = a.sm * 1.4426950408889634f;  // scores in log2 units
    WaveState ws;
    ws.m_run = NEG_INF;
    ws.l_run = 0.0f;
    ws.e_run = 0.0f;
    ws.smax = 0u;
    ws.amax = 0u;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) ws.acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};

    // Step in stage s.  Copies complete in issue order, and the only stage
    // issued after s is s + 1, so waiting until at most its copies are
    // outstanding makes stage s resident.  Once this step's key part is in
    // the matrix cores, the stage consumed by the previous step (s + 2) takes
    // the next claim (unless it still holds a speculative half).  Returns
    // false once the wave has no step left.
    auto step = [&](int s) -> bool {
        if (!((live >> s) & 1u)) return false;
        const int s1 = s + 1 == NSTAGE ? 0 : s + 1;
        const int s2 = s1 + 1 == NSTAGE ? 0 : s1 + 1;
        if ((live >> s1) & 1u)
            wait_vmcnt<DMA_PER_STEP>();
        else
            wait_vmcnt<0>();
        auto mid = [&]() {
            if (!((live >> s2) & 1u)) claim_issue(s2);
        };
        const int t = tq[s];
        int blk, sub;
        uint32_t mk;
        bool keep = true;
        if (t < 0) {
            const int j = -1 - t;
            blk = a0 + (j >> 1);
            sub = j & 1;
            mk = 0u;
            keep = maskb[blk] == MK_SPEC;  // else its block is in the pool
        } else {
            resolve(pwin, t, blk, sub, mk);
        }
        uint8_t *stage = &ring[wave][s][0];
        const int step_len = BLK / steps_of(mk);
        if (keep && blk == blk_new && p_new / step_len == sub)
            patch_new_token(stage, mk, p_new & 31, nk_lds, nv_lds, nks_lds, nvs_lds, lane);
        const int p_lo = (step_len * sub) & 31;
        const int64_t left = a.length - ((int64_t)blk * BLK + step_len * sub);
        const int nvalid = keep ? (int)(left < step_len ? (left > 0 ? left : 0) : step_len) : 0;
        if (nvalid > 0)
            process_step<false, false, ROT, false>(stage, mk, p_lo, p_lo + nvalid, qb, qrh, qrl, sml2, ws, lane, 0.0f,
                                            nullptr, 0, g, mid);
        else
            mid();
        live &= ~(1u << s);
        return true;
    };
    for (bool more = true; more;) {
#pragma unroll
        for (int s = 0; s < NSTAGE; ++s)
            if (more) more = step(s);
    }

    // ---------------- merge waves, then write this split's partial
    const float l_run = sum_across_rows(ws.l_run);
    __syncthreads();  // every wave is done with the ring
    float *wacc = reinterpret_cast<float *>(&ring[0][0][0]);
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
    write_partial<NW>(a, bh, split, 16, wm, wl, wacc);
    if (a.arrive) {
        __syncthreads();  // the wave merge's LDS is read; the ring is free for the split merge
        fold_merge(a, bh, b, kvh, &ring[0][0][0]);
    }
}

template <bool ROT>
__global__ __launch_bounds__(NW * 64, NW / 4) void decode_stream_kernel(DecodeArgs a) {
    decode_group_stream<ROT>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

bool stream_fits(int64_t nb) { return nb >= 1 && nb <= STREAM_MAX_NB; }

bool stream_supports(const DecodeArgs &a) {
    return !a.cert_mode && !a.gate && !a.promote && !a.step_ml && a.nb >= 1 && a.nb <= STREAM_MAX_NB &&
           a.bps >= 1;
}

template <bool CERT, bool RANK, bool ROT>
__global__ __launch_bounds__(NW * 64, NW / 4) void decode_mfma_kernel(DecodeArgs a) {
    // the compact key-only fallback steps in the adaptive decode, where the
    // promoted tiles make them common (elsewhere their extra registers cost
    // more than they save)
    decode_group<CERT, RANK, ROT, RANK && !ROT>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Index of the rank-th group i in [0, n) (in index order) with a set byte
// among flags[i*g, i*g + g), or -1: a count over chunks of NT groups, with
// each wave's ballot and the per-wave totals in wcnt.  Every thread returns
// the same value.
__device__ int64_t nth_set(const uint8_t *flags, const int g, const int64_t n, const int rank, int *wcnt,
                           int64_t *pick) {
    constexpr int NT = NW * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __syncthreads();  // earlier readers of pick and wcnt are done
    if (tid == 0) *pick = -1;
    int base = 0;
    for (int64_t c0 = 0; c0 < n && base <= rank; c0 += NT) {
        const int64_t i = c0 + tid;
        bool f = false;
        if (i < n)
            for (int k = 0; k < g; ++k) f = f || flags[i * g + k] != 0;
        const uint64_t bal = __ballot(f);
        if (lane == 0) wcnt[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int v = wcnt[w];
            before += w < wave ? v : 0;
            tot += v;
        }
        if (f && base + before + __popcll(bal & ((1ull << lane) - 1ull)) == rank) *pick = i;
        base += tot;
        __syncthreads();  // wcnt is rewritten by the next chunk; pick is final
    }
    __syncthreads();
    return *pick;
}

// Recompute pass over the (b, kvh) groups holding a flagged head: grid
// (splits, slots), slot y taking the set groups of rank y, y + slots, ...
// Few groups are expected, and their count is known only on the device, so
// a small grid spreads them over the chip instead of a grid over every group.
template <bool ROT>
__global__ __launch_bounds__(NW * 64, NW / 4) void decode_mfma_gated_kernel(DecodeArgs a, int64_t nbh) {
    __shared__ int wcnt[NW];
    __shared__ int64_t pick;
    for (int rank = blockIdx.y;; rank += gridDim.y) {
        const int64_t bh = nth_set(a.gate, a.g, nbh, rank, wcnt, &pick);
        if (bh < 0) break;
        decode_group<false, false, ROT, false>(a, blockIdx.x, bh % a.hkv, bh / a.hkv);  // tolerances 0: no key-only step
    }
}

bool mfma_supports(int g) { return g >= 1 && g <= 16; }

hipError_t launch_decode_mfma(const DecodeArgs &a, int batch, hipStream_t s) {
    dim3 grid((unsigned)a.splits, (unsigned)a.hkv, (unsigned)batch);
    const dim3 blk(NW * 64);
    if (stream_supports(a) && !a.no_stream) {
        if (a.key_rot)
            hipLaunchKernelGGL(decode_stream_kernel<true>, grid, blk, 0, s, a);
        else
            hipLaunchKernelGGL(decode_stream_kernel<false>, grid, blk, 0, s, a);
        return hipGetLastError();
    }
    if (a.key_rot) {
        if (a.cert_mode && a.step_ml)
            hipLaunchKernelGGL((decode_mfma_kernel<true, true, true>), grid, blk, 0, s, a);
        else if (a.cert_mode)
            hipLaunchKernelGGL((decode_mfma_kernel<true, false, true>), grid, blk, 0, s, a);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<false, false, true>), grid, blk, 0, s, a);
    } else {
        if (a.cert_mode && a.step_ml)
            hipLaunchKernelGGL((decode_mfma_kernel<true, true, false>), grid, blk, 0, s, a);
        else if (a.cert_mode)
            hipLaunchKernelGGL((decode_mfma_kernel<true, false, false>), grid, blk, 0, s, a);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<false, false, false>), grid, blk, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_decode_mfma_gated(const DecodeArgs &a, int batch, int slots, hipStream_t s) {
    dim3 grid((unsigned)a.splits, (unsigned)slots, 1);
    if (a.key_rot)
        hipLaunchKernelGGL(decode_mfma_gated_kernel<true>, grid, dim3(NW * 64), 0, s, a, (int64_t)batch * a.hkv);
    else
        hipLaunchKernelGGL(decode_mfma_gated_kernel<false>, grid, dim3(NW * 64), 0, s, a, (int64_t)batch * a.hkv);
    return hipGetLastError();
}

}  // namespace kvq
