// kvq_quant_row.hpp -- quantization of one token row of one KV head
// (quantize-on-append): quant_row4 for the append kernel (a row per quad) and
// quant_row16 for the fused append-and-decode path (a row per 16 lanes).  The
// two share the code arithmetic below and give the same bytes.
//
// "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1: INT8
// keys (one fp16 scale per token and KV head, absmax/127) and INT4 values (one
// fp16 scale per 32-channel group, absmax/7), with the per-token key error
// ||k - k^||_2 (fp64 pinned tree) and value error max |v - v^|.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Max of |x| over the 8 fp16 values of a lane, as a bit pattern (for
// non-negative fp16 the bit pattern orders like the value; Inf and NaN sort
// above every finite value).
__device__ __forceinline__ uint32_t absmax_bits(const uint32_t w[4]) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = umax(m, umax(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    return m;
}

__device__ __forceinline__ float elem(const uint32_t w[4], int k) {
    return h2f((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu));
}

// Codes by one rounding: fma(x, r, RND_BIAS) = RND_BIAS + rint(x * r) for
// |x * r| < 2^22 (the sum's ulp is 1 and RND_BIAS is even, so ties go to the
// even integer), and the low byte of the sum's bit pattern is that integer
// mod 256.  Clamping the biased value to RND_BIAS +- lim clamps the code.
constexpr float RND_BIAS = 12582912.0f;  // 1.5 * 2^23

// Biased code of x for scale s > 0 with r ~ 1/s within 2 ulps (v_rcp_f32).
// A quotient of two fp16 values that is not a half-integer lies at least
// 2^-14 from one (write x = X 2^a, s = S 2^b with 11-bit X, S: the distance
// is a nonzero multiple of 2^min(a,b) / (2 s), and near a half-integer x/s >=
// 1/4 bounds 2^(a-b) from below), while x*r is within 191 * 2^-22 < 2^-14 of
// x/s (|x/s| <= 190.5 for every scale of the codec, subnormal ones included).
// So the biased code is round_half_even(x/s), clamped, except at an exact
// tie, where it may be the odd neighbour (fix_ties).  r = 0 (a zero scale)
// gives code 0 for finite x.
__device__ __forceinline__ float code_biased(float x, float r, float lim) {
    const float cb = __builtin_fmaf(x, r, RND_BIAS);
    return __builtin_fminf(__builtin_fmaxf(cb, RND_BIAS - lim), RND_BIAS + lim);
}

// Residual x - c*s of a biased code: exact in fp32 (c*s has at most 19
// significant bits, and x and c*s lie on the grid of the smaller of their
// fp16 ulps whenever c is nonzero).
__device__ __forceinline__ float code_residual(float x, float cb, float s) {
    return __builtin_fmaf(-(cb - RND_BIAS), s, x);
}

// Low bytes of four codes, in order, as one dword (byte permutes).
__device__ __forceinline__ uint32_t pack_bytes(int c0, int c1, int c2, int c3) {
    const uint32_t lo = __builtin_amdgcn_perm((uint32_t)c1, (uint32_t)c0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm((uint32_t)c3, (uint32_t)c2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Ties: where |x - c*s| = s/2 exactly and c is odd, the even neighbour c +-
// 1 (toward x) is the rounded code, clamped again.  |e| is the same for both
// neighbours, so the residual statistics need no change.  `lane_tie` flags a
// lane whose largest |e| reached s/2 (ties, and clamped quotients beyond lim +
// 1/2); the pass runs only when some lane of the wave is flagged.
__device__ __forceinline__ void fix_ties(const uint32_t w[4], float cb[8], float s, float hs, float lim,
                                         bool lane_tie) {
    if (__builtin_amdgcn_ballot_w64(lane_tie) == 0) return;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float e = code_residual(elem(w, k), cb[k], s);
        if (__builtin_fabsf(e) == hs && (__float_as_uint(cb[k]) & 1u) != 0)
            cb[k] = __builtin_fminf(__builtin_fmaxf(cb[k] + __builtin_copysignf(1.0f, e), RND_BIAS - lim),
                                    RND_BIAS + lim);
    }
}

// One token row quantized by a group of 16 lanes, for the fused append of one
// token (lane16 holds channels 8*lane16 .. +7; load_row16 lets the caller
// issue the loads early).  Every
// lane returns its 8 key codes (bytes), its 8 value codes (low nibble of each
// byte), the row's key scale and key error, its 32-channel group's value
// scale, and the row's value error (max over the four groups).  Uses
// lane exchanges within the 16-lane group (one DPP row) only.
struct RowQuant {
    uint32_t kc[2], vc[2];
    uint32_t ksb, vsb;
    float kerr, verr;
};

// The raw fp16 channels of one token row held by a lane: keys and values.
struct RowIn {
    uint4 k, v;
};

__device__ __forceinline__ RowIn load_row16(const uint16_t *k16row, const uint16_t *v16row, int lane16) {
    RowIn r;
    r.k = *reinterpret_cast<const uint4 *>(k16row + 8 * lane16);
    r.v = *reinterpret_cast<const uint4 *>(v16row + 8 * lane16);
    return r;
}

// Key row with the Hadamard rotation (KVQ_CODEC_ROTATE_K): u = H k / 16
// over the 16-lane group, in fp64 where every butterfly is exact (k's values
// are multiples of 2^-24 below 2^16, so the sums fit 47 bits and their order
// does not matter): strides 1, 2, 4 in the lane, 8 .. 64 across lanes xor
// 1 .. 8.  Then the key codec on u: the estimate rint(u * RN(1/s)) is within
// one of round_half_even(u / s) (its error is below 2^-44 for |u / s| < 256),
// and the exact residual d = u - c s (u is a multiple of 2^-28 below 2^20,
// s c has at most 19 significant bits) moves it one step toward d when |d| >
// s/2, or when |d| = s/2 and c is odd.  e = u - s c is exact, and the error
// is sqrt(2 * T128(e^2)) with the squares rounded to fp64 (the keys read back
// are H (s c) / 8).
__device__ __forceinline__ void quant_key_rot16(const uint32_t kw[4], bool knonfin, int lane16, uint32_t kc[2],
                                                uint32_t &ksb, float &kerr) {
    double u[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) u[k] = (double)elem(kw, k);
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (!(j & h)) {
                const double x = u[j], y = u[j + h];
                u[j] = x + y;
                u[j + h] = x - y;
            }
    // lane with bit mk clear: u + partner; set: partner - u (exact either way)
#pragma unroll
    for (int mk = 1; mk < 16; mk <<= 1) {
        const double sg = (lane16 & mk) ? -1.0 : 1.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) u[k] = __builtin_fma(u[k], sg, xor16d(u[k], mk));
    }
    double am = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        u[k] = u[k] * 0.0625;
        am = fmax(am, fabs(u[k]));
    }
    // the row max as f32 (rounding is monotonic, so it commutes with the max)
    float amf = (float)am;
#pragma unroll
    for (int mk = 1; mk < 16; mk <<= 1) amf = fmaxf(amf, xor16f(amf, mk));
    ksb = knonfin ? 0u : f2h_rn(__fdiv_rn(amf, 127.0f));
    const double s = (double)h2f(ksb);
    const double rs = s != 0.0 ? 1.0 / s : 0.0, hs = 0.5 * s;
    double sq[8];
    int cc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        double c = __builtin_rint(u[k] * rs);
        const double d = __builtin_fma(-c, s, u[k]);
        const double ad = __builtin_fabs(d);
        const bool odd = (((int)c) & 1) != 0;
        c = (ad > hs || (ad == hs && odd)) ? c + __builtin_copysign(1.0, d) : c;
        c = __builtin_fmin(__builtin_fmax(c, -127.0), 127.0);
        c = s != 0.0 ? c : 0.0;
        const double e = __builtin_fma(-c, s, u[k]);  // exact
        sq[k] = __dmul_rn(e, e);
        cc[k] = (int)c;
    }
    kc[0] = pack_bytes(cc[0], cc[1], cc[2], cc[3]);
    kc[1] = pack_bytes(cc[4], cc[5], cc[6], cc[7]);
    const double ss = tree128(sq);
    kerr = knonfin ? __builtin_huge_valf() : (float)__dsqrt_rn(2.0 * ss);
}

// Max over the 16 lanes of a DPP row, in every lane: xor 1 and xor 2 make
// each quad uniform, then the row rotations by 4 and 8 bring in the other
// three quads.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = umax(v, xor16u(v, 1));
    v = umax(v, xor16u(v, 2));
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
    return v;
}
// The same for non-negative floats (+inf included), whose bit patterns order
// like their values.
__device__ __forceinline__ float row16_max_nonneg(float v) {
    return __uint_as_float(row16_max_u32(__float_as_uint(v)));
}

// One token row.  rot: the key row uses the Hadamard-rotated codec
// (KVQ_CODEC_ROTATE_K).  A row or value group holding Inf or NaN gets scale 0,
// codes 0 and error +inf.
__device__ __forceinline__ RowQuant quant_row16(const RowIn &in, bool rot, int lane16) {
    RowQuant o;
    // ---------------- key row: int8 per token, scale absmax/127
    const uint4 kr = in.k;
    const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
    const uint32_t am = row16_max_u32(absmax_bits(kw));
    const bool knonfin = am >= 0x7C00u;
    uint32_t kc[2] = {0u, 0u};
    uint32_t ksb;
    float kerr;
    if (rot) {
        quant_key_rot16(kw, knonfin, lane16, kc, ksb, kerr);
    } else {
        ksb = knonfin ? 0u : f2h_rn(__fdiv_rn(h2f(am), 127.0f));
        const float ks = h2f(ksb);
        // a zero scale (tiny or all-zero row) gives codes 0
        const float kr_ = ks != 0.0f ? __builtin_amdgcn_rcpf(ks) : 0.0f;
        const float khs = ks != 0.0f ? 0.5f * ks : __builtin_huge_valf();
        double sq[8];
        float cb[8];
        float emax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float x = elem(kw, k);
            cb[k] = code_biased(x, kr_, 127.0f);
            const float e = code_residual(x, cb[k], ks);
            emax = __builtin_fmaxf(emax, __builtin_fabsf(e));
            sq[k] = sq64(e);
        }
        fix_ties(kw, cb, ks, khs, 127.0f, emax >= khs);
        if (__builtin_amdgcn_ballot_w64(knonfin) != 0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) cb[k] = knonfin ? RND_BIAS : cb[k];
        }
        kc[0] = pack_bytes(__float_as_int(cb[0]), __float_as_int(cb[1]), __float_as_int(cb[2]), __float_as_int(cb[3]));
        kc[1] = pack_bytes(__float_as_int(cb[4]), __float_as_int(cb[5]), __float_as_int(cb[6]), __float_as_int(cb[7]));
        const double ss = tree128(sq);
        kerr = knonfin ? __builtin_huge_valf() : (float)__dsqrt_rn(ss);
    }

    // ---------------- value row: int4 per 32-channel group, scale absmax/7
    const uint4 vr = in.v;
    const uint32_t vw[4] = {vr.x, vr.y, vr.z, vr.w};
    uint32_t vm = absmax_bits(vw);
    vm = umax(vm, xor16u(vm, 1));
    vm = umax(vm, xor16u(vm, 2));
    const bool vnonfin = vm >= 0x7C00u;
    const uint32_t vsb = vnonfin ? 0u : f2h_rn(__fdiv_rn(h2f(vm), 7.0f));
    const float vs = h2f(vsb);
    const float vr_ = vs != 0.0f ? __builtin_amdgcn_rcpf(vs) : 0.0f;
    const float vhs = vs != 0.0f ? 0.5f * vs : __builtin_huge_valf();
    float cv[8];
    float verr = 0.0f;  // max |e| over the lane's channels
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float x = elem(vw, k);
        cv[k] = code_biased(x, vr_, 7.0f);
        verr = __builtin_fmaxf(verr, __builtin_fabsf(code_residual(x, cv[k], vs)));
    }
    fix_ties(vw, cv, vs, vhs, 7.0f, verr >= vhs);
    if (__builtin_amdgcn_ballot_w64(vnonfin) != 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) cv[k] = vnonfin ? RND_BIAS : cv[k];
    }
    const uint32_t vc0 = pack_bytes(__float_as_int(cv[0]), __float_as_int(cv[1]), __float_as_int(cv[2]), __float_as_int(cv[3]));
    const uint32_t vc1 = pack_bytes(__float_as_int(cv[4]), __float_as_int(cv[5]), __float_as_int(cv[6]), __float_as_int(cv[7]));
    verr = vnonfin ? __builtin_huge_valf() : verr;
    verr = row16_max_nonneg(verr);  // row: max over the 4 groups

    o.kc[0] = kc[0];
    o.kc[1] = kc[1];
    o.vc[0] = vc0 & 0x0F0F0F0Fu;
    o.vc[1] = vc1 & 0x0F0F0F0Fu;
    o.ksb = ksb;
    o.vsb = vsb;
    o.kerr = kerr;
    o.verr = verr;
    return o;
}

// ---------------------------------------------------------------------------
// One token row quantized by the 4 lanes of a quad (plain codec), for bulk
// appends: four times the channels per lane of quant_row16, so the per-row
// work (absmax, scales, the fp64 tree's tail, the square root) is shared by
// 32 channels instead of 8.  Lane j of the quad holds key channels
// 8j + 32i .. +7 (i = 0..3: the 8-channel chunks j, j+4, j+8, j+12, so that
// the pinned fp64 tree pairs chunks c and c^8, then c^4, inside the lane, and
// c^2, c^1 across it, as tree128 does) and value channels 32j .. 32j+31 (the
// lane's own value group).  Same bytes as quant_row16.
struct Row4In {
    uint4 k[4], v[4];
};
// Scales and errors of a row; the codes go straight to memory.
struct Row4Quant {
    uint32_t ksb, vsb;
    float kerr, verr;
};

__device__ __forceinline__ Row4In load_row4(const uint16_t *k16row, const uint16_t *v16row, int j) {
    Row4In r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.k[i] = *reinterpret_cast<const uint4 *>(k16row + 8 * j + 32 * i);
        r.v[i] = *reinterpret_cast<const uint4 *>(v16row + 32 * j + 8 * i);
    }
    return r;
}

// absmax_bits over the 32 fp16 values of four uint4, on packed 16-bit maxima.
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t absmax_bits32(const uint4 (&q)[4]) {
    ushort2_t m = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2_t, w[k] & 0x7FFF7FFFu));
    }
    return umax(m[0], m[1]);
}

// kdst: the row's key codes + 8j (chunk i at kdst + 32i); vdst: 32 bytes for
// the value group's codes (low nibbles, channel order).
// ROT: the key row uses the Hadamard-rotated codec, u = H k / 16 as in
// quant_key_rot16: butterflies at channel strides 1, 2, 4 inside each chunk,
// 32 and 64 across the lane's chunks, 8 and 16 across the quad (lanes xor 1,
// 2), all exact in fp64, then the same codes, scale and error.
template <bool ROT>
__device__ __forceinline__ Row4Quant quant_row4(const Row4In &in, int8_t *kdst, uint8_t *vdst) {
    Row4Quant o;
    // ---------------- key row: int8 per token, scale absmax/127
    uint32_t am = absmax_bits32(in.k);
    am = umax(am, xor16u(am, 1));
    am = umax(am, xor16u(am, 2));
    const bool knonfin = am >= 0x7C00u;
    if constexpr (ROT) {
        const int j = __lane_id() & 3;
        double u[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w[4] = {in.k[i].x, in.k[i].y, in.k[i].z, in.k[i].w};
#pragma unroll
            for (int k = 0; k < 8; ++k) u[i][k] = (double)elem(w, k);
#pragma unroll
            for (int h = 1; h < 8; h <<= 1)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (!(k & h)) {
                        const double x = u[i][k], y = u[i][k + h];
                        u[i][k] = x + y;
                        u[i][k + h] = x - y;
                    }
        }
#pragma unroll
        for (int h = 1; h < 4; h <<= 1)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!(i & h)) {
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const double x = u[i][k], y = u[i + h][k];
                        u[i][k] = x + y;
                        u[i + h][k] = x - y;
                    }
                }
        // lane with bit mk clear: u + partner; set: partner - u
#pragma unroll
        for (int mk = 1; mk < 4; mk <<= 1) {
            const double sg = (j & mk) ? -1.0 : 1.0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < 8; ++k) u[i][k] = __builtin_fma(u[i][k], sg, xor16d(u[i][k], mk));
        }
        double amd = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                u[i][k] = u[i][k] * 0.0625;
                amd = fmax(amd, fabs(u[i][k]));
            }
        // the row max as f32 (rounding is monotonic, so it commutes with the max)
        uint32_t amb = __float_as_uint((float)amd);
        amb = umax(amb, xor16u(amb, 1));
        amb = umax(amb, xor16u(amb, 2));
        o.ksb = knonfin ? 0u : f2h_rn(__fdiv_rn(__uint_as_float(amb), 127.0f));
        const double s = (double)h2f(o.ksb);
        const double rs = s != 0.0 ? 1.0 / s : 0.0, hs = 0.5 * s;
        double part[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            double sq[8];
            int cc[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                double c = __builtin_rint(u[i][k] * rs);
                const double d = __builtin_fma(-c, s, u[i][k]);
                const double ad = __builtin_fabs(d);
                const bool odd = (((int)c) & 1) != 0;
                c = (ad > hs || (ad == hs && odd)) ? c + __builtin_copysign(1.0, d) : c;
                c = __builtin_fmin(__builtin_fmax(c, -127.0), 127.0);
                c = s != 0.0 ? c : 0.0;
                const double e = __builtin_fma(-c, s, u[i][k]);  // exact
                sq[k] = __dmul_rn(e, e);
                cc[k] = (int)c;
            }
            *reinterpret_cast<uint2 *>(kdst + 32 * i) =
                make_uint2(pack_bytes(cc[0], cc[1], cc[2], cc[3]), pack_bytes(cc[4], cc[5], cc[6], cc[7]));
            part[i] = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
        }
        double ss = (part[0] + part[2]) + (part[1] + part[3]);
        ss = ss + xor16d(ss, 2);
        ss = ss + xor16d(ss, 1);
        o.kerr = knonfin ? __builtin_huge_valf() : (float)__dsqrt_rn(2.0 * ss);
    } else {
        o.ksb = knonfin ? 0u : f2h_rn(__fdiv_rn(h2f(am), 127.0f));
        const float ks = h2f(o.ksb);
        const float kr_ = ks != 0.0f ? __builtin_amdgcn_rcpf(ks) : 0.0f;
        const float khs = ks != 0.0f ? 0.5f * ks : __builtin_huge_valf();
        double part[4];  // fp64 sum of the squared residuals of chunk i (levels 1-3 of the tree)
    #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w[4] = {in.k[i].x, in.k[i].y, in.k[i].z, in.k[i].w};
            float cb[8];
            double sq[8];
            float emax = 0.0f;
    #pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float x = elem(w, k);
                cb[k] = code_biased(x, kr_, 127.0f);
                const float e = code_residual(x, cb[k], ks);
                emax = __builtin_fmaxf(emax, __builtin_fabsf(e));
                sq[k] = sq64(e);
            }
            fix_ties(w, cb, ks, khs, 127.0f, emax >= khs);
            const uint32_t c0 = pack_bytes(__float_as_int(cb[0]), __float_as_int(cb[1]), __float_as_int(cb[2]),
                                           __float_as_int(cb[3]));
            const uint32_t c1 = pack_bytes(__float_as_int(cb[4]), __float_as_int(cb[5]), __float_as_int(cb[6]),
                                           __float_as_int(cb[7]));
            // a row holding Inf/NaN: codes 0
            *reinterpret_cast<uint2 *>(kdst + 32 * i) = knonfin ? make_uint2(0u, 0u) : make_uint2(c0, c1);
            part[i] = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
        }
        // chunks c + c^8 (i, i + 2), then + c^4 (i + 1), then across the quad
        double ss = (part[0] + part[2]) + (part[1] + part[3]);
        ss = ss + xor16d(ss, 2);
        ss = ss + xor16d(ss, 1);
        o.kerr = knonfin ? __builtin_huge_valf() : (float)__dsqrt_rn(ss);
    }

    // ---------------- value group: int4, scale absmax/7
    const uint32_t vm = absmax_bits32(in.v);
    const bool vnonfin = vm >= 0x7C00u;
    o.vsb = vnonfin ? 0u : f2h_rn(__fdiv_rn(h2f(vm), 7.0f));
    const float vs = h2f(o.vsb);
    const float vr_ = vs != 0.0f ? __builtin_amdgcn_rcpf(vs) : 0.0f;
    const float vhs = vs != 0.0f ? 0.5f * vs : __builtin_huge_valf();
    float verr = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {in.v[i].x, in.v[i].y, in.v[i].z, in.v[i].w};
        float cb[8];
        float emax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float x = elem(w, k);
            cb[k] = code_biased(x, vr_, 7.0f);
            emax = __builtin_fmaxf(emax, __builtin_fabsf(code_residual(x, cb[k], vs)));
        }
        fix_ties(w, cb, vs, vhs, 7.0f, emax >= vhs);
        verr = __builtin_fmaxf(verr, emax);
        const uint32_t c0 = pack_bytes(__float_as_int(cb[0]), __float_as_int(cb[1]), __float_as_int(cb[2]),
                                       __float_as_int(cb[3]));
        const uint32_t c1 = pack_bytes(__float_as_int(cb[4]), __float_as_int(cb[5]), __float_as_int(cb[6]),
                                       __float_as_int(cb[7]));
        *reinterpret_cast<uint2 *>(vdst + 8 * i) =
            vnonfin ? make_uint2(0u, 0u) : make_uint2(c0 & 0x0F0F0F0Fu, c1 & 0x0F0F0F0Fu);
    }
    // row: max over the quad's four groups (non-negative: compare bit patterns)
    uint32_t vb = vnonfin ? 0x7F800000u : __float_as_uint(verr);
    vb = umax(vb, xor16u(vb, 1));
    vb = umax(vb, xor16u(vb, 2));
    o.verr = __uint_as_float(vb);
    return o;
}

__device__ __forceinline__ RowQuant quant_row16(const uint16_t *k16row, const uint16_t *v16row, int lane16,
                                                bool rot) {
    return quant_row16(load_row16(k16row, v16row, lane16), rot, lane16);
}

}  // namespace kvq
