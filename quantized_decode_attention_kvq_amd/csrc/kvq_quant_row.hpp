// kvq_quant_row.hpp -- quantization of one token row of one KV head
// (quantize-on-append), shared by the append kernel and the fused
// append-and-decode path so that both give the same bytes.
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

// round_half_even(x / s) clamped to [-lim, lim], for fp16 values x and s > 0,
// with r ~ 1/s (any estimate within a few ulps) and hs = s/2.  The estimate
// rint(x*r) is off by at most one, and only next to a half-integer; the
// residual x - c*s is exact in fp32 (c*s has at most 19 significant bits, and
// x and c*s lie on the grid of the smaller of their fp16 ulps whenever c is
// nonzero), so comparing it with s/2 -- ties going to the even code --
// corrects the estimate exactly.  r == 0 marks a zero scale.  Returns the
// code; e receives x - c*s for the final (clamped) code, also exact.
__device__ __forceinline__ int quant_code(float x, float s, float r, float hs, int lim, float &e) {
    float c = __builtin_rintf(x * r);
    const float d = __builtin_fmaf(-c, s, x);
    const bool odd = ((int)c & 1) != 0;
    if (d > hs || (d == hs && odd))
        c += 1.0f;
    else if (d < -hs || (d == -hs && odd))
        c -= 1.0f;
    c = __builtin_fminf(__builtin_fmaxf(c, (float)-lim), (float)lim);
    c = r == 0.0f ? 0.0f : c;  // zero scale (also rows holding Inf/NaN): code 0
    e = __builtin_fmaf(-c, s, x);
    return (int)c;
}

// One token row quantized by a group of 16 lanes (lane16 holds channels
// 8*lane16 .. +7; load_row16 lets the caller issue the loads early).  Every
// lane returns its 8 key codes (bytes), its 8 value codes (low nibble of each
// byte), the row's key scale and key error, its 32-channel group's value
// scale, and the row's value error (max over the four groups).  Uses
// xor-shuffles within the 16-lane group only.
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
// 1 .. 8.  Then the key codec on u with the quotient u / s in fp64 (u is a
// multiple of 2^-28, so a quotient that is not a half-integer lies at least
// 2^-43 from one, beyond its fp64 rounding: rint gives the exact round half
// to even), e = u - s c exact, and the error sqrt(2 * T128(e^2)) with the
// squares rounded to fp64 (the keys read back are H (s c) / 8).
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
#pragma unroll
    for (int mk = 1; mk < 16; mk <<= 1) {
        const bool hi = (lane16 & mk) != 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const double o = shfl_xor_d(u[k], mk);
            u[k] = hi ? o - u[k] : u[k] + o;
        }
    }
    double am = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        u[k] = u[k] * 0.0625;
        am = fmax(am, fabs(u[k]));
    }
#pragma unroll
    for (int mk = 1; mk < 16; mk <<= 1) am = fmax(am, shfl_xor_d(am, mk));
    ksb = knonfin ? 0u : f2h_rn(__fdiv_rn((float)am, 127.0f));
    const double s = (double)h2f(ksb);
    kc[0] = kc[1] = 0u;
    double sq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        int c = 0;
        if (s != 0.0) {
            const double qv = __builtin_rint(u[k] / s);
            c = (int)(qv > 127.0 ? 127.0 : (qv < -127.0 ? -127.0 : qv));
        }
        const double e = u[k] - s * (double)c;  // s * c exact: no rounding to fuse
        sq[k] = __dmul_rn(e, e);
        kc[k >> 2] |= ((uint32_t)c & 0xFFu) << (8 * (k & 3));
    }
    const double ss = tree128(sq);
    kerr = knonfin ? __builtin_huge_valf() : (float)__dsqrt_rn(2.0 * ss);
}

// rot: the key row uses the Hadamard-rotated codec (KVQ_CODEC_ROTATE_K).
__device__ __forceinline__ RowQuant quant_row16(const RowIn &in, bool rot, int lane16) {
    RowQuant o;
    // ---------------- key row: int8 per token, scale absmax/127
    const uint4 kr = in.k;
    const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
    uint32_t am = absmax_bits(kw);
    am = umax(am, __shfl_xor(am, 1));
    am = umax(am, __shfl_xor(am, 2));
    am = umax(am, __shfl_xor(am, 4));
    am = umax(am, __shfl_xor(am, 8));
    const bool knonfin = am >= 0x7C00u;
    uint32_t kc[2] = {0u, 0u};
    uint32_t ksb;
    float kerr;
    if (rot) {
        quant_key_rot16(kw, knonfin, lane16, kc, ksb, kerr);
    } else {
        ksb = knonfin ? 0u : f2h_rn(__fdiv_rn(h2f(am), 127.0f));
        const float ks = h2f(ksb);
        // a zero scale (tiny, all-zero or non-finite row) gives codes 0
        const float kr_ = ks != 0.0f ? __builtin_amdgcn_rcpf(ks) : 0.0f;
        const float khs = ks != 0.0f ? 0.5f * ks : __builtin_huge_valf();
        double sq[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float x = elem(kw, k);
            float e;
            const int c = quant_code(x, ks, kr_, khs, 127, e);
            sq[k] = sq64(e);
            kc[k >> 2] |= ((uint32_t)c & 0xFFu) << (8 * (k & 3));
        }
        const double ss = tree128(sq);
        kerr = knonfin ? __builtin_huge_valf() : (float)__dsqrt_rn(ss);
    }

    // ---------------- value row: int4 per 32-channel group, scale absmax/7
    const uint4 vr = in.v;
    const uint32_t vw[4] = {vr.x, vr.y, vr.z, vr.w};
    uint32_t vm = absmax_bits(vw);
    vm = umax(vm, __shfl_xor(vm, 1));
    vm = umax(vm, __shfl_xor(vm, 2));
    const bool vnonfin = vm >= 0x7C00u;
    const uint32_t vsb = vnonfin ? 0u : f2h_rn(__fdiv_rn(h2f(vm), 7.0f));
    const float vs = h2f(vsb);
    const float vr_ = vs != 0.0f ? __builtin_amdgcn_rcpf(vs) : 0.0f;
    const float vhs = vs != 0.0f ? 0.5f * vs : __builtin_huge_valf();
    uint32_t vc[2] = {0u, 0u};
    float verr = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float x = elem(vw, k);
        float e;
        const int c = quant_code(x, vs, vr_, vhs, 7, e);
        e = __builtin_fabsf(e);
        verr = verr > e ? verr : e;
        vc[k >> 2] |= ((uint32_t)c & 0x0Fu) << (8 * (k & 3));
    }
    verr = vnonfin ? __builtin_huge_valf() : verr;
    verr = fmaxf(verr, __shfl_xor(verr, 1));
    verr = fmaxf(verr, __shfl_xor(verr, 2));
    verr = fmaxf(verr, __shfl_xor(verr, 4));  // row: max over the 4 groups
    verr = fmaxf(verr, __shfl_xor(verr, 8));

    o.kc[0] = kc[0];
    o.kc[1] = kc[1];
    o.vc[0] = vc[0];
    o.vc[1] = vc[1];
    o.ksb = ksb;
    o.vsb = vsb;
    o.kerr = kerr;
    o.verr = verr;
    return o;
}

__device__ __forceinline__ RowQuant quant_row16(const uint16_t *k16row, const uint16_t *v16row, int lane16,
                                                bool rot) {
    return quant_row16(load_row16(k16row, v16row, lane16), rot, lane16);
}

}  // namespace kvq
