// kvq_quantize.hip -- quantize-on-append for the tier-1 cache (gfx950).
//
// "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1: the
// compressed tier holds INT8 keys and INT4 values with their scales and
// per-block error annotations, derived from the FP16 originals kept in tier 2.
//
// One workgroup (256 threads = 4 waves) owns one 64-token block of one
// (batch, KV head), so a block's codes and statistics have a single writer and
// appends of any size compose bit-exactly.  Each token row (128 fp16 = 256 B)
// is handled by 16 lanes that each load 16 B (8 channels); a wave covers 4
// rows per pass, the workgroup 16.  Reductions inside a row are xor-shuffles
// within the 16-lane group: absmax over 16 lanes for the key scale, over 4
// lanes for a 32-channel value group, and the fixed fp64 tree for ||k - k^||.
// Value nibbles are staged as bytes in LDS and packed channel-major on the way
// out; key codes go straight from registers to HBM (128 B per row, coalesced).
#include "kvq_device.hpp"
#include "kvq_internal.hpp"

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

__global__ __launch_bounds__(256) void quantize_append_kernel(AppendArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t vtile[BLK][D];  // new value codes (low nibble), [token][channel]
    __shared__ float red[2][4];

    const int tid = threadIdx.x;
    const int lane16 = tid & 15;
    const int row0 = tid >> 4;  // 0..15
    const int64_t blk = a.blk_lo + blockIdx.x;
    const int64_t head = (int64_t)blockIdx.z * a.hkv + blockIdx.y;
    const int64_t t_first = blk * BLK;
    const int64_t t_begin = a.len0 > t_first ? a.len0 : t_first;
    const int64_t t_end = a.len1 < t_first + BLK ? a.len1 : t_first + BLK;
    const int64_t row_base = head * a.cap;

    float kmax = 0.0f, vmax = 0.0f;

    for (int r = row0; r < BLK; r += 16) {
        const int64_t t = t_first + r;
        // rows outside the appended range are neither read nor written; the
        // test is uniform in the 16-lane group, so the group's shuffles below
        // only ever involve active lanes
        if (t < t_begin || t >= t_end) continue;
        const int64_t roff = (row_base + t) * D + 8 * lane16;

        // ---------------- key row: int8 per token, scale absmax/127
        const uint4 kr = *reinterpret_cast<const uint4 *>(a.c.k16 + roff);
        const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
        uint32_t am = absmax_bits(kw);
        am = umax(am, __shfl_xor(am, 1));
        am = umax(am, __shfl_xor(am, 2));
        am = umax(am, __shfl_xor(am, 4));
        am = umax(am, __shfl_xor(am, 8));
        const bool knonfin = am >= 0x7C00u;
        const uint32_t ksb = knonfin ? 0u : f2h_rn(__fdiv_rn(h2f(am), 127.0f));
        const float ks = h2f(ksb);
        // a zero scale (tiny, all-zero or non-finite row) gives codes 0
        const float kr_ = ks != 0.0f ? __builtin_amdgcn_rcpf(ks) : 0.0f;
        const float khs = ks != 0.0f ? 0.5f * ks : __builtin_huge_valf();
        uint32_t kc[2] = {0u, 0u};
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
        const float kerr = knonfin ? __builtin_huge_valf() : (float)__dsqrt_rn(ss);

        // ---------------- value row: int4 per 32-channel group, scale absmax/7
        const uint4 vr = *reinterpret_cast<const uint4 *>(a.c.v16 + roff);
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

        *reinterpret_cast<uint2 *>(a.c.k_codes + roff) = make_uint2(kc[0], kc[1]);
        if (lane16 == 0) a.c.k_scales[row_base + t] = (uint16_t)ksb;
        if ((lane16 & 3) == 0) a.c.v_scales[(row_base + t) * 4 + (lane16 >> 2)] = (uint16_t)vsb;
        *reinterpret_cast<uint2 *>(&vtile[r][8 * lane16]) = make_uint2(vc[0], vc[1]);
        kmax = fmaxf(kmax, kerr);
        vmax = fmaxf(vmax, verr);
    }

    // block statistics: max over this workgroup's rows, then over old rows
    kmax = fmaxf(kmax, __shfl_xor(kmax, 16));
    kmax = fmaxf(kmax, __shfl_xor(kmax, 32));
    vmax = fmaxf(vmax, __shfl_xor(vmax, 16));
    vmax = fmaxf(vmax, __shfl_xor(vmax, 32));
    if ((tid & 63) == 0) {
        red[0][tid >> 6] = kmax;
        red[1][tid >> 6] = vmax;
    }
    __syncthreads();

    const bool has_old = t_first < a.len0;
    if (tid == 0) {
        float km = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
        float vm2 = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
        const int64_t si = head * (a.cap / BLK) + blk;
        if (has_old) {
            km = fmaxf(km, a.c.k_err[si]);
            vm2 = fmaxf(vm2, a.c.v_err[si]);
        }
        a.c.k_err[si] = km;
        a.c.v_err[si] = vm2;
    }

    // value codes: channel-major nibble pairs, 16 bytes per thread
    {
        const int j = tid >> 1;         // channel
        const int i0 = (tid & 1) * 16;  // first byte (token pair) of this thread
        uint8_t *dst = a.c.v_codes + (head * (a.cap / BLK) + blk) * (D * BLK / 2) + j * (BLK / 2) + i0;
        // tokens [lo, hi) of the block are new, [0, lo) kept, [hi, 64) zero
        const int lo = (int)(t_begin - t_first), hi = (int)(t_end - t_first);
        uint32_t nw[4] = {0u, 0u, 0u, 0u};
        if (lo == 0 && hi == BLK) {
            // the whole block is new: pair the staged low nibbles
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tk = 2 * (i0 + i);
                const uint32_t byte = (vtile[tk][j] & 0x0Fu) | ((uint32_t)(vtile[tk + 1][j] & 0x0Fu) << 4);
                nw[i >> 2] |= byte << (8 * (i & 3));
            }
        } else {
            uint4 old = make_uint4(0, 0, 0, 0);
            if (has_old) old = *reinterpret_cast<const uint4 *>(dst);
            const uint32_t ow[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t byte = 0;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int tk = 2 * (i0 + i) + half;
                    uint32_t nib;
                    if (tk < lo)
                        nib = (ow[i >> 2] >> (8 * (i & 3) + 4 * half)) & 0x0Fu;
                    else if (tk < hi)
                        nib = vtile[tk][j] & 0x0Fu;
                    else
                        nib = 0u;
                    byte |= nib << (4 * half);
                }
                nw[i >> 2] |= byte << (8 * (i & 3));
            }
        }
        *reinterpret_cast<uint4 *>(dst) = make_uint4(nw[0], nw[1], nw[2], nw[3]);
    }
}

hipError_t launch_append(const AppendArgs &a, int batch, int64_t nblk, hipStream_t s) {
    dim3 grid((unsigned)nblk, (unsigned)a.hkv, (unsigned)batch);
    hipLaunchKernelGGL(quantize_append_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
