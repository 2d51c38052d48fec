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
// rows per pass, the workgroup 16, and all four rows of a group are loaded
// before the first is quantized.  Reductions inside a row are lane exchanges
// within the 16-lane group (a DPP row, VALU moves with no LDS round trip):
// absmax over 16 lanes for the key scale, over 4
// lanes for a 32-channel value group, and the fixed fp64 tree for ||k - k^||.
// Value nibbles are staged as bytes in LDS and packed channel-major on the way
// out; key codes go straight from registers to HBM (128 B per row, coalesced).
#include "kvq_internal.hpp"
#include "kvq_quant_row.hpp"

namespace kvq {

template <bool ROT>
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

    // the group's four rows are loaded before any is quantized, so that four
    // loads per lane are in flight; rows outside the appended range are
    // neither read nor written (a one-token append reads one row, also when
    // tier 2 is host memory).  The range test is uniform in the 16-lane group,
    // so the group's shuffles only ever involve active lanes.
    RowIn rin[BLK / 16];
#pragma unroll
    for (int i = 0; i < BLK / 16; ++i) {
        const int64_t t = t_first + row0 + 16 * i;
        rin[i].k = rin[i].v = make_uint4(0u, 0u, 0u, 0u);
        if (t >= t_begin && t < t_end)
            rin[i] = load_row16(a.c.k16 + (row_base + t) * D, a.c.v16 + (row_base + t) * D, lane16);
    }
#pragma unroll
    for (int i = 0; i < BLK / 16; ++i) {
        const int r = row0 + 16 * i;
        const int64_t t = t_first + r;
        if (t < t_begin || t >= t_end) continue;
        const int64_t roff = (row_base + t) * D + 8 * lane16;

        const RowQuant rq = quant_row16(rin[i], ROT, lane16);
        const uint32_t kc[2] = {rq.kc[0], rq.kc[1]}, vc[2] = {rq.vc[0], rq.vc[1]};
        const uint32_t ksb = rq.ksb, vsb = rq.vsb;
        const float kerr = rq.kerr, verr = rq.verr;

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
    if (a.key_rot)
        hipLaunchKernelGGL(quantize_append_kernel<true>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(quantize_append_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
