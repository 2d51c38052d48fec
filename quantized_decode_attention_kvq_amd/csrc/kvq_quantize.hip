// kvq_quantize.hip -- quantize-on-append for the tier-1 cache (gfx950).
//
// "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1: the
// compressed tier holds INT8 keys and INT4 values with their scales and
// per-block error annotations, derived from the FP16 originals kept in tier 2.
//
// One workgroup (256 threads = 4 waves) owns one 64-token block of one
// (batch, KV head), so a block's codes and statistics have a single writer and
// appends of any size compose bit-exactly.  Each token row (128 fp16 = 256 B
// of keys, as much of values) goes to the 4 lanes of a quad, 32 channels per
// lane and tensor, so the workgroup takes the whole block in one pass and the
// per-row work (absmax, scale, the tail of the fp64 tree, the square root; the
// Hadamard butterflies of the rotated codec) is spread over 32 channels.
// Reductions inside a row are lane exchanges on DPP moves (VALU, no LDS round
// trip).  The per-element work is one biased fma for the code, a clamp, an
// exact residual and, for keys, the fp64 square; with 16 lanes per row the
// kernel was bound by VALU issue, with 4 it runs close to the same kernel with
// the arithmetic removed.  Value nibbles are staged as bytes in LDS and packed
// channel-major on the way out; key codes go straight from registers to HBM.
#include "kvq_internal.hpp"
#include "kvq_quant_row.hpp"

namespace kvq {

template <bool ROT>
__global__ __launch_bounds__(256) void quantize_append_kernel(AppendArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t vtile[BLK][D];  // new value codes (low nibble), [token][channel]
    __shared__ float red[2][4];

    const int tid = threadIdx.x;
    const int64_t blk = a.blk_lo + blockIdx.x;
    const int64_t head = (int64_t)blockIdx.z * a.hkv + blockIdx.y;
    const int64_t t_first = blk * BLK;
    const int64_t t_begin = a.len0 > t_first ? a.len0 : t_first;
    const int64_t t_end = a.len1 < t_first + BLK ? a.len1 : t_first + BLK;
    const int64_t row_base = head * a.cap;

    // a block that already holds tokens: its statistics and the thread's 16
    // bytes of value nibbles are loaded with the new rows
    const bool has_old = t_first < a.len0;
    const int64_t si = head * (a.cap / BLK) + blk;
    const int vj = tid & (D - 1);   // the thread's channel in the value packing (a wave reads 64
    const int vi0 = (tid / D) * 16;  // consecutive channels of one token row: no bank conflicts)
    uint8_t *vdst = a.c.v_codes + si * (D * BLK / 2) + vj * (BLK / 2) + vi0;
    float kold = 0.0f, vold = 0.0f;
    uint4 vold16 = make_uint4(0u, 0u, 0u, 0u);
    if (has_old) {
        vold16 = *reinterpret_cast<const uint4 *>(vdst);
        if (tid == 0) {
            kold = a.c.k_err[si];
            vold = a.c.v_err[si];
        }
    }

    float kmax = 0.0f, vmax = 0.0f;

    // one row per quad; wave w takes rows 16w .. 16w+15.  Rows outside the
    // appended range are neither read nor written (a one-token append reads
    // one row, also when tier 2 is host memory); the range test is uniform in
    // the quad, whose lane exchanges only involve active lanes.
    const int j = tid & 3;
    const int r = tid >> 2;  // 0..63
    const int64_t t = t_first + r;
    if (t >= t_begin && t < t_end) {
        const Row4In in = load_row4(a.c.k16 + (row_base + t) * D, a.c.v16 + (row_base + t) * D, j);
        const Row4Quant rq = quant_row4<ROT>(in, a.c.k_codes + (row_base + t) * D + 8 * j, &vtile[r][32 * j]);
        if (j == 0) a.c.k_scales[row_base + t] = (uint16_t)rq.ksb;
        a.c.v_scales[(row_base + t) * 4 + j] = (uint16_t)rq.vsb;
        kmax = rq.kerr;
        vmax = rq.verr;
    }
    // max over the wave's 16 rows (non-negative: bit patterns order like values)
    kmax = __uint_as_float(row16_max_u32(__float_as_uint(kmax)));
    vmax = __uint_as_float(row16_max_u32(__float_as_uint(vmax)));

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

    if (tid == 0) {
        float km = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
        float vm2 = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
        if (has_old) {
            km = fmaxf(km, kold);
            vm2 = fmaxf(vm2, vold);
        }
        a.c.k_err[si] = km;
        a.c.v_err[si] = vm2;
    }

    // value codes: channel-major nibble pairs, 16 bytes per thread
    {
        const int j = vj, i0 = vi0;  // channel, first byte (token pair) of this thread
        uint8_t *dst = vdst;
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
            const uint32_t ow[4] = {vold16.x, vold16.y, vold16.z, vold16.w};
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

// Zeroes n floats of each statistics array (a fill kernel rather than a
// memset node, so that the call can be captured into a graph).
__global__ __launch_bounds__(256) void zero_stats_kernel(float *k_err, float *v_err, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        k_err[i] = 0.0f;
        v_err[i] = 0.0f;
    }
}

hipError_t launch_zero_stats(float *k_err, float *v_err, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t want = (n + 255) / 256;
    const unsigned grid = (unsigned)(want < 1024 ? want : 1024);
    hipLaunchKernelGGL(zero_stats_kernel, dim3(grid), dim3(256), 0, s, k_err, v_err, n);
    return hipGetLastError();
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
