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

__global__ __launch_bounds__(256) void merge_cert_kernel(DecodeArgs a) {
    __shared__ float wgt[MAX_SPLITS][16];
    __shared__ float2 ml[MAX_SPLITS][16];
    __shared__ float qn_lds[16];
    __shared__ uint8_t flag_lds[16];
    const int64_t kvh = blockIdx.x, b = blockIdx.y;
    const int64_t bh = b * a.hkv + kvh;
    const int g = a.g, S = a.splits;
    const int tid = threadIdx.x;
    const float2 *pml = a.part_ml + bh * S * g;
    for (int i = tid; i < S * g; i += blockDim.x) ml[i / g][i % g] = pml[i];
    {
        // per-head query norm: 16-lane group h holds head h's 128 channels
        const int h = tid >> 4, l16 = tid & 15;
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (h < g) raw = *reinterpret_cast<const uint4 *>(a.q + ((b * a.hq) + kvh * g + h) * D + 8 * l16);
        const float n = qnorm16(raw);  // all 16 lanes of the group take part
        if (l16 == 0 && h < g) qn_lds[h] = n;
    }
    __syncthreads();
    for (int i = tid; i < S * g; i += blockDim.x) {
        const int s = i / g, h = i % g;
        float M = -__builtin_huge_valf();
        for (int r = 0; r < S; ++r) M = fmaxf(M, ml[r][h].x);
        float L = 0.0f;
        for (int r = 0; r < S; ++r)
            if (ml[r][h].x != -__builtin_huge_valf()) L += ml[r][h].y * __builtin_amdgcn_exp2f(ml[r][h].x - M);
        const float m_s = ml[s][h].x;
        wgt[s][h] = (L > 0.0f && m_s != -__builtin_huge_valf()) ? __builtin_amdgcn_exp2f(m_s - M) / L : 0.0f;
    }
    if (tid < g) {
        const int h = tid;
        float M = -__builtin_huge_valf();
        for (int r = 0; r < S; ++r) M = fmaxf(M, ml[r][h].x);
        double L = 0.0, E = 0.0;
        float smax = 0.0f, amax = 0.0f;
        for (int r = 0; r < S; ++r) {
            if (ml[r][h].x != -__builtin_huge_valf()) {
                const double f = (double)__builtin_amdgcn_exp2f(ml[r][h].x - M);
                L += (double)ml[r][h].y * f;
                E += (double)a.part_e[(bh * S + r) * g + h] * f;
            }
            const float2 sa = a.part_sa[bh * S + r];
            smax = fmaxf(smax, sa.x);
            amax = (sa.y != sa.y || sa.y > amax) ? sa.y : amax;  // a NaN value keeps the certificate NaN
        }
        const float2 kv = a.part_kv[bh];
        const double e_val = L > 0.0 ? E / L : 0.0;
        const double delta = (double)key_bound(a.sm, qn_lds[h], kv.x);
        const double r1 = 7.0 * (double)smax + (double)kv.y;
        const double range = 2.0 * ((double)amax != (double)amax || (double)amax > r1 ? (double)amax : r1);
        const double c = tanh(0.5 * delta) * range + e_val;
        float cf = (float)c;
        if ((double)cf < c) cf = __uint_as_float(__float_as_uint(cf) + 1u);  // c >= 0: the next float up
        const int64_t oh = b * a.hq + kvh * g + h;
        a.cert[oh] = cf;
        const uint8_t fl = cf > a.tau_out ? 1 : 0;
        a.flags[oh] = fl;
        flag_lds[h] = fl;
    }
    __syncthreads();
    if (tid == 0) {
        uint8_t any = 0;
        for (int h = 0; h < g; ++h) any |= flag_lds[h];
        a.gate_out[bh] = any;
    }
    const float *pacc = a.part_acc + bh * S * g * D;
    for (int idx = tid; idx < g * D; idx += blockDim.x) {
        const int h = idx / D;
        float o = 0.0f;
        for (int s = 0; s < S; ++s) o += wgt[s][h] * pacc[(int64_t)s * g * D + idx];
        a.out[((b * a.hq) + kvh * g) * D + idx] = (uint16_t)f2h_rn(o);
    }
}

}  // namespace

hipError_t launch_merge_cert(const DecodeArgs &a, int batch, hipStream_t s) {
    hipLaunchKernelGGL(merge_cert_kernel, dim3((unsigned)a.hkv, (unsigned)batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
