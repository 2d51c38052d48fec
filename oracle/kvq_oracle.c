/*
 * kvq_oracle.c -- plain CPU oracle for certified quantized-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it and shares no code,
 * header, table or helper with it.
 *
 * Source of the method: "Runtime-Certified Bounded-Error Quantized Attention"
 * (gist.science explainer of arXiv 2605.20868), technical summary:
 *   - Methodology 1, "Tiered Storage with Deterministic Fallback": tier 1 holds
 *     INT8 keys and INT4 values with scales and per-block error annotations;
 *     tier 2 holds the FP16 originals used as ground truth for fallback.
 *   - Methodology 2, "Two-Term Error Decomposition": a key term driven by the
 *     per-token score perturbation and a value term driven by per-block value
 *     reconstruction errors, both computed online from scales and query norms.
 *   - Key Contributions, "Deterministic Recovery": when a bound cannot be met
 *     the exact dense FP16 result is recovered.
 * The page prints no formulas or constants for these steps.  The readings this
 * oracle implements (each listed in the design notes) are:
 *   K codec  : int8 per token and KV head, fp16 scale s = f16(f32(absmax)/127),
 *              c = clamp(RNE(x/s), -127, 127); s == 0 gives c == 0.
 *   V codec  : int4 per token and 32-channel group, fp16 scale
 *              s = f16(f32(absmax)/7), c = clamp(RNE(x/s), -7, 7).
 *   non-finite rows/groups: codes 0, scale 0, error +Inf (forces fallback).
 *   key error  k_err(token) = f32(sqrt(T128(e_j^2))), e = x - s*c (exact);
 *   value error v_err(token) = max_j |x_j - s*c_j| (exact);
 *   block statistics = max over the block's valid tokens.
 *   query norm qn_h = f32(sqrt(T128(q_j^2))); qn(b,kvh) = max over its group.
 *   key bound  KB = ((sm*qn)*k_err)*(1+2^-16) in fp32 (Cauchy-Schwarz on the
 *              logit perturbation, inflated past fp32 rounding);
 *   value bound VB = v_err;
 *   fallback   fb_k = !(KB finite and KB <= tau_k), likewise fb_v with VB
 *              and tau_v, per (batch, kv head, 64-token block).
 *   attention  fp64 softmax attention over k~ = fb_k ? K16 : s*c and
 *              v~ = fb_v ? V16 : s*c, tokens t < length.
 * T128 is a pinned fp64 summation tree over 128 terms: within each run of 8
 * contiguous terms, pairwise with strides 1, 2, 4; then across the 16 run sums
 * with strides 64, 32, 16, 8 (in terms).  Every element pair it adds is fixed,
 * so the result is a fixed function of the inputs.
 *
 * Physical layouts (per batch b and KV head h; cap = capacity, a multiple of 64):
 *   k16, v16  : uint16 fp16 bits [B][Hkv][cap][128]
 *   k_codes   : int8  [B][Hkv][cap][128]
 *   k_scales  : fp16  [B][Hkv][cap]
 *   v_codes   : uint8 [B][Hkv][cap/64][128][32]  per 64-token block, channel-
 *               major: byte (j, i) holds token 2i of channel j in its low
 *               nibble and token 2i+1 in its high nibble, two's complement.
 *               Nibbles of tokens >= length inside a written block are 0.
 *   v_scales  : fp16  [B][Hkv][cap][4]
 *   k_err, v_err : float [B][Hkv][cap/64]
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D 128
#define BLK 64
#define VG 32

/* Number of threads the OpenMP loops below use (1 without OpenMP). */
int kvqo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- fp16 */

/* Exact value of an IEEE binary16 bit pattern. */
double kvqo_f16_to_f64(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp((double)(m + 1024), e - 25);
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even (IEEE 754). */
uint16_t kvqo_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f))
        return sign | 0x7E00;
    double x = fabs((double)f);
    if (x == 0.0)
        return sign;
    if (isinf(f))
        return sign | 0x7C00;
    int E;
    frexp(x, &E);
    E -= 1; /* x in [2^E, 2^(E+1)) */
    if (E < -14) {
        /* subnormal range: multiples of 2^-24; r == 1024 is the least normal */
        double r = nearbyint(ldexp(x, 24));
        return sign | (uint16_t)r;
    }
    double r = nearbyint(ldexp(x, 10 - E)); /* 11-bit significand, RNE */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)r - 1024));
}

/* Element-wise kvqo_f32_to_f16 over n values. */
void kvqo_f32_to_f16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = kvqo_f32_to_f16(in[i]);
}

/* ---------------------------------------------------------------- T128 */

/* The pinned fp64 summation tree over 128 terms (see header). */
double kvqo_tree128(const double *in)
{
    double v[D];
    memcpy(v, in, sizeof v);
    for (int st = 1; st <= 4; st *= 2)
        for (int i = 0; i < D; i += 2 * st)
            v[i] += v[i + st];
    for (int st = 64; st >= 8; st /= 2)
        for (int i = 0; i < st; i += 8)
            v[i] += v[i + st];
    return v[0];
}

/* ||q||_2 of one 128-channel fp16 query row: f32(sqrt(T128(q_j^2))). */
float kvqo_qnorm(const uint16_t *q)
{
    double sq[D];
    for (int j = 0; j < D; ++j) {
        double x = kvqo_f16_to_f64(q[j]);
        sq[j] = x * x; /* exact: 22 significant bits */
    }
    return (float)sqrt(kvqo_tree128(sq));
}

/* ---------------------------------------------------------------- codec */

/* RNE(x / s) for fp16-valued x and s != 0: IEEE binary32 division then rint.
 * The division's rounding cannot move the quotient across a half-integer
 * (the quotient of two 11-bit significands is at least 2^-12 away from any
 * half-integer it does not equal), so this is RNE of the exact quotient. */
static int rne_div(double x, float s)
{
    float q = (float)x / s;
    return (int)rintf(q);
}

static int clampi(int c, int lo, int hi) { return c < lo ? lo : (c > hi ? hi : c); }

/* Quantize one key row of 128 fp16 values. */
void kvqo_quant_k_row(const uint16_t *x16, int8_t *codes, uint16_t *scale, float *err)
{
    double x[D];
    double a = 0.0;
    int finite = 1;
    for (int j = 0; j < D; ++j) {
        x[j] = kvqo_f16_to_f64(x16[j]);
        if (!isfinite(x[j]))
            finite = 0;
        else if (fabs(x[j]) > a)
            a = fabs(x[j]);
    }
    if (!finite) {
        memset(codes, 0, D);
        *scale = 0;
        *err = INFINITY;
        return;
    }
    uint16_t sh = kvqo_f32_to_f16((float)a / 127.0f);
    double s = kvqo_f16_to_f64(sh);
    double sq[D];
    for (int j = 0; j < D; ++j) {
        int c = (s == 0.0) ? 0 : clampi(rne_div(x[j], (float)s), -127, 127);
        double e = x[j] - s * (double)c; /* exact in fp64 (and in fp32) */
        codes[j] = (int8_t)c;
        sq[j] = e * e;                   /* exact: at most 48 significant bits */
    }
    *scale = sh;
    *err = (float)sqrt(kvqo_tree128(sq));
}

/* Walsh-Hadamard transform of 128 values in place, Sylvester order:
 * out_j = sum_i (-1)^popcount(i & j) in_i, by butterflies at strides 1 .. 64.
 * Exact in fp64 for the rows below (every partial sum fits the significand),
 * so the order of the butterflies does not matter. */
static void wht128(double *x)
{
    for (int h = 1; h < D; h <<= 1)
        for (int i = 0; i < D; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                double a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
}

/* Quantize one key row with the Hadamard rotation (outlier-aware codec: the
 * Walsh-Hadamard transform applied before scalar quantization in the KQV
 * scheme of "Statistical Inference and Quality Measures of KV Cache
 * Quantisations Inspired by TurboQuant", technical summary, quantisation
 * schemes, whose results credit it with robustness to heavy tails; read here
 * as a rotation of the keys alone, the values keeping their codec).  u = H k / 16 (exact in fp64: k's
 * values are multiples of 2^-24 below 2^16, so the sums fit 47 bits); the
 * key codec on u: s = f16(f32(max|u|) / 127), c = clamp(RNE(u / s), -127,
 * 127) with the quotient in fp64 (u is a multiple of 2^-28, so a quotient
 * that is not a half-integer lies at least 2^-43 from one, well beyond its
 * fp64 rounding); e = u - s c (exact).  The decode's key is k~ = H (s c) / 8,
 * so ||k - k~|| = sqrt(128) ||e|| / 8 = sqrt(2) ||e||, and the row's error is
 * f32(sqrt(2 * T128(e^2))). */
void kvqo_quant_k_row_rot(const uint16_t *x16, int8_t *codes, uint16_t *scale, float *err)
{
    double u[D];
    int finite = 1;
    for (int j = 0; j < D; ++j) {
        u[j] = kvqo_f16_to_f64(x16[j]);
        if (!isfinite(u[j]))
            finite = 0;
    }
    if (!finite) {
        memset(codes, 0, D);
        *scale = 0;
        *err = INFINITY;
        return;
    }
    wht128(u);
    double a = 0.0;
    for (int j = 0; j < D; ++j) {
        u[j] /= 16.0;
        if (fabs(u[j]) > a)
            a = fabs(u[j]);
    }
    uint16_t sh = kvqo_f32_to_f16((float)a / 127.0f);
    double s = kvqo_f16_to_f64(sh);
    double sq[D];
    for (int j = 0; j < D; ++j) {
        int c = (s == 0.0) ? 0 : clampi((int)rint(u[j] / s), -127, 127);
        double e = u[j] - s * (double)c;
        codes[j] = (int8_t)c;
        sq[j] = e * e;
    }
    *scale = sh;
    *err = (float)sqrt(2.0 * kvqo_tree128(sq));
}

/* The key the decode uses for a row of codes: s c, or with the rotation
 * H (s c) / 8 = s (H c) / 8 (H c is an integer below 2^14: exact). */
static void dequant_key_row(const int8_t *codes, uint16_t scale, int key_rot, double *out)
{
    double s = kvqo_f16_to_f64(scale);
    if (!key_rot) {
        for (int j = 0; j < D; ++j)
            out[j] = s * (double)codes[j];
        return;
    }
    for (int j = 0; j < D; ++j)
        out[j] = (double)codes[j];
    wht128(out);
    for (int j = 0; j < D; ++j)
        out[j] = s * out[j] / 8.0;
}

/* Quantize one value row: 4 groups of 32 channels.  Writes 128 int4 codes as
 * ints in [-7, 7], 4 scales, and returns the row's max |v - v^|. */
void kvqo_quant_v_row(const uint16_t *x16, int8_t *codes, uint16_t *scales, float *err)
{
    double row_err = 0.0;
    for (int g = 0; g < D / VG; ++g) {
        double x[VG];
        double a = 0.0;
        int finite = 1;
        for (int j = 0; j < VG; ++j) {
            x[j] = kvqo_f16_to_f64(x16[g * VG + j]);
            if (!isfinite(x[j]))
                finite = 0;
            else if (fabs(x[j]) > a)
                a = fabs(x[j]);
        }
        if (!finite) {
            for (int j = 0; j < VG; ++j)
                codes[g * VG + j] = 0;
            scales[g] = 0;
            row_err = INFINITY;
            continue;
        }
        uint16_t sh = kvqo_f32_to_f16((float)a / 7.0f);
        double s = kvqo_f16_to_f64(sh);
        scales[g] = sh;
        for (int j = 0; j < VG; ++j) {
            int c = (s == 0.0) ? 0 : clampi(rne_div(x[j], (float)s), -7, 7);
            double e = fabs(x[j] - s * (double)c); /* exact */
            codes[g * VG + j] = (int8_t)c;
            if (e > row_err)
                row_err = e;
        }
    }
    *err = (float)row_err;
}

/* ---------------------------------------------------------------- cache */

static size_t row_index(int b, int h, int64_t t, int Hkv, int64_t cap)
{
    return ((size_t)b * Hkv + h) * (size_t)cap + (size_t)t;
}

static size_t blk_index(int b, int h, int64_t blk, int Hkv, int64_t cap)
{
    return ((size_t)b * Hkv + h) * (size_t)(cap / BLK) + (size_t)blk;
}

/* Byte offset of (token t, channel j) in v_codes, and whether it is the high
 * nibble. */
static size_t v_byte(int b, int h, int64_t t, int j, int Hkv, int64_t cap, int *high)
{
    *high = (int)(t & 1);
    return blk_index(b, h, t / BLK, Hkv, cap) * (size_t)(D * BLK / 2) + (size_t)j * (BLK / 2) +
           (size_t)((t % BLK) / 2);
}

/* Quantize tokens [0, length) of every (b, kv head) from scratch.  Blocks that
 * hold at least one valid token get their statistics and v_codes bytes fully
 * defined; other blocks are left untouched. */
void kvqo_quantize_cache(int B, int Hkv, int64_t cap, int64_t length, const uint16_t *k16,
                         const uint16_t *v16, int8_t *k_codes, uint16_t *k_scales, uint8_t *v_codes,
                         uint16_t *v_scales, float *k_err, float *v_err, int key_rot)
{
    int64_t nblk = (length + BLK - 1) / BLK;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h)
            for (int64_t blk = 0; blk < nblk; ++blk) {
                float kmax = 0.0f, vmax = 0.0f;
                int high;
                size_t byte0 = v_byte(b, h, blk * BLK, 0, Hkv, cap, &high);
                memset(v_codes + byte0, 0, D * BLK / 2);
                for (int64_t t = blk * BLK; t < length && t < (blk + 1) * BLK; ++t) {
                    size_t r = row_index(b, h, t, Hkv, cap);
                    float ke, ve;
                    if (key_rot)
                        kvqo_quant_k_row_rot(k16 + r * D, k_codes + r * D, k_scales + r, &ke);
                    else
                        kvqo_quant_k_row(k16 + r * D, k_codes + r * D, k_scales + r, &ke);
                    int8_t vc[D];
                    kvqo_quant_v_row(v16 + r * D, vc, v_scales + r * (D / VG), &ve);
                    for (int j = 0; j < D; ++j) {
                        size_t o = v_byte(b, h, t, j, Hkv, cap, &high);
                        uint8_t nib = (uint8_t)vc[j] & 0x0F;
                        v_codes[o] |= high ? (uint8_t)(nib << 4) : nib;
                    }
                    if (ke > kmax)
                        kmax = ke;
                    if (ve > vmax)
                        vmax = ve;
                }
                size_t s = blk_index(b, h, blk, Hkv, cap);
                k_err[s] = kmax;
                v_err[s] = vmax;
            }
}

/* ---------------------------------------------------------------- bounds */

/* Per-(b, kv head) group query norm: max over the G heads of the group
 * (heads h*G .. h*G+G-1); NaN if any head's norm is NaN. */
float kvqo_group_qnorm(const uint16_t *q, int b, int h, int Hq, int G)
{
    float qn = 0.0f;
    int any_nan = 0;
    for (int g = 0; g < G; ++g) {
        float n = kvqo_qnorm(q + ((size_t)b * Hq + (size_t)h * G + g) * D);
        if (isnan(n))
            any_nan = 1;
        else if (n > qn)
            qn = n;
    }
    return any_nan ? NAN : qn;
}

/* Key bound of one block: ((sm*qn)*k_err)*(1+2^-16), fp32, left to right.
 * volatile stores force each product to be rounded to binary32. */
float kvqo_key_bound(float sm, float qn, float kerr)
{
    volatile float p1 = sm * qn;
    volatile float p2 = p1 * kerr;
    volatile float p3 = p2 * (1.0f + 0x1p-16f);
    return p3;
}

/* A block keeps its quantized tile only when its bound is certified: finite
 * and not above the tolerance.  NaN or +Inf bounds (non-finite inputs) always
 * fall back, whatever the tolerance. */
static int falls_back(float bound, float tau)
{
    return !(isfinite(bound) && bound <= tau);
}

void kvqo_bounds(int B, int Hq, int Hkv, int64_t cap, int64_t length, const uint16_t *q, float sm,
                 float tau_k, float tau_v, const float *k_err, const float *v_err, float *kb,
                 float *vb, uint8_t *mask)
{
    int G = Hq / Hkv;
    int64_t nblk = (length + BLK - 1) / BLK;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h) {
            float qn = kvqo_group_qnorm(q, b, h, Hq, G);
            for (int64_t blk = 0; blk < nblk; ++blk) {
                size_t s = blk_index(b, h, blk, Hkv, cap);
                size_t o = ((size_t)b * Hkv + h) * (size_t)nblk + (size_t)blk;
                float kbv = kvqo_key_bound(sm, qn, k_err[s]);
                float vbv = v_err[s];
                uint8_t m = (uint8_t)(falls_back(kbv, tau_k) | (falls_back(vbv, tau_v) << 1));
                if (kb)
                    kb[o] = kbv;
                if (vb)
                    vb[o] = vbv;
                if (mask)
                    mask[o] = m;
            }
        }
}

/* ---------------------------------------------------------------- attention */

/* fp64 attention for every (b, query head).  out: double [B][Hq][128];
 * mask: uint8 [B][Hkv][ceil(length/64)] (bit0 key fallback, bit1 value
 * fallback).  length == 0 gives a zero output. */
void kvqo_attention(int B, int Hq, int Hkv, int64_t cap, int64_t length, const uint16_t *q, float sm,
                    float tau_k, float tau_v, const uint16_t *k16, const uint16_t *v16,
                    const int8_t *k_codes, const uint16_t *k_scales, const uint8_t *v_codes,
                    const uint16_t *v_scales, const float *k_err, const float *v_err, double *out,
                    uint8_t *mask, int key_rot)
{
    int G = Hq / Hkv;
    int64_t nblk = (length + BLK - 1) / BLK;
    uint8_t *m = mask ? mask : (uint8_t *)malloc((size_t)B * Hkv * (size_t)(nblk ? nblk : 1));
    kvqo_bounds(B, Hq, Hkv, cap, length, q, sm, tau_k, tau_v, k_err, v_err, NULL, NULL, m);

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int hq = 0; hq < Hq; ++hq) {
            int h = hq / G;
            double qv[D];
            for (int j = 0; j < D; ++j)
                qv[j] = kvqo_f16_to_f64(q[((size_t)b * Hq + hq) * D + j]);
            double *o = out + ((size_t)b * Hq + hq) * D;
            for (int j = 0; j < D; ++j)
                o[j] = 0.0;
            if (length == 0)
                continue;
            double *logit = (double *)malloc(sizeof(double) * (size_t)length);
            double mx = -INFINITY;
            for (int64_t t = 0; t < length; ++t) {
                size_t r = row_index(b, h, t, Hkv, cap);
                int fbk = m[((size_t)b * Hkv + h) * (size_t)nblk + (size_t)(t / BLK)] & 1;
                double kr[D];
                if (!fbk)
                    dequant_key_row(k_codes + r * D, k_scales[r], key_rot, kr);
                double acc = 0.0;
                for (int j = 0; j < D; ++j) {
                    double k = fbk ? kvqo_f16_to_f64(k16[r * D + j]) : kr[j];
                    acc += qv[j] * k;
                }
                logit[t] = (double)sm * acc;
                if (logit[t] > mx)
                    mx = logit[t];
            }
            double wsum = 0.0;
            for (int64_t t = 0; t < length; ++t) {
                size_t r = row_index(b, h, t, Hkv, cap);
                int fbv = (m[((size_t)b * Hkv + h) * (size_t)nblk + (size_t)(t / BLK)] >> 1) & 1;
                double w = exp(logit[t] - mx);
                wsum += w;
                for (int j = 0; j < D; ++j) {
                    double v;
                    if (fbv) {
                        v = kvqo_f16_to_f64(v16[r * D + j]);
                    } else {
                        int high;
                        size_t ob = v_byte(b, h, t, j, Hkv, cap, &high);
                        int nib = high ? (v_codes[ob] >> 4) : (v_codes[ob] & 0x0F);
                        int c = nib >= 8 ? nib - 16 : nib;
                        v = kvqo_f16_to_f64(v_scales[r * (D / VG) + j / VG]) * (double)c;
                    }
                    o[j] += w * v;
                }
            }
            for (int j = 0; j < D; ++j)
                o[j] /= wsum;
            free(logit);
        }
    if (!mask)
        free(m);
}

/* ------------------------------------------------------------ certificate */

/* Per-head output certificate and per-head recompute ("Runtime-Certified
 * Bounded-Error Quantized Attention", technical summary, Methodology 2,
 * "Two-Term Error Decomposition", and Methodology 3, rung 3 of the fallback
 * ladder, "Per-Head Fallback").  For every (b, query head h):
 *   p^   : the softmax weights of the decode above (keys k~ per the masks);
 *   o^   : sum_t p^_t v~_t, the decode output;
 *   o    : the dense output over the FP16 keys and values.
 * Reading of the two terms (the page names them, prints no formula):
 *   key term   E_key = tanh(Delta/2) * R.  Every key-certified block moves a
 *              logit by at most its key bound for this head,
 *              kvqo_key_bound(sm, qn_h, k_err) (Cauchy-Schwarz with qn_h this
 *              head's own norm; the fp32 product's 2^-16 inflation covers the
 *              rounding of the stored norm and error), fallback blocks not at
 *              all, so all logit moves lie in [-Delta, Delta] with
 *              Delta = kvqo_key_bound(sm, qn_h, max{k_err_b : b key-certified});
 *              then the total
 *              variation between the dense and the decode softmax is at most
 *              tanh(Delta/2), and sum_t (p_t - p^_t) v_tj is at most that times
 *              the range of channel j over the tokens, bounded by
 *              R = 2*max(7*S + eta_max, A): S is the largest value scale of a
 *              value-certified token (|v~| <= 7*S there), eta_max the largest
 *              v_err of a value-certified block (|v - v~| <= eta_max), A the
 *              largest |v| of a value-fallback token.
 *   value term E_val = sum over value-certified blocks b of m^_b * v_err_b,
 *              m^_b = sum_{t in b} p^_t, which bounds sum_t p^_t (v_t - v~_t).
 * Since o - o^ = sum_t (p_t - p^_t) v_t + sum_t p^_t (v_t - v~_t), every
 * |o_j - o^_j| <= cert = E_key + E_val (exact arithmetic).
 * Rung 3: a head with cert > tau_out is recomputed on the FP16 keys and
 * values: its output is o and recomputed[h] = 1.
 * out, cert, e_key, e_val: double [B][Hq](x128 for out); recomputed uint8
 * [B][Hq].  length == 0 gives zeros. */
static void certify_masked(int B, int Hq, int Hkv, int64_t cap, int64_t length, const uint16_t *q,
                           float sm, const uint8_t *m, double tau_out, const uint8_t *force,
                           const uint16_t *k16, const uint16_t *v16, const int8_t *k_codes,
                           const uint16_t *k_scales, const uint8_t *v_codes, const uint16_t *v_scales,
                           const float *k_err, const float *v_err, double *out, double *cert,
                           double *e_key, double *e_val, uint8_t *recomputed, int key_rot);

void kvqo_certificate(int B, int Hq, int Hkv, int64_t cap, int64_t length, const uint16_t *q,
                      float sm, float tau_k, float tau_v, double tau_out, const uint16_t *k16,
                      const uint16_t *v16, const int8_t *k_codes, const uint16_t *k_scales,
                      const uint8_t *v_codes, const uint16_t *v_scales, const float *k_err,
                      const float *v_err, double *out, double *cert, double *e_key, double *e_val,
                      uint8_t *recomputed, int key_rot)
{
    int64_t nblk = (length + BLK - 1) / BLK;
    uint8_t *m = (uint8_t *)malloc((size_t)B * Hkv * (size_t)(nblk ? nblk : 1));
    kvqo_bounds(B, Hq, Hkv, cap, length, q, sm, tau_k, tau_v, k_err, v_err, NULL, NULL, m);
    certify_masked(B, Hq, Hkv, cap, length, q, sm, m, tau_out, NULL, k16, v16, k_codes, k_scales,
                   v_codes, v_scales, k_err, v_err, out, cert, e_key, e_val, recomputed, key_rot);
    free(m);
}

/* The decode over the fallback masks m ([B][Hkv][nblk]), its certificate,
 * and the FP16 recompute of the heads whose certificate exceeds tau_out or
 * whose force[b][h] is set (force may be NULL). */
static void certify_masked(int B, int Hq, int Hkv, int64_t cap, int64_t length, const uint16_t *q,
                           float sm, const uint8_t *m, double tau_out, const uint8_t *force,
                           const uint16_t *k16, const uint16_t *v16, const int8_t *k_codes,
                           const uint16_t *k_scales, const uint8_t *v_codes, const uint16_t *v_scales,
                           const float *k_err, const float *v_err, double *out, double *cert,
                           double *e_key, double *e_val, uint8_t *recomputed, int key_rot)
{
    int G = Hq / Hkv;
    int64_t nblk = (length + BLK - 1) / BLK;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int hq = 0; hq < Hq; ++hq) {
            int h = hq / G;
            size_t oi = (size_t)b * Hq + hq;
            const uint8_t *mb = m + ((size_t)b * Hkv + h) * (size_t)nblk;
            double qv[D];
            for (int j = 0; j < D; ++j)
                qv[j] = kvqo_f16_to_f64(q[oi * D + j]);
            double *o = out + oi * D;
            for (int j = 0; j < D; ++j)
                o[j] = 0.0;
            cert[oi] = e_key[oi] = e_val[oi] = 0.0;
            recomputed[oi] = 0;
            if (length == 0)
                continue;
            /* the decode's weights and output */
            double *logit = (double *)malloc(sizeof(double) * (size_t)length);
            double *dlogit = (double *)malloc(sizeof(double) * (size_t)length);
            double mx = -INFINITY, dmx = -INFINITY;
            for (int64_t t = 0; t < length; ++t) {
                size_t r = row_index(b, h, t, Hkv, cap);
                int fbk = mb[t / BLK] & 1;
                double kr[D];
                if (!fbk)
                    dequant_key_row(k_codes + r * D, k_scales[r], key_rot, kr);
                double acc = 0.0, dacc = 0.0;
                for (int j = 0; j < D; ++j) {
                    double k16v = kvqo_f16_to_f64(k16[r * D + j]);
                    double k = fbk ? k16v : kr[j];
                    acc += qv[j] * k;
                    dacc += qv[j] * k16v;
                }
                logit[t] = (double)sm * acc;
                dlogit[t] = (double)sm * dacc;
                if (logit[t] > mx)
                    mx = logit[t];
                if (dlogit[t] > dmx)
                    dmx = dlogit[t];
            }
            double wsum = 0.0, dsum = 0.0;
            for (int64_t t = 0; t < length; ++t) {
                wsum += exp(logit[t] - mx);
                dsum += exp(dlogit[t] - dmx);
            }
            double od[D];
            for (int j = 0; j < D; ++j)
                od[j] = 0.0;
            double kmax = 0.0, etamax = 0.0, smax = 0.0, amax = 0.0, ev = 0.0;
            double mass = 0.0; /* m^ of the current block */
            for (int64_t t = 0; t < length; ++t) {
                size_t r = row_index(b, h, t, Hkv, cap);
                int64_t blk = t / BLK;
                int fbk = mb[blk] & 1, fbv = (mb[blk] >> 1) & 1;
                size_t si = blk_index(b, h, blk, Hkv, cap);
                double p = exp(logit[t] - mx) / wsum;
                double pd = exp(dlogit[t] - dmx) / dsum;
                if (!fbk && (double)k_err[si] > kmax)
                    kmax = (double)k_err[si];
                if (!fbv && (double)v_err[si] > etamax)
                    etamax = (double)v_err[si];
                for (int g = 0; g < D / VG; ++g) {
                    double sv = kvqo_f16_to_f64(v_scales[r * (D / VG) + g]);
                    if (!fbv && sv > smax)
                        smax = sv;
                }
                for (int j = 0; j < D; ++j) {
                    double v16j = kvqo_f16_to_f64(v16[r * D + j]);
                    double v;
                    if (fbv) {
                        v = v16j;
                        if (fabs(v16j) > amax)
                            amax = fabs(v16j);
                    } else {
                        int high;
                        size_t ob = v_byte(b, h, t, j, Hkv, cap, &high);
                        int nib = high ? (v_codes[ob] >> 4) : (v_codes[ob] & 0x0F);
                        int c = nib >= 8 ? nib - 16 : nib;
                        v = kvqo_f16_to_f64(v_scales[r * (D / VG) + j / VG]) * (double)c;
                    }
                    o[j] += p * v;
                    od[j] += pd * v16j;
                }
                /* value term: the block's mass times its value error */
                mass += p;
                if (t % BLK == BLK - 1 || t == length - 1) {
                    if (!fbv)
                        ev += mass * (double)v_err[si];
                    mass = 0.0;
                }
            }
            double qn = (double)kvqo_qnorm(q + oi * D);
            /* every logit move of a key-certified token is at most the key
             * bound of its block's error, hence of the largest such error */
            double delta = (double)kvqo_key_bound(sm, (float)qn, (float)kmax);
            double r2 = 7.0 * smax + etamax;
            double rng = 2.0 * (r2 > amax ? r2 : amax);
            double ek = tanh(delta / 2.0) * rng;
            e_key[oi] = ek;
            e_val[oi] = ev;
            cert[oi] = ek + ev;
            if (cert[oi] > tau_out || (force && force[oi])) {
                recomputed[oi] = 1;
                for (int j = 0; j < D; ++j)
                    o[j] = od[j];
            }
            free(logit);
            free(dlogit);
        }
}

/* The decode, certificate and rung-3 recompute under fallback masks given by
 * the caller (m: uint8 [B][Hkv][nblk], bit 0 keys, bit 1 values from FP16)
 * rather than formed from the bounds, with the recompute also forced where
 * force[b][h] is set (force may be NULL).  Lets a caller evaluate the method
 * under another side's decisions (promotions taken on fp32 block masses). */
void kvqo_certify_masked(int B, int Hq, int Hkv, int64_t cap, int64_t length, const uint16_t *q,
                         float sm, const uint8_t *m, double tau_out, const uint8_t *force,
                         const uint16_t *k16, const uint16_t *v16, const int8_t *k_codes,
                         const uint16_t *k_scales, const uint8_t *v_codes, const uint16_t *v_scales,
                         const float *k_err, const float *v_err, double *out, double *cert,
                         double *e_key, double *e_val, uint8_t *recomputed, int key_rot)
{
    certify_masked(B, Hq, Hkv, cap, length, q, sm, m, tau_out, force, k16, v16, k_codes, k_scales,
                   v_codes, v_scales, k_err, v_err, out, cert, e_key, e_val, recomputed, key_rot);
}

/* -------------------------------------------------------- adaptive precision */

/* Block log-masses of one (b, query head) over blocks [0, nblk):
 * l[i] = ln sum_{t in block i, t < length} exp(sm * q . k_t), with k_t the
 * dequantized INT8 key s_t * c_t (fp16 == 0) or the FP16 original
 * (fp16 == 1).  A log-sum-exp per block, shifted by the block's largest
 * logit. */
static void block_logmass(int b, int h, int Hkv, int64_t cap, int64_t length, const double *qv, float sm,
                          int fp16, const uint16_t *k16, const int8_t *k_codes, const uint16_t *k_scales,
                          int key_rot, double *l)
{
    int64_t nblk = (length + BLK - 1) / BLK;
    double lg[BLK];
    for (int64_t i = 0; i < nblk; ++i) {
        int64_t t0 = i * BLK, t1 = t0 + BLK < length ? t0 + BLK : length;
        double mx = -INFINITY;
        for (int64_t t = t0; t < t1; ++t) {
            size_t r = row_index(b, h, t, Hkv, cap);
            double kr[D];
            if (!fp16)
                dequant_key_row(k_codes + r * D, k_scales[r], key_rot, kr);
            double acc = 0.0;
            for (int j = 0; j < D; ++j) {
                double k = fp16 ? kvqo_f16_to_f64(k16[r * D + j]) : kr[j];
                acc += qv[j] * k;
            }
            lg[t - t0] = (double)sm * acc;
            if (lg[t - t0] > mx)
                mx = lg[t - t0];
        }
        double sum = 0.0;
        for (int64_t t = t0; t < t1; ++t)
            sum += exp(lg[t - t0] - mx);
        l[i] = mx + log(sum);
    }
}

static const double *g_sort_keys; /* qsort has no context argument */
static int by_mass_desc(const void *a, const void *b)
{
    double x = g_sort_keys[*(const int64_t *)a], y = g_sort_keys[*(const int64_t *)b];
    if (x > y)
        return -1;
    if (x < y)
        return 1;
    return (*(const int64_t *)a > *(const int64_t *)b) - (*(const int64_t *)a < *(const int64_t *)b);
}

/* Adaptive precision and the fallback ladder ("Runtime-Certified Bounded-Error
 * Quantized Attention", technical summary, Methodology 3: "Adaptive Top-K
 * Selection", "Ranking-Consistency Check" and rungs 1-3 of the "Four-Rung
 * Fallback Ladder"; Key Contributions, "Adaptive Precision").  The page gives
 * the steps and names tau_cov (its example: 99.5%); the readings below fix
 * what it leaves open.  For every (b, query head h):
 *   scoring pass  lhat_i = ln sum_{t in block i} exp(sm * q_h . khat_t) over the
 *                 dequantized INT8 keys of every block; masses
 *                 mhat_i = exp(lhat_i - LSE), LSE = ln sum_i exp(lhat_i).
 *   rung 1        K* = the smallest k whose k largest masses sum to at least
 *                 tau_cov (0 when tau_cov <= 0; every block when no k does);
 *                 the head promotes the blocks whose mass is at least the
 *                 K*-th largest (blocks tied with it are all promoted).  The
 *                 key tile of a block is promoted when any head of its KV
 *                 group promotes it.
 *   rung 2        the value tile of a block is promoted when, for some head
 *                 of its group, mhat_i * v_err_i > tau_vc.
 *   masks         the bound masks (kvqo_bounds) OR these promotions.
 *   ranking check over the head's own promoted blocks P, the FP16 log-masses
 *                 l_i (the same sum over the FP16 keys); the discordant share
 *                 disc = #{i < j in P : (lhat_i - lhat_j) * (l_i - l_j) < 0}
 *                 / (|P| (|P| - 1) / 2), 0 when |P| < 2; the ranking is
 *                 inconsistent when disc > tau_rank.
 *   rung 3        the decode over the masks with its certificate
 *                 (kvqo_certificate's terms); heads whose ranking is
 *                 inconsistent or whose certificate exceeds tau_out are
 *                 recomputed on FP16.
 * Outputs: out, cert, e_key, e_val, recomputed as kvqo_certificate;
 * masks uint8 [B][Hkv][nblk]; lhat, lfp double [B][Hq][nblk] (lfp for every
 * block); kstar int32 [B][Hq] (blocks the head promotes, ties included);
 * ndisc int64 [B][Hq] (discordant pairs);
 * npairs int64 [B][Hq]; inconsistent uint8 [B][Hq]. */
void kvqo_adaptive(int B, int Hq, int Hkv, int64_t cap, int64_t length, const uint16_t *q, float sm,
                   float tau_k, float tau_v, double tau_cov, double tau_vc, double tau_rank, double tau_out,
                   const uint16_t *k16, const uint16_t *v16, const int8_t *k_codes, const uint16_t *k_scales,
                   const uint8_t *v_codes, const uint16_t *v_scales, const float *k_err, const float *v_err,
                   double *out, double *cert, double *e_key, double *e_val, uint8_t *recomputed,
                   uint8_t *masks, double *lhat, double *lfp, int32_t *kstar, int64_t *ndisc,
                   int64_t *npairs, uint8_t *inconsistent, int key_rot)
{
    int G = Hq / Hkv;
    int64_t nblk = (length + BLK - 1) / BLK;
    size_t nb1 = (size_t)(nblk ? nblk : 1);
    uint8_t *prom = (uint8_t *)calloc((size_t)B * Hq * nb1, 1); /* each head's own promotions */
    kvqo_bounds(B, Hq, Hkv, cap, length, q, sm, tau_k, tau_v, k_err, v_err, NULL, NULL, masks);

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int hq = 0; hq < Hq; ++hq) {
            int h = hq / G;
            size_t oi = (size_t)b * Hq + hq;
            double qv[D];
            for (int j = 0; j < D; ++j)
                qv[j] = kvqo_f16_to_f64(q[oi * D + j]);
            double *lh = lhat + oi * nb1, *lf = lfp + oi * nb1;
            uint8_t *ph = prom + oi * nb1;
            block_logmass(b, h, Hkv, cap, length, qv, sm, 0, k16, k_codes, k_scales, key_rot, lh);
            block_logmass(b, h, Hkv, cap, length, qv, sm, 1, k16, k_codes, k_scales, key_rot, lf);
            kstar[oi] = 0;
            ndisc[oi] = npairs[oi] = 0;
            inconsistent[oi] = 0;
            if (nblk == 0)
                continue;
            /* masses of the scoring pass */
            double mx = -INFINITY, tot = 0.0;
            for (int64_t i = 0; i < nblk; ++i)
                if (lh[i] > mx)
                    mx = lh[i];
            for (int64_t i = 0; i < nblk; ++i)
                tot += exp(lh[i] - mx);
            double lse = mx + log(tot);
            double *mh = (double *)malloc(sizeof(double) * (size_t)nblk);
            int64_t *ord = (int64_t *)malloc(sizeof(int64_t) * (size_t)nblk);
            for (int64_t i = 0; i < nblk; ++i) {
                mh[i] = exp(lh[i] - lse);
                ord[i] = i;
            }
            /* rung 1: the smallest top set covering tau_cov, ties included */
            int64_t k = 0;
            if (tau_cov > 0.0) {
#pragma omp critical(kvqo_sort)
                {
                    g_sort_keys = mh;
                    qsort(ord, (size_t)nblk, sizeof(int64_t), by_mass_desc);
                }
                double cum = 0.0;
                k = nblk;
                for (int64_t r = 0; r < nblk; ++r) {
                    cum += mh[ord[r]];
                    if (cum >= tau_cov) {
                        k = r + 1;
                        break;
                    }
                }
            }
            if (k > 0) {
                double theta = mh[ord[k - 1]];
                for (int64_t i = 0; i < nblk; ++i) {
                    ph[i] = mh[i] >= theta;
                    kstar[oi] += ph[i];
                }
            }
            /* ranking check over the head's promoted blocks */
            int64_t nd = 0, np = 0;
            for (int64_t i = 0; i < nblk; ++i) {
                if (!ph[i])
                    continue;
                for (int64_t j = i + 1; j < nblk; ++j) {
                    if (!ph[j])
                        continue;
                    ++np;
                    if ((lh[i] - lh[j]) * (lf[i] - lf[j]) < 0.0)
                        ++nd;
                }
            }
            ndisc[oi] = nd;
            npairs[oi] = np;
            inconsistent[oi] = np > 0 && (double)nd > tau_rank * (double)np;
            /* rung 2 marks go to the group's masks below; keep mh in prom's
             * place via the value flag bit 1 */
            for (int64_t i = 0; i < nblk; ++i) {
                size_t si = blk_index(b, h, i, Hkv, cap);
                if (mh[i] * (double)v_err[si] > tau_vc)
                    ph[i] |= 2;
            }
            free(mh);
            free(ord);
        }
    /* the group's union of its heads' promotions into the masks */
    for (int b = 0; b < B; ++b)
        for (int hq = 0; hq < Hq; ++hq) {
            int h = hq / G;
            const uint8_t *ph = prom + ((size_t)b * Hq + hq) * nb1;
            uint8_t *mk = masks + ((size_t)b * Hkv + h) * (size_t)nblk;
            for (int64_t i = 0; i < nblk; ++i)
                mk[i] |= ph[i];
        }
    free(prom);
    certify_masked(B, Hq, Hkv, cap, length, q, sm, masks, tau_out, inconsistent, k16, v16, k_codes, k_scales,
                   v_codes, v_scales, k_err, v_err, out, cert, e_key, e_val, recomputed, key_rot);
}
