/*
 * kvq.h -- C ABI of libkvq: certified quantized-KV decode attention on AMD
 * MI355X (gfx950).
 *
 * Method: "Runtime-Certified Bounded-Error Quantized Attention" (Dean Calver;
 * gist.science explainer of arXiv 2605.20868), technical summary:
 *   Methodology 1 "Tiered Storage with Deterministic Fallback" -- a compressed
 *     tier of INT8 keys and INT4 values with scales and per-block error
 *     annotations, and a tier of FP16 originals used for fallback;
 *   Methodology 2 "Two-Term Error Decomposition" -- a key term bounded through
 *     the per-token score perturbation and a value term from per-block
 *     reconstruction errors, both computed online from scales and query norms,
 *     giving per-head, per-step precision decisions;
 *   Key Contributions "Deterministic Recovery" -- blocks whose bound is not
 *     certified are served from the FP16 originals.
 *
 * Codec and bounds implemented here (this library's reading of the page,
 * which names INT8 keys, INT4 values, scales and per-block annotations but
 * prints no formulas):
 *   key codes   int8 per (token, KV head); fp16 scale s = f16(f32(max|x|)/127);
 *               c = clamp(round_half_even(x/s), -127, 127); s = 0 -> c = 0.
 *   value codes int4 per (token, KV head, 32-channel group); fp16 scale
 *               s = f16(f32(max|x|)/7); c = clamp(round_half_even(x/s), -7, 7).
 *   a key row or value group holding Inf/NaN gets codes 0, scale 0 and an
 *   error of +Inf, so its block always falls back.
 *   per-token key error  ||k - k^||_2 = f32(sqrt(T128(e_j^2))) in fp64, with
 *   T128 the fixed pairwise tree (within 8 contiguous channels: strides 1, 2,
 *   4; then across the 16 partial sums: channel strides 64, 32, 16, 8);
 *   per-token value error max_j |v_j - v^_j| (exact).
 *   block statistics k_err, v_err = max over the block's valid tokens.
 *   query norm of head h: f32(sqrt(T128(q_j^2))); per (batch, KV head) the max
 *   over its G = q_heads/kv_heads query heads (heads kvh*G .. kvh*G+G-1).
 *   key bound   KB = ((sm*qn)*k_err)*(1+2^-16), fp32 products left to right:
 *               an upper bound (Cauchy-Schwarz) on |sm * q.(k - k^)| for every
 *               head of the group and token of the block, in logit units.
 *   value bound VB = v_err.
 *   fallback    mask bit 0 (key) = !(KB finite && KB <= tau_k);
 *               mask bit 1 (value) = !(VB finite && VB <= tau_v).
 *   attention   softmax(sm * q.k~) v~ over tokens t < length with, per block,
 *               k~ = bit0 ? fp16 original : s*c and v~ = bit1 ? fp16 original
 *               : s*c.  Output fp16.  length 0 gives a zero output.
 *
 * Memory layout (device memory, caller-allocated, head-major so that each
 * 64-token block of one (batch, KV head) is contiguous; tier 2 may instead be
 * pinned host memory, see kvq_tier2_location).  cap = capacity in tokens, a
 * multiple of 64; NBc = cap/64.
 *   k16, v16   uint16 (fp16 bits) [B][Hkv][cap][128]  FP16 originals (tier 2)
 *   k_codes    int8               [B][Hkv][cap][128]
 *   k_scales   uint16 (fp16)      [B][Hkv][cap]
 *   v_codes    uint8              [B][Hkv][NBc][128][32]  per block, channel-
 *              major: byte (j, i) holds token 2i of channel j in its low
 *              nibble and token 2i+1 in its high nibble (two's complement).
 *              Nibbles of tokens >= length inside a written block are 0.
 *   v_scales   uint16 (fp16)      [B][Hkv][cap][4]
 *   k_err, v_err float            [B][Hkv][NBc]
 *   q          uint16 (fp16)      [B][Hq][128]
 *   out        uint16 (fp16)      [B][Hq][128]
 *   kb, vb     float, mask uint8  [B][Hkv][NB], NB = ceil(length/64)
 *
 * Streams: every entry point that touches the GPU takes a hipStream_t passed
 * as void* (NULL = the null stream) and only enqueues work on it; nothing
 * blocks the host.  Calls on one cache must be ordered by the caller (same
 * stream or explicit events).  Argument errors are reported synchronously and
 * enqueue nothing.  A failed launch returns KVQ_ERR_HIP; kvq_last_hip_error()
 * then holds the hipError_t code (thread-local).  Faults during execution
 * surface at the caller's next synchronisation.
 *
 * Preconditions checked by every entry point: head_dim == 128,
 * block_tokens == 64, v_group == 32, batch >= 1, kv_heads >= 1,
 * capacity % 64 == 0, 0 <= length <= capacity, q_heads % kv_heads == 0 with
 * 1 <= q_heads/kv_heads <= 16, tolerances not NaN and >= 0, every device
 * pointer 16-byte aligned (fp16/int8 arrays) or 4-byte aligned (float).
 * The library never allocates memory and keeps no state besides the
 * thread-local error code.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = -1, /* null pointer, bad shape, NaN/negative tolerance */
    KVQ_ERR_UNSUPPORTED = -2, /* head_dim/block/group other than 128/64/32, G > 16 */
    KVQ_ERR_CAPACITY = -3,    /* length + n_new > capacity */
    KVQ_ERR_ALIGNMENT = -4,   /* a device pointer is misaligned */
    KVQ_ERR_WORKSPACE = -5,   /* workspace null or smaller than kvq_decode_workspace_bytes */
    KVQ_ERR_HIP = -6          /* a HIP call failed; see kvq_last_hip_error() */
} kvq_status;

/* Key codecs.  KVQ_CODEC_ROTATE_K (outlier-aware codec: the Walsh-Hadamard
 * transform before scalar quantization of the KQV scheme in "Statistical
 * Inference and Quality Measures of KV Cache Quantisations Inspired by
 * TurboQuant", technical summary, quantisation schemes, applied to the keys
 * alone) quantizes each key row after the rotation u = H k / 16, H the +-1
 * Sylvester-Hadamard matrix of order 128 (exact in fp64): s = f16(f32(max|u|)
 * / 127), c = clamp(round_half_even(u / s), -127, 127) with the quotient in
 * fp64, and reads keys back as k~ = H (s c) / 8; the key error is
 * ||k - k~|| = f32(sqrt(2 * T128((u - s c)^2))), so the key bound and the
 * certificate keep their meaning.  The decode rotates q instead of the keys
 * (q . k~ = (H q / 8) . (s c)); outlier channels spread over the row, which
 * lowers the key errors and the fallback share.  Values keep their codec.
 * A cache's codec is fixed when its first token is quantized. */
#define KVQ_CODEC_PLAIN 0
#define KVQ_CODEC_ROTATE_K 1

/* A quantized KV cache for one attention layer.  The struct is host memory;
 * every pointer in it is owned by the caller: device memory, except that
 * k16/v16 may be pinned host memory the device reads (kvq_tier2_location). */
typedef struct kvq_cache {
    int32_t batch;        /* B */
    int32_t kv_heads;     /* Hkv */
    int32_t head_dim;     /* must be 128 */
    int32_t block_tokens; /* must be 64 */
    int32_t v_group;      /* must be 32 */
    int32_t codec;        /* KVQ_CODEC_PLAIN or KVQ_CODEC_ROTATE_K */
    int64_t capacity;     /* tokens per sequence, multiple of 64 */
    int64_t length;       /* valid tokens per sequence (host-side) */
    const uint16_t *k16;  /* FP16 originals, written by the caller */
    const uint16_t *v16;
    int8_t *k_codes;
    uint16_t *k_scales;
    uint8_t *v_codes;
    uint16_t *v_scales;
    float *k_err;
    float *v_err;
} kvq_cache;

/* Byte sizes of the six tier-1 buffers, in the order k_codes, k_scales,
 * v_codes, v_scales, k_err, v_err, for the shape fields of *c (pointers and
 * length are ignored).  Host only. */
kvq_status kvq_cache_bytes(const kvq_cache *c, size_t bytes_out[6]);

/* Where tier 2 lives (Methodology 1 keeps the FP16 originals in pinned
 * system RAM, as the ground truth that fallback pages in).  *where_out = 0
 * when k16 and v16 are both device memory of the current device; 1 when both
 * are pinned host memory that the current device reads at the same address.
 * With 1, every kernel reads tier 2 in place over the host link (zero-copy:
 * the fused append's new rows, the bulk append's rows and every fallback
 * tile), with no staging copy.  Call it once when the cache is set up, before
 * any other entry point touches a host tier 2.  Host only, enqueues nothing.
 * Errors: INVALID_ARG for null pointers, a mix of the two kinds, pageable or
 * unknown host memory, another device's memory, or host memory the device
 * sees at another address; HIP when the attribute query itself fails. */
kvq_status kvq_tier2_location(const kvq_cache *c, int32_t *where_out);

/* Empties the cache for reuse by another sequence (Methodology 1's per-block
 * error annotations start over): enqueues on the stream a fill of k_err and
 * v_err with zeros over the whole capacity (a kernel, not a memset, so the
 * call can be captured into a graph) and sets c->length = 0.  The other
 * tier-1 buffers keep their bytes, which no entry point reads at positions
 * >= length: the first append into a block overwrites its statistics and
 * writes every nibble byte of the block, so appends after a reset give the
 * same tier-1 bytes as appends into a fresh cache.  Allocates nothing, does
 * not block.  Errors: INVALID_ARG (shape, null statistics), ALIGNMENT, HIP. */
kvq_status kvq_cache_reset(kvq_cache *c, void *stream);

/* Quantize-on-append (Methodology 1: tier-1 codes, scales and per-block error
 * annotations derived from the FP16 originals).  Quantizes tokens
 * [length, length + n_new) of every (batch, KV head) from k16/v16 into the
 * tier-1 buffers, updates the statistics of every block those tokens touch
 * (max with the block's earlier tokens), and on success advances c->length by
 * n_new.  Blocks are written whole by one workgroup, so appends of any size
 * and alignment give bit-identical buffers to one bulk append of the same
 * tokens.  n_new == 0 is a no-op.  Errors: INVALID_ARG, UNSUPPORTED,
 * CAPACITY, ALIGNMENT, HIP. */
kvq_status kvq_quantize_append(kvq_cache *c, int64_t n_new, void *stream);

/* Per-block bounds and fallback masks (Methodology 2: key and value terms
 * from the block statistics and the query norms, no FP16 access).  For
 * q [B][q_heads][128] writes, for every (batch, KV head, block < NB), the key
 * bound KB, the value bound VB and the 2-bit fallback mask.  Each of kb, vb,
 * mask may be NULL.  Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT, HIP. */
kvq_status kvq_bounds(const kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                      float tau_k, float tau_v, float *kb, float *vb, uint8_t *mask, void *stream);

/* Workspace size in bytes needed by kvq_decode_attn for this cache shape and
 * query-head count (independent of length).  0 on invalid arguments. */
size_t kvq_decode_workspace_bytes(const kvq_cache *c, int32_t q_heads);

/* Certified decode attention (Methodology 1-3 on the decode step): one query
 * token per sequence, q [B][q_heads][128] fp16 -> out [B][q_heads][128] fp16.
 * Bounds and masks are evaluated inside the kernel from the block statistics
 * (same arithmetic as kvq_bounds); fallback blocks read k16/v16, the others
 * read the int8/int4 codes.  mask_out [B][Hkv][NB] receives the masks used
 * (may be NULL).  workspace: device memory of at least
 * kvq_decode_workspace_bytes() bytes, 256-byte aligned.  Its first
 * 4 * batch * kv_heads bytes are arrival counters, one per (batch, KV head):
 * zero them before the first use (and again before using the workspace for
 * a cache with a larger batch * kv_heads); every call leaves them at zero,
 * so the workspace is allocated and cleared once and reused.  The rest holds
 * the per-split partial results, with no required contents: the last of the
 * matrix-core kernel's workgroups of each (batch, KV head) to finish merges
 * that group's splits in the same launch (one kernel per call); the VALU
 * kernel is followed by a merge kernel.  Concurrent calls need distinct
 * workspaces.  Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT, WORKSPACE,
 * HIP. */
kvq_status kvq_decode_attn(const kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                           float tau_k, float tau_v, uint16_t *out, uint8_t *mask_out,
                           void *workspace, size_t ws_bytes, void *stream);

/* One decode step in one launch: quantize-on-append of token `length` of
 * every sequence (its FP16 rows must already be in k16/v16), then certified
 * decode attention over length+1 tokens; on success c->length grows by one.
 * Equivalent to kvq_quantize_append(c, 1, stream) followed by
 * kvq_decode_attn(): the same tier-1 bytes, block statistics and masks, and
 * the same output up to the order of floating-point accumulation.  The
 * matrix-core kernel performs the append itself (every workgroup of a
 * (batch, KV head) quantizes the new token for its masks, one of them writes
 * it), saving the append launch; with the VALU kernel the append is a
 * separate launch.  Errors: as kvq_decode_attn, plus CAPACITY when
 * length == capacity. */
kvq_status kvq_append_decode(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                             float tau_k, float tau_v, uint16_t *out, uint8_t *mask_out,
                             void *workspace, size_t ws_bytes, void *stream);

/* Allocation-free decode step, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): kvq_append_decode, with the per-split partial results
 * in a static device array of KVQ_SCRATCH_BYTES inside the library instead
 * of a caller workspace.  Each device the library runs on holds its own
 * copy of the array until the process ends; it starts zeroed, keeps the
 * last call's partials and is left fit for the next call (its arrival
 * counters back at zero).  Every call on a device shares that device's
 * copy, so calls that overlap on one device (other streams, other host
 * threads) race and must be serialized by the caller.  The call allocates
 * nothing.  Errors: as kvq_append_decode; KVQ_ERR_WORKSPACE when
 * batch * kv_heads exceeds KVQ_SCRATCH_MAX_GROUPS (the arrival counters at
 * the head of the array) or the partials of the split count used, about 524
 * bytes per (batch, query head, split), do not fit in the rest of
 * KVQ_SCRATCH_BYTES. */
#define KVQ_SCRATCH_BYTES (8u << 20)
#define KVQ_SCRATCH_MAX_GROUPS 16384u
kvq_status kvq_append_decode_noalloc(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                                     float tau_k, float tau_v, uint16_t *out, uint8_t *mask_out, void *stream);

/* Certified decode with a per-head output certificate and per-head FP16
 * recompute ("Runtime-Certified Bounded-Error Quantized Attention",
 * Methodology 2, two-term error decomposition; Methodology 3, rung 3 of the
 * fallback ladder, per-head fallback).  As kvq_decode_attn (or, with
 * append != 0, as kvq_append_decode: token `length` is quantized first and
 * c->length grows by one), and in addition, for every query head h:
 *   cert [B][q_heads] (float, required) receives E_key + E_val, a bound on
 *     max_j |o_dense[h][j] - o[h][j]| between the decode output and dense
 *     FP16 attention, in exact arithmetic: E_key = tanh(Delta/2)*R with
 *     Delta = sm*||q_h||*(largest key error of a key-certified block) and
 *     R = 2*max(7*S + eta, A) (S: largest value scale of a value-certified
 *     token, eta: largest value error of a value-certified block, A: largest
 *     |v| of a value-fallback token); E_val = sum over value-certified blocks
 *     of (attention mass of the block) * (its value error).  Rounded up to
 *     fp32; the kernel's own floating-point rounding is not included.
 *   heads with cert > tau_out are recomputed over the FP16 keys and values
 *     (their out rows become the dense result) and get recomputed[h] = 1
 *     (recomputed [B][q_heads] uint8, may be NULL).  tau_out = +INFINITY
 *     skips the recompute launches.
 * Runs on the matrix-core kernel only (KVQ_ERR_UNSUPPORTED where
 * kvq_decode_attn would pick the VALU kernel).  The recompute costs two more
 * launches (a decode and a merge restricted on the device to the groups and
 * heads flagged), whatever the flags.  Errors: as kvq_decode_attn; also
 * INVALID_ARG for cert == NULL or a NaN tau_out, CAPACITY for append at
 * length == capacity. */
kvq_status kvq_decode_attn_cert(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                                float tau_k, float tau_v, float tau_out, int32_t append, uint16_t *out,
                                float *cert, uint8_t *recomputed, uint8_t *mask_out, void *workspace,
                                size_t ws_bytes, void *stream);

/* Workspace of kvq_decode_attn_adaptive: the decode workspace plus the
 * scoring pass's block log-masses, the promotions and the FP16 step
 * statistics (about 4*q_heads*(1 + 16*capacity/64) bytes per sequence more).
 * 0 on an invalid shape. */
size_t kvq_adaptive_workspace_bytes(const kvq_cache *c, int32_t q_heads);

/* Adaptive precision with the fallback ladder ("Runtime-Certified Bounded-
 * Error Quantized Attention", technical summary, Methodology 3: "Adaptive
 * Top-K Selection", "Ranking-Consistency Check" and rungs 1-3 of the
 * fallback ladder; Key Contributions "Adaptive Precision").  As
 * kvq_decode_attn_cert (cert required; recomputed may be NULL; append as
 * there), with these steps before the decode, for every query head h:
 *   scoring  a pass over the INT8 keys of every block gives the block's
 *            log-mass lhat_i = log sum_{t in block i} exp(sm * q_h . k^_t),
 *            and its mass m_i (the share of sum_i exp(lhat_i)).
 *   rung 1   the head promotes the blocks whose mass is at least the K*-th
 *            largest, K* the smallest count whose largest masses sum to
 *            tau_cov (none for tau_cov == 0; every block when no count gets
 *            there, e.g. tau_cov > 1); a block's key tile is read as FP16 when
 *            any head of its KV group promotes it.  kstar [B][q_heads] (int32,
 *            may be NULL) receives the count each head promotes.
 *   rung 2   a block's value tile is read as FP16 when m_i * v_err_i >
 *            tau_vc for some head of the group (+INFINITY: never).
 *   masks    the bound masks OR these promotions (mask_out receives them).
 *   check    over the head's own promoted blocks, the pairs whose INT8 and
 *            FP16 block log-masses are ordered oppositely (the FP16 ones
 *            from the decode's FP16 key tiles) are counted into ndisc
 *            [B][q_heads] (int32, may be NULL); a head with more than
 *            tau_rank * (pairs) of them is inconsistent (tau_rank >= 1: never).
 *   rung 3   heads that are inconsistent or whose certificate (over the masks
 *            above) exceeds tau_out are recomputed over the FP16 keys and
 *            values (recomputed[h] = 1).
 * The masses and the ranking are evaluated in fp32, so near-ties may fall
 * either way.  Matrix-core path only; at most 8192 blocks (524,288 tokens)
 * per sequence.  Errors: as kvq_decode_attn_cert; also INVALID_ARG for NaN
 * or negative tau_cov, tau_vc or tau_rank, WORKSPACE below
 * kvq_adaptive_workspace_bytes, UNSUPPORTED past 8192 blocks. */
kvq_status kvq_decode_attn_adaptive(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                                    float tau_k, float tau_v, float tau_cov, float tau_vc, float tau_rank,
                                    float tau_out, int32_t append, uint16_t *out, float *cert,
                                    uint8_t *recomputed, int32_t *kstar, int32_t *ndisc, uint8_t *mask_out,
                                    void *workspace, size_t ws_bytes, void *stream);

/* Decode kernel selection and timing, for measurement.  kvq_decode_attn and
 * kvq_append_decode use KVQ_KERNEL_AUTO: the matrix-core kernel for every
 * group size up to 16 and up to 1,048,576 tokens per sequence, else the VALU
 * kernel.  The matrix-core kernel has two variants with the same results:
 * up to 2048 blocks (131,072 tokens) per sequence, without the certificate
 * and adaptive passes, a streaming variant that starts copying tiles before
 * the masks are known (KVQ_KERNEL_MFMA picks it where it applies), and a
 * general one that forms every mask first (KVQ_KERNEL_MFMA_TABLE forces it).
 * The _ex forms let a benchmark force a kernel and a split count (0 =
 * automatic), and, when split_done is a hipEvent_t (passed as void*, NULL =
 * none), record it on the stream right after the split-K kernel (before the
 * merge kernel, where there is one), so that the split-K kernel can be
 * timed alone.  Same semantics and
 * errors as kvq_decode_attn; a kernel that does not support the group size
 * or the context length returns KVQ_ERR_UNSUPPORTED.  The environment
 * variable KVQ_SPLITS, when set, replaces the automatic split count. */
typedef enum {
    KVQ_KERNEL_AUTO = 0,
    KVQ_KERNEL_VALU = 1,
    KVQ_KERNEL_MFMA = 2,
    KVQ_KERNEL_MFMA_TABLE = 3
} kvq_kernel;
kvq_status kvq_decode_attn_ex(const kvq_cache *c, const uint16_t *q, int32_t q_heads,
                              float sm_scale, float tau_k, float tau_v, uint16_t *out,
                              uint8_t *mask_out, void *workspace, size_t ws_bytes, void *stream,
                              int32_t kernel, int32_t splits, void *split_done);
kvq_status kvq_append_decode_ex(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                                float tau_k, float tau_v, uint16_t *out, uint8_t *mask_out,
                                void *workspace, size_t ws_bytes, void *stream, int32_t kernel,
                                int32_t splits, void *split_done);

/* Human-readable name of a status code (static string). */
const char *kvq_status_str(kvq_status s);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int kvq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
