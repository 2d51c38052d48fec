// kvq_api.hip -- the C ABI of libkvq (see include/kvq.h): argument checks,
// workspace sizing, split selection and kernel dispatch.  Host code only; no
// allocation, no synchronisation.
#include <math.h>
#include <stdlib.h>

#include <mutex>

#include "kvq.h"
#include "kvq_internal.hpp"

namespace {

thread_local int g_last_hip_error = 0;

kvq_status hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return KVQ_ERR_HIP;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

kvq_status check_shape(const kvq_cache *c) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    if (c->head_dim != kvq::D || c->block_tokens != kvq::BLK || c->v_group != kvq::VG)
        return KVQ_ERR_UNSUPPORTED;
    if (c->batch < 1 || c->kv_heads < 1 || c->capacity < 0 || c->capacity % kvq::BLK != 0)
        return KVQ_ERR_INVALID_ARG;
    if (c->length < 0 || c->length > c->capacity) return KVQ_ERR_INVALID_ARG;
    if (c->batch > 65535 || c->kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
    if (c->codec != KVQ_CODEC_PLAIN && c->codec != KVQ_CODEC_ROTATE_K) return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
}

kvq_status check_buffers(const kvq_cache *c, bool need_fp16) {
    if (!c->k_codes || !c->k_scales || !c->v_codes || !c->v_scales || !c->k_err || !c->v_err)
        return KVQ_ERR_INVALID_ARG;
    if (need_fp16 && (!c->k16 || !c->v16)) return KVQ_ERR_INVALID_ARG;
    if (!aligned(c->k_codes, 16) || !aligned(c->k_scales, 16) || !aligned(c->v_codes, 16) ||
        !aligned(c->v_scales, 16) || !aligned(c->k_err, 4) || !aligned(c->v_err, 4) ||
        !aligned(c->k16, 16) || !aligned(c->v16, 16))
        return KVQ_ERR_ALIGNMENT;
    return KVQ_OK;
}

kvq_status check_query(const kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm,
                       float tau_k, float tau_v) {
    if (!q || q_heads < 1 || q_heads % c->kv_heads != 0) return KVQ_ERR_INVALID_ARG;
    if (q_heads / c->kv_heads > 16) return KVQ_ERR_UNSUPPORTED;
    if (!isfinite(sm) || isnan(tau_k) || isnan(tau_v) || tau_k < 0.0f || tau_v < 0.0f)
        return KVQ_ERR_INVALID_ARG;
    if (!aligned(q, 16)) return KVQ_ERR_ALIGNMENT;
    return KVQ_OK;
}

kvq::CachePtrs ptrs(const kvq_cache *c) {
    return kvq::CachePtrs{c->k16, c->v16, c->k_codes, c->k_scales, c->v_codes, c->v_scales, c->k_err,
                          c->v_err};
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout: [arrival counters uint32 x slots: zero before the first
//                    call, left zero by every call]
//                   [part_ml float2 x B*Hkv*S*G] [part_acc float x B*Hkv*S*G*128]
//                   certificate: [part_e float x B*Hkv*S*G] [part_sa float2 x
//                   B*Hkv*S] [part_kv float2 x B*Hkv] [flags uint8 x B*Hq],
//                   each padded to 256 B.  The counters come first, so that
//                   no other region of a later call with another split count
//                   (the static scratch) or a smaller B*Hkv lands on them.
struct WsLayout {
    size_t arrive, ml, acc, e, sa, kv, flags, total;
};

WsLayout ws_layout(const kvq_cache *c, int32_t g, int64_t splits, size_t slots) {
    const size_t bh = (size_t)c->batch * (size_t)c->kv_heads;
    const size_t parts = bh * (size_t)splits * (size_t)g;
    WsLayout w;
    w.arrive = 0;
    w.ml = round_up(slots * sizeof(uint32_t), 256);
    w.acc = round_up(w.ml + parts * sizeof(float2), 256);
    w.e = round_up(w.acc + parts * kvq::D * sizeof(float), 256);
    w.sa = round_up(w.e + parts * sizeof(float), 256);
    w.kv = round_up(w.sa + bh * (size_t)splits * sizeof(float2), 256);
    w.flags = round_up(w.kv + bh * sizeof(float2), 256);
    w.total = w.flags + bh * (size_t)g;
    return w;
}

// Adaptive workspace: the decode workspace, then [lhat float x B*Hq*NBc]
// [phead uint8 x B*Hq*NBc] [promote uint8 x B*Hkv*NBc] [step statistics
// float2 x B*Hkv*G*NBc*8, each head's blocks and slots contiguous] [rotated
// query, fp16 hi and lo parts x B*Hq*2*128], each padded to 256 B.
struct AdaptLayout {
    size_t lhat, phead, promote, step, qrot, total;
};

AdaptLayout adapt_layout(const kvq_cache *c, int32_t q_heads, size_t base) {
    const size_t nbc = (size_t)(c->capacity / kvq::BLK);
    const size_t bq = (size_t)c->batch * (size_t)q_heads, bh = (size_t)c->batch * (size_t)c->kv_heads;
    AdaptLayout w;
    w.lhat = round_up(base, 256);
    w.phead = round_up(w.lhat + bq * nbc * sizeof(float), 256);
    w.promote = round_up(w.phead + bq * nbc, 256);
    w.step = round_up(w.promote + bh * nbc, 256);
    w.qrot = round_up(w.step + bq * nbc * 8 * sizeof(float2), 256);
    w.total = w.qrot + bq * 2 * kvq::D * sizeof(uint16_t);
    return w;
}

int64_t max_splits(const kvq_cache *c) {
    const int64_t nbc = c->capacity / kvq::BLK;
    int64_t s = nbc < kvq::MAX_SPLITS ? nbc : kvq::MAX_SPLITS;
    return s < 1 ? 1 : s;
}

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Splits: about `per_cu` workgroups per CU over the launch (the matrix-core
// kernel holds one per CU, so a second round fills CUs that finish early;
// the VALU kernel keeps four resident), never more splits than blocks, never
// more blocks per split than the kernel's LDS table holds (max_bps).
int64_t choose_splits(const kvq_cache *c, int64_t nb, int32_t requested, int per_cu, int64_t max_bps) {
    const int64_t bh = (int64_t)c->batch * c->kv_heads;
    const int64_t smax = max_splits(c);
    int64_t s;
    if (requested > 0) {
        s = requested;
    } else if (const char *env = getenv("KVQ_SPLITS")) {
        s = atoll(env);
    } else {
        const int64_t target_wgs = (int64_t)per_cu * device_cus();
        s = (target_wgs + bh - 1) / bh;
    }
    if (s > nb) s = nb;
    const int64_t need = (nb + max_bps - 1) / max_bps;
    if (s < need) s = need;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    return s;
}

}  // namespace

extern "C" {

const char *kvq_status_str(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_INVALID_ARG: return "invalid argument";
        case KVQ_ERR_UNSUPPORTED: return "unsupported shape";
        case KVQ_ERR_CAPACITY: return "capacity exceeded";
        case KVQ_ERR_ALIGNMENT: return "misaligned pointer";
        case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
        case KVQ_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

int kvq_last_hip_error(void) { return g_last_hip_error; }

// Kind of the memory at p for the current device: 0 device memory, 1 pinned
// host memory mapped at the same address, -1 anything else; -2 (with *err
// set) when the query fails for another reason.
static int tier2_kind(const void *p, hipError_t *err) {
    hipPointerAttribute_t at;
    const hipError_t e = hipPointerGetAttributes(&at, p);
    if (e == hipErrorInvalidValue) {  // memory HIP does not know (pageable)
        (void)hipGetLastError();
        return -1;
    }
    if (e != hipSuccess) {
        *err = e;
        return -2;
    }
    int dev = 0;
    const hipError_t ed = hipGetDevice(&dev);
    if (ed != hipSuccess) {
        *err = ed;
        return -2;
    }
    if (at.type == hipMemoryTypeDevice && at.device == dev) return 0;
    if (at.type == hipMemoryTypeHost && at.devicePointer == p) return 1;
    return -1;
}

kvq_status kvq_tier2_location(const kvq_cache *c, int32_t *where_out) {
    if (!c || !where_out || !c->k16 || !c->v16) return KVQ_ERR_INVALID_ARG;
    hipError_t err = hipSuccess;
    const int kk = tier2_kind(c->k16, &err);
    const int kv = kk == -2 ? -2 : tier2_kind(c->v16, &err);
    if (kk == -2 || kv == -2) return hip_fail(err);
    if (kk < 0 || kv < 0 || kk != kv) return KVQ_ERR_INVALID_ARG;
    *where_out = kk;
    return KVQ_OK;
}

kvq_status kvq_cache_bytes(const kvq_cache *c, size_t bytes_out[6]) {
    kvq_status st = check_shape(c);
    if (st != KVQ_OK) return st;
    if (!bytes_out) return KVQ_ERR_INVALID_ARG;
    const size_t rows = (size_t)c->batch * c->kv_heads * (size_t)c->capacity;
    const size_t blocks = rows / kvq::BLK;
    bytes_out[0] = rows * kvq::D;                // k_codes
    bytes_out[1] = rows * sizeof(uint16_t);      // k_scales
    bytes_out[2] = rows * kvq::D / 2;            // v_codes
    bytes_out[3] = rows * 4 * sizeof(uint16_t);  // v_scales
    bytes_out[4] = blocks * sizeof(float);       // k_err
    bytes_out[5] = blocks * sizeof(float);       // v_err
    return KVQ_OK;
}

kvq_status kvq_quantize_append(kvq_cache *c, int64_t n_new, void *stream) {
    kvq_status st = check_shape(c);
    if (st != KVQ_OK) return st;
    if (n_new < 0) return KVQ_ERR_INVALID_ARG;
    if (n_new > c->capacity - c->length) return KVQ_ERR_CAPACITY;
    if ((st = check_buffers(c, true)) != KVQ_OK) return st;
    if (n_new == 0) return KVQ_OK;
    kvq::AppendArgs a;
    a.c = ptrs(c);
    a.cap = c->capacity;
    a.len0 = c->length;
    a.len1 = c->length + n_new;
    a.blk_lo = a.len0 / kvq::BLK;
    a.hkv = c->kv_heads;
    a.key_rot = c->codec == KVQ_CODEC_ROTATE_K ? 1 : 0;
    const int64_t nblk = (a.len1 - 1) / kvq::BLK - a.blk_lo + 1;
    if (nblk > 0x7FFFFFFF) return KVQ_ERR_UNSUPPORTED;
    hipError_t e = kvq::launch_append(a, c->batch, nblk, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    c->length = a.len1;
    return KVQ_OK;
}

kvq_status kvq_cache_reset(kvq_cache *c, void *stream) {
    kvq_status st = check_shape(c);
    if (st != KVQ_OK) return st;
    if (!c->k_err || !c->v_err) return KVQ_ERR_INVALID_ARG;
    if (!aligned(c->k_err, 4) || !aligned(c->v_err, 4)) return KVQ_ERR_ALIGNMENT;
    const int64_t n = (int64_t)c->batch * c->kv_heads * (c->capacity / kvq::BLK);
    hipError_t e = kvq::launch_zero_stats(c->k_err, c->v_err, n, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    c->length = 0;
    return KVQ_OK;
}

kvq_status kvq_bounds(const kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                      float tau_k, float tau_v, float *kb, float *vb, uint8_t *mask, void *stream) {
    kvq_status st = check_shape(c);
    if (st != KVQ_OK) return st;
    if ((st = check_query(c, q, q_heads, sm_scale, tau_k, tau_v)) != KVQ_OK) return st;
    if (!c->k_err || !c->v_err) return KVQ_ERR_INVALID_ARG;
    if (!aligned(c->k_err, 4) || !aligned(c->v_err, 4) || !aligned(kb, 4) || !aligned(vb, 4))
        return KVQ_ERR_ALIGNMENT;
    const int64_t nb = (c->length + kvq::BLK - 1) / kvq::BLK;
    if (nb == 0) return KVQ_OK;
    kvq::BoundsArgs a;
    a.k_err = c->k_err;
    a.v_err = c->v_err;
    a.q = q;
    a.kb = kb;
    a.vb = vb;
    a.mask = mask;
    a.nbc = c->capacity / kvq::BLK;
    a.nb = nb;
    a.hkv = c->kv_heads;
    a.hq = q_heads;
    a.g = q_heads / c->kv_heads;
    a.sm = sm_scale;
    a.tau_k = tau_k;
    a.tau_v = tau_v;
    hipError_t e = kvq::launch_bounds(a, c->batch, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return KVQ_OK;
}

size_t kvq_decode_workspace_bytes(const kvq_cache *c, int32_t q_heads) {
    if (check_shape(c) != KVQ_OK || q_heads < 1 || q_heads % c->kv_heads != 0 ||
        q_heads / c->kv_heads > 16)
        return 0;
    return ws_layout(c, q_heads / c->kv_heads, max_splits(c), (size_t)c->batch * (size_t)c->kv_heads).total;
}

size_t kvq_adaptive_workspace_bytes(const kvq_cache *c, int32_t q_heads) {
    const size_t base = kvq_decode_workspace_bytes(c, q_heads);
    return base ? adapt_layout(c, q_heads, base).total : 0;
}

}  // extern "C"

namespace {

// Options of the adaptive-precision decode (kvq_decode_attn_adaptive).
struct AdaptOpts {
    float tau_cov, tau_vc, tau_rank;
    int32_t *kstar, *ndisc;
};

bool bad_tol(float t) { return t != t || t < 0.0f; }

// Decode over the cache's tokens; with append, token `length` (already in
// k16/v16) is first quantized into tier 1 and joins the decode: fused into
// the matrix-core kernel (or, in the adaptive decode, into the scoring pass
// that runs first), or as an append launch before the VALU kernel.  On
// success with append, c->length grows by one.
kvq_status decode_impl(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale, float tau_k,
                       float tau_v, uint16_t *out, uint8_t *mask_out, void *workspace, size_t ws_bytes,
                       void *stream, int32_t kernel, int32_t splits, void *split_done, bool append,
                       float *cert = nullptr, float tau_out = 0.0f, uint8_t *recomputed = nullptr,
                       const AdaptOpts *ad = nullptr, bool scratch_ws = false) {
    kvq_status st = check_shape(c);
    if (st != KVQ_OK) return st;
    if ((st = check_query(c, q, q_heads, sm_scale, tau_k, tau_v)) != KVQ_OK) return st;
    if ((st = check_buffers(c, true)) != KVQ_OK) return st;
    if (!out) return KVQ_ERR_INVALID_ARG;
    if (!aligned(out, 16)) return KVQ_ERR_ALIGNMENT;
    if (kernel < KVQ_KERNEL_AUTO || kernel > KVQ_KERNEL_MFMA_TABLE || splits < 0) return KVQ_ERR_INVALID_ARG;
    const bool no_stream = kernel == KVQ_KERNEL_MFMA_TABLE;
    if (no_stream) kernel = KVQ_KERNEL_MFMA;
    const bool certify = cert != nullptr;
    if (certify && (tau_out != tau_out || !aligned(cert, 4))) return tau_out != tau_out ? KVQ_ERR_INVALID_ARG : KVQ_ERR_ALIGNMENT;
    if (append && c->length >= c->capacity) return KVQ_ERR_CAPACITY;
    const int32_t g = q_heads / c->kv_heads;
    // the static scratch (scratch_ws) is checked below against the layout of
    // the split count actually used
    if (!workspace || (!scratch_ws && ws_bytes < kvq_decode_workspace_bytes(c, q_heads))) return KVQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KVQ_ERR_ALIGNMENT;
    if (ad) {
        if (!certify || bad_tol(ad->tau_cov) || bad_tol(ad->tau_vc) || bad_tol(ad->tau_rank))
            return KVQ_ERR_INVALID_ARG;
        if ((ad->kstar && !aligned(ad->kstar, 4)) || (ad->ndisc && !aligned(ad->ndisc, 4))) return KVQ_ERR_ALIGNMENT;
        if (ws_bytes < kvq_adaptive_workspace_bytes(c, q_heads)) return KVQ_ERR_WORKSPACE;
        const int64_t len1 = c->length + (append ? 1 : 0);
        if ((len1 + kvq::BLK - 1) / kvq::BLK > kvq::ADAPT_MAX_NB) return KVQ_ERR_UNSUPPORTED;
        if (kernel == KVQ_KERNEL_VALU) return KVQ_ERR_UNSUPPORTED;
    }

    const int64_t length = c->length + (append ? 1 : 0);  // tokens the decode attends to
    const int64_t nb = (length + kvq::BLK - 1) / kvq::BLK;
    const int64_t nbc = c->capacity / kvq::BLK;
    if (nb > (int64_t)kvq::MAX_BPS * kvq::MAX_SPLITS) return KVQ_ERR_UNSUPPORTED;
    // the matrix-core kernel lists at most MFMA_MAX_BPS blocks per split
    const bool mfma_fits = kvq::mfma_supports(g) && nb <= (int64_t)kvq::MFMA_MAX_BPS * max_splits(c);
    int32_t k = kernel;
    if (k == KVQ_KERNEL_AUTO) k = mfma_fits ? KVQ_KERNEL_MFMA : KVQ_KERNEL_VALU;
    if (certify && k != KVQ_KERNEL_MFMA) return KVQ_ERR_UNSUPPORTED;  // the certificate is a matrix-core path
    // the rotated key codec is read by the matrix-core kernel only
    if (c->codec == KVQ_CODEC_ROTATE_K && k != KVQ_KERNEL_MFMA) return KVQ_ERR_UNSUPPORTED;
    if (k == KVQ_KERNEL_MFMA && !mfma_fits) return KVQ_ERR_UNSUPPORTED;
    const bool mf = k == KVQ_KERNEL_MFMA;
    // one round of matrix-core workgroups (a second round evens out groups
    // with many FP16 tiles, but pays the set-up twice: measured 3% faster on
    // the needle workload's adaptive step and 4% slower on the diffuse one).
    // The streaming kernel (plain decode) has no per-split block limit, so a
    // long sequence keeps one round there too: 8 splits of 256 blocks for
    // the 128k workload instead of 16 of 128 in two rounds.
    const bool use_stream = mf && !certify && !ad && !no_stream && kvq::stream_fits(nb);
    const int64_t max_bps = use_stream ? nb : (mf ? (int64_t)kvq::MFMA_MAX_BPS : (int64_t)kvq::MAX_BPS);
    const int64_t s = nb > 0 ? choose_splits(c, nb, splits, mf ? 1 : 4, max_bps) : 1;
    const int64_t bps = nb > 0 ? (nb + s - 1) / s : 1;
    const int64_t s_eff = nb > 0 ? (nb + bps - 1) / bps : 1;
    // offsets for the largest split count, so that passes with different
    // split counts share the certificate regions; the static scratch is laid
    // out for the split count used (no certificate or recompute pass there),
    // and checked before anything is enqueued
    const int64_t nbh = (int64_t)c->batch * c->kv_heads;
    const WsLayout w = scratch_ws ? ws_layout(c, g, s_eff, KVQ_SCRATCH_MAX_GROUPS)
                                  : ws_layout(c, g, max_splits(c), (size_t)nbh);
    if (scratch_ws && (certify || ad || nbh > (int64_t)KVQ_SCRATCH_MAX_GROUPS || w.total > ws_bytes))
        return KVQ_ERR_WORKSPACE;

    if (append && !mf) {
        // no fused path in the VALU kernel: append first
        if ((st = kvq_quantize_append(c, 1, stream)) != KVQ_OK) return st;
        append = false;
    }

    kvq::DecodeArgs a;
    a.c = ptrs(c);
    a.q = q;
    a.out = out;
    a.mask_out = mask_out;
    a.part_ml = reinterpret_cast<float2 *>((char *)workspace + w.ml);
    a.part_acc = reinterpret_cast<float *>((char *)workspace + w.acc);
    a.cap = c->capacity;
    a.length = length;
    a.nbc = nbc;
    a.nb = nb;
    a.hkv = c->kv_heads;
    a.hq = q_heads;
    a.g = g;
    a.splits = (int32_t)s_eff;
    a.bps = (int32_t)bps;
    a.sm = sm_scale;
    a.tau_k = tau_k;
    a.tau_v = tau_v;
    a.t_new = append ? c->length : -1;
    a.key_rot = c->codec == KVQ_CODEC_ROTATE_K ? 1 : 0;
    a.no_stream = no_stream ? 1 : 0;
    a.cert_mode = certify ? 1 : 0;
    a.part_e = reinterpret_cast<float *>((char *)workspace + w.e);
    a.part_sa = reinterpret_cast<float2 *>((char *)workspace + w.sa);
    a.part_kv = reinterpret_cast<float2 *>((char *)workspace + w.kv);
    a.tau_out = tau_out;
    a.cert = cert;
    a.flags = recomputed ? recomputed : reinterpret_cast<uint8_t *>((char *)workspace + w.flags);
    a.gate = nullptr;
    a.promote = nullptr;
    a.step_ml = nullptr;
    a.phead = nullptr;
    a.lhat = nullptr;
    a.ndisc = nullptr;
    a.tau_rank = 1.0f;
    // the plain matrix-core decode merges its splits in the same launch
    a.arrive = (mf && !certify && !ad) ? reinterpret_cast<uint32_t *>((char *)workspace + w.arrive) : nullptr;

    hipError_t e = hipSuccess;
    kvq::AdaptArgs aa;
    if (ad) {
        // rungs 1-2: INT8 scoring pass and selection, then the decode with the
        // promoted tiles and the FP16 step statistics of the ranking check
        const AdaptLayout al = adapt_layout(c, q_heads, kvq_decode_workspace_bytes(c, q_heads));
        aa.c = a.c;
        aa.q = q;
        aa.lhat = reinterpret_cast<float *>((char *)workspace + al.lhat);
        aa.phead = reinterpret_cast<uint8_t *>((char *)workspace + al.phead);
        aa.promote = reinterpret_cast<uint8_t *>((char *)workspace + al.promote);
        aa.kstar = ad->kstar;
        aa.qrot = reinterpret_cast<uint16_t *>((char *)workspace + al.qrot);
        aa.cap = c->capacity;
        aa.length = length;
        aa.nbc = nbc;
        aa.nb = nb;
        aa.hkv = c->kv_heads;
        aa.hq = q_heads;
        aa.g = g;
        aa.key_rot = a.key_rot;
        // the scoring pass appends the new token (it reads its codes first);
        // the decode then finds it in tier 1
        aa.t_new = a.t_new;
        a.t_new = -1;
        aa.sm = sm_scale;
        aa.tau_cov = ad->tau_cov;
        aa.tau_vc = ad->tau_vc;
        if (nb > 0) e = kvq::launch_score(aa, c->batch, (hipStream_t)stream);
        if (e == hipSuccess) e = kvq::launch_select(aa, c->batch, (hipStream_t)stream);
        a.promote = aa.promote;
        a.step_ml = reinterpret_cast<float2 *>((char *)workspace + al.step);
        a.phead = aa.phead;
        a.lhat = aa.lhat;
        a.ndisc = ad->ndisc;
        a.tau_rank = ad->tau_rank;
    }
    if (e == hipSuccess)
        e = mf ? kvq::launch_decode_mfma(a, c->batch, (hipStream_t)stream)
               : kvq::launch_decode_valu(a, c->batch, (hipStream_t)stream);
    if (e == hipSuccess && split_done) e = hipEventRecord((hipEvent_t)split_done, (hipStream_t)stream);
    if (e == hipSuccess && !a.arrive)
        e = certify ? kvq::launch_merge_cert(a, c->batch, (hipStream_t)stream)
                    : kvq::launch_merge(a, c->batch, (hipStream_t)stream);
    const bool rung3 = certify && (tau_out != __builtin_huge_valf() || (ad && ad->tau_rank < 1.0f));
    if (e == hipSuccess && rung3) {
        // rung 3: the groups holding a flagged head run again with every
        // block on FP16 (tolerances 0), and the flagged heads take the result
        // (few groups are expected to hold one: every split count the cache
        // allows, so that each spreads over many workgroups)
        const int64_t s_r = nb > 0 ? (nb < max_splits(c) ? nb : max_splits(c)) : 1;
        const int64_t bps_r = nb > 0 ? (nb + s_r - 1) / s_r : 1;
        kvq::DecodeArgs r = a;
        r.splits = (int32_t)(nb > 0 ? (nb + bps_r - 1) / bps_r : 1);
        r.bps = (int32_t)bps_r;
        r.tau_k = 0.0f;
        r.tau_v = 0.0f;
        r.t_new = -1;
        r.mask_out = nullptr;
        r.cert_mode = 0;
        r.gate = a.flags;
        r.arrive = nullptr;
        r.promote = nullptr;
        r.step_ml = nullptr;
        int64_t slots = (device_cus() + r.splits - 1) / r.splits;  // about one workgroup per CU
        if (slots > nbh) slots = nbh;
        if (slots < 1) slots = 1;
        e = kvq::launch_decode_mfma_gated(r, c->batch, (int)slots, (hipStream_t)stream);
        if (e == hipSuccess) e = kvq::launch_merge(r, c->batch, (hipStream_t)stream);
    }
    if (e != hipSuccess) return hip_fail(e);
    if (append) c->length = length;
    return KVQ_OK;
}

// Static device scratch of kvq_append_decode_noalloc: a file-scope array, one
// copy per device, whose address is looked up once per device (with that
// device current) and kept; host code uses only that address.
static __device__ __align__(256) unsigned char scratch[KVQ_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {nullptr};

kvq_status scratch_address(void **p) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= 64) return KVQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        g_scratch_ptr[dev] = ptr;
    }
    *p = g_scratch_ptr[dev];
    return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_append_decode_noalloc(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                                     float tau_k, float tau_v, uint16_t *out, uint8_t *mask_out, void *stream) {
    // argument errors first, before any device query
    kvq_status st = check_shape(c);
    if (st != KVQ_OK) return st;
    if ((st = check_query(c, q, q_heads, sm_scale, tau_k, tau_v)) != KVQ_OK) return st;
    if ((st = check_buffers(c, true)) != KVQ_OK) return st;
    if (!out) return KVQ_ERR_INVALID_ARG;
    if (!aligned(out, 16)) return KVQ_ERR_ALIGNMENT;
    if (c->length >= c->capacity) return KVQ_ERR_CAPACITY;
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != KVQ_OK) return st;
    return decode_impl(c, q, q_heads, sm_scale, tau_k, tau_v, out, mask_out, ws, KVQ_SCRATCH_BYTES, stream,
                       KVQ_KERNEL_AUTO, 0, nullptr, true, nullptr, 0.0f, nullptr, nullptr, true);
}

kvq_status kvq_decode_attn_ex(const kvq_cache *c, const uint16_t *q, int32_t q_heads,
                              float sm_scale, float tau_k, float tau_v, uint16_t *out,
                              uint8_t *mask_out, void *workspace, size_t ws_bytes, void *stream,
                              int32_t kernel, int32_t splits, void *split_done) {
    return decode_impl(const_cast<kvq_cache *>(c), q, q_heads, sm_scale, tau_k, tau_v, out, mask_out, workspace,
                       ws_bytes, stream, kernel, splits, split_done, false);
}

kvq_status kvq_decode_attn(const kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                           float tau_k, float tau_v, uint16_t *out, uint8_t *mask_out,
                           void *workspace, size_t ws_bytes, void *stream) {
    return kvq_decode_attn_ex(c, q, q_heads, sm_scale, tau_k, tau_v, out, mask_out, workspace,
                              ws_bytes, stream, KVQ_KERNEL_AUTO, 0, nullptr);
}

kvq_status kvq_append_decode_ex(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                                float tau_k, float tau_v, uint16_t *out, uint8_t *mask_out,
                                void *workspace, size_t ws_bytes, void *stream, int32_t kernel,
                                int32_t splits, void *split_done) {
    return decode_impl(c, q, q_heads, sm_scale, tau_k, tau_v, out, mask_out, workspace, ws_bytes, stream,
                       kernel, splits, split_done, true);
}

kvq_status kvq_decode_attn_cert(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale, float tau_k,
                                float tau_v, float tau_out, int32_t append, uint16_t *out, float *cert,
                                uint8_t *recomputed, uint8_t *mask_out, void *workspace, size_t ws_bytes,
                                void *stream) {
    if (!cert) return KVQ_ERR_INVALID_ARG;
    return decode_impl(c, q, q_heads, sm_scale, tau_k, tau_v, out, mask_out, workspace, ws_bytes, stream,
                       KVQ_KERNEL_AUTO, 0, nullptr, append != 0, cert, tau_out, recomputed);
}

kvq_status kvq_decode_attn_adaptive(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                                    float tau_k, float tau_v, float tau_cov, float tau_vc, float tau_rank,
                                    float tau_out, int32_t append, uint16_t *out, float *cert,
                                    uint8_t *recomputed, int32_t *kstar, int32_t *ndisc, uint8_t *mask_out,
                                    void *workspace, size_t ws_bytes, void *stream) {
    if (!cert) return KVQ_ERR_INVALID_ARG;
    const AdaptOpts ad{tau_cov, tau_vc, tau_rank, kstar, ndisc};
    return decode_impl(c, q, q_heads, sm_scale, tau_k, tau_v, out, mask_out, workspace, ws_bytes, stream,
                       KVQ_KERNEL_AUTO, 0, nullptr, append != 0, cert, tau_out, recomputed, &ad);
}

kvq_status kvq_append_decode(kvq_cache *c, const uint16_t *q, int32_t q_heads, float sm_scale,
                             float tau_k, float tau_v, uint16_t *out, uint8_t *mask_out,
                             void *workspace, size_t ws_bytes, void *stream) {
    return kvq_append_decode_ex(c, q, q_heads, sm_scale, tau_k, tau_v, out, mask_out, workspace, ws_bytes,
                                stream, KVQ_KERNEL_AUTO, 0, nullptr);
}

}  // extern "C"
