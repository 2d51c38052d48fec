// kvq_internal.hpp -- launch arguments and launcher declarations shared by the
// libkvq host code and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int D = 128;   // head dim
constexpr int BLK = 64;  // tokens per block
constexpr int VG = 32;   // channels per value group

struct CachePtrs {
    const uint16_t *k16, *v16;
    int8_t *k_codes;
    uint16_t *k_scales;
    uint8_t *v_codes;
    uint16_t *v_scales;
    float *k_err, *v_err;
};

struct AppendArgs {
    CachePtrs c;
    int64_t cap;     // tokens per sequence
    int64_t len0;    // first new token
    int64_t len1;    // one past the last new token
    int64_t blk_lo;  // first block touched (len0 / 64)
    int32_t hkv;
    int32_t key_rot;  // KVQ_CODEC_ROTATE_K: Hadamard-rotated key codec
};

struct BoundsArgs {
    const float *k_err, *v_err;
    const uint16_t *q;
    float *kb, *vb;
    uint8_t *mask;
    int64_t nbc;  // blocks of capacity (stride of k_err/v_err)
    int64_t nb;   // blocks holding valid tokens (stride of kb/vb/mask)
    int32_t hkv, hq, g;
    float sm, tau_k, tau_v;
};

struct DecodeArgs {
    CachePtrs c;
    const uint16_t *q;
    uint16_t *out;
    uint8_t *mask_out;
    float2 *part_ml;     // [B*Hkv][S][G] (running max, running sum)
    float *part_acc;     // [B*Hkv][S][G][128] unnormalised
    int64_t cap, length, nbc, nb;
    int32_t hkv, hq, g;
    int32_t splits, bps;  // number of splits and blocks per split
    float sm, tau_k, tau_v;
    int64_t t_new;  // token appended by this launch (fused append), or -1
    int32_t key_rot;  // KVQ_CODEC_ROTATE_K: codes of the rotated keys (rotate q for them)
    int32_t no_stream;  // 1: the general matrix-core kernel even where the streaming one applies
    // per-(b, kvh) arrival counters [B*Hkv], zero on entry and left zero:
    // the last workgroup of a group to write its partial merges the group's
    // splits into out in the same launch (null: a merge kernel follows)
    uint32_t *arrive;
    // per-head output certificate (matrix-core kernel with cert_mode set)
    int32_t cert_mode;
    float *part_e;          // [B*Hkv][S][G] mass-weighted value error, on the split's running-max scale
    float2 *part_sa;        // [B*Hkv][S] largest certified value scale, largest fallback |v|
    float2 *part_kv;        // [B*Hkv] largest certified key error, value error
    float tau_out;          // heads whose certificate exceeds it are recomputed on FP16
    float *cert;            // [B][Hq] certificate (written by the certificate merge)
    uint8_t *flags;         // [B][Hq] 1: the head is recomputed
    // recompute pass: per-head flags [B*Hq]; only groups holding a flagged
    // head run and only flagged heads are written (null otherwise)
    const uint8_t *gate;
    // adaptive precision (null otherwise): promoted tiles per (b, kvh,
    // block) [B*Hkv][nbc] (bit 0 key, bit 1 value), OR-ed into the bound
    // masks; with the certificate, per FP16 key step its per-head largest
    // score and exp2-sum, [B*Hkv][G][nbc][8] (log2 units), and for the
    // ranking check in the certificate merge each head's own key promotions
    // [B][Hq][nbc], its INT8 block log-masses [B][Hq][nbc], the discordant
    // pair counts [B][Hq] (or null) and tau_rank
    const uint8_t *promote;
    float2 *step_ml;
    const uint8_t *phead;
    const float *lhat;
    int32_t *ndisc;
    float tau_rank;
};

// Adaptive precision (scoring pass, top-K* selection, ranking check).
struct AdaptArgs {
    CachePtrs c;
    const uint16_t *q;
    float *lhat;             // [B][Hq][nbc] INT8 block log-masses (log2 units)
    uint8_t *phead;          // [B][Hq][nbc] 1: the head promotes the block's keys
    uint8_t *promote;        // [B][Hkv][nbc] bit 0 key, bit 1 value promotion (union over the group)
    int32_t *kstar;          // [B][Hq] blocks each head promotes, or null
    uint16_t *qrot;          // [B][Hq][2][D] rotated query, fp16 hi and lo parts (rotated codec)
    int64_t cap, length, nbc, nb;
    int64_t t_new;           // token the scoring pass appends first (its rows in k16/v16), or -1
    int32_t hkv, hq, g;
    int32_t key_rot;         // KVQ_CODEC_ROTATE_K
    float sm, tau_cov, tau_vc;
};

// Upper limits that size the workspace and LDS tables.
constexpr int MAX_SPLITS = 128;
constexpr int MAX_BPS = 1024;  // blocks per split (mask table in LDS)
constexpr int MFMA_MAX_BPS = 128;  // blocks per split of the matrix-core kernel (block table in LDS)
constexpr int ADAPT_MAX_NB = 8192;  // blocks per sequence of the adaptive path (LDS arrays)

hipError_t launch_append(const AppendArgs &a, int batch, int64_t nblk, hipStream_t s);
hipError_t launch_zero_stats(float *k_err, float *v_err, int64_t n, hipStream_t s);
hipError_t launch_bounds(const BoundsArgs &a, int batch, hipStream_t s);
// The split-K kernels (the cross-split merge is launched separately).
hipError_t launch_decode_valu(const DecodeArgs &a, int batch, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs &a, int batch, hipStream_t s);
// recompute pass: only the (b, kvh) groups holding a head with a.gate set,
// on a grid of (a.splits, slots) workgroups
hipError_t launch_decode_mfma_gated(const DecodeArgs &a, int batch, int slots, hipStream_t s);
hipError_t launch_merge(const DecodeArgs &a, int batch, hipStream_t s);
// The merge of a certified decode: outputs, per-head certificates, recompute flags.
hipError_t launch_merge_cert(const DecodeArgs &a, int batch, hipStream_t s);
bool mfma_supports(int g);
// True when a plain decode (no certificate, no promotions) of nb blocks per
// sequence runs the streaming matrix-core kernel, which takes any number of
// blocks per split (the table kernel at most MFMA_MAX_BPS).
bool stream_fits(int64_t nb);

// adaptive precision: INT8 scoring pass (a.nb > 0) and selection (the
// ranking check runs in the certificate merge when a.step_ml is set)
hipError_t launch_score(const AdaptArgs &a, int batch, hipStream_t s);
hipError_t launch_select(const AdaptArgs &a, int batch, hipStream_t s);

}  // namespace kvq
