"""Python binding of libkvq (include/kvq.h): certified quantized-KV decode
attention for AMD MI355X.

Argument marshalling only: every step runs in the HIP kernels of libkvq.so.
PyTorch provides device memory (tensors) and streams; nothing here computes
on the data, and there is no CPU fallback: without the built library every
call raises.

Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1
(INT8 keys / INT4 values with scales and per-block error annotations, FP16
originals for fallback) and Methodology 2 (key and value error terms
evaluated online per block from the statistics and the query norm).
"""
import ctypes
import math
import os

import torch

from . import build as _build

D = 128
BLK = 64
VG = 32

KVQ_OK = 0
KERNEL_AUTO, KERNEL_VALU, KERNEL_MFMA, KERNEL_MFMA_TABLE = 0, 1, 2, 3
KVQ_CODEC_PLAIN, KVQ_CODEC_ROTATE_K = 0, 1
DEFAULT_SM_SCALE = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))


class KvqError(RuntimeError):
    def __init__(self, fn, status, hip):
        msg = f"{fn} failed: {lib().kvq_status_str(status).decode()} (status {status}"
        if hip:
            msg += f", hipError {hip}"
        super().__init__(msg + ")")
        self.status = status


class _Cache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32), ("v_group", ctypes.c_int32), ("codec", ctypes.c_int32),
        ("capacity", ctypes.c_int64), ("length", ctypes.c_int64),
        ("k16", ctypes.c_void_p), ("v16", ctypes.c_void_p),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("k_err", ctypes.c_void_p), ("v_err", ctypes.c_void_p),
    ]


_lib = None
EXPORTS = ("kvq_cache_bytes", "kvq_cache_reset", "kvq_quantize_append", "kvq_bounds", "kvq_decode_workspace_bytes",
           "kvq_decode_attn", "kvq_decode_attn_ex", "kvq_append_decode", "kvq_append_decode_ex",
           "kvq_decode_attn_cert", "kvq_adaptive_workspace_bytes", "kvq_decode_attn_adaptive",
           "kvq_tier2_location", "kvq_append_decode_noalloc", "kvq_status_str", "kvq_last_hip_error")


def lib_path():
    return _build.LIB


def lib():
    """Load libkvq.so (building it in-tree first if it is absent).  A library
    built from other sources than the present csrc/ and include/kvq.h is
    refused: rebuild it with quantized_decode_attention_kvq_amd.build.build()."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        if not _build.is_current():
            raise RuntimeError(f"{_build.LIB} was not built from the present sources (csrc/, include/kvq.h); "
                               "rebuild it (python -m quantized_decode_attention_kvq_amd.build)")
        L = ctypes.CDLL(_build.LIB)
        P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        CP = ctypes.POINTER(_Cache)
        L.kvq_cache_bytes.argtypes = [CP, ctypes.POINTER(sz)]
        L.kvq_cache_bytes.restype = ctypes.c_int
        L.kvq_quantize_append.argtypes = [CP, i64, P]
        L.kvq_quantize_append.restype = ctypes.c_int
        L.kvq_cache_reset.argtypes = [CP, P]
        L.kvq_cache_reset.restype = ctypes.c_int
        L.kvq_bounds.argtypes = [CP, P, i32, f32, f32, f32, P, P, P, P]
        L.kvq_bounds.restype = ctypes.c_int
        L.kvq_decode_workspace_bytes.argtypes = [CP, i32]
        L.kvq_decode_workspace_bytes.restype = sz
        L.kvq_decode_attn.argtypes = [CP, P, i32, f32, f32, f32, P, P, P, sz, P]
        L.kvq_decode_attn.restype = ctypes.c_int
        L.kvq_decode_attn_ex.argtypes = [CP, P, i32, f32, f32, f32, P, P, P, sz, P, i32, i32, P]
        L.kvq_decode_attn_ex.restype = ctypes.c_int
        L.kvq_append_decode.argtypes = [CP, P, i32, f32, f32, f32, P, P, P, sz, P]
        L.kvq_append_decode.restype = ctypes.c_int
        L.kvq_append_decode_ex.argtypes = [CP, P, i32, f32, f32, f32, P, P, P, sz, P, i32, i32, P]
        L.kvq_append_decode_ex.restype = ctypes.c_int
        L.kvq_decode_attn_cert.argtypes = [CP, P, i32, f32, f32, f32, f32, i32, P, P, P, P, P, sz, P]
        L.kvq_decode_attn_cert.restype = ctypes.c_int
        L.kvq_adaptive_workspace_bytes.argtypes = [CP, i32]
        L.kvq_adaptive_workspace_bytes.restype = sz
        L.kvq_decode_attn_adaptive.argtypes = [CP, P, i32, f32, f32, f32, f32, f32, f32, f32, i32,
                                               P, P, P, P, P, P, P, sz, P]
        L.kvq_decode_attn_adaptive.restype = ctypes.c_int
        L.kvq_append_decode_noalloc.argtypes = [CP, P, i32, f32, f32, f32, P, P, P]
        L.kvq_append_decode_noalloc.restype = ctypes.c_int
        L.kvq_tier2_location.argtypes = [CP, ctypes.POINTER(i32)]
        L.kvq_tier2_location.restype = ctypes.c_int
        L.kvq_status_str.argtypes = [ctypes.c_int]
        L.kvq_status_str.restype = ctypes.c_char_p
        L.kvq_last_hip_error.argtypes = []
        L.kvq_last_hip_error.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn, status):
    if status != KVQ_OK:
        raise KvqError(fn, status, lib().kvq_last_hip_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _event(ev):
    """A torch.cuda.Event, a raw hipEvent_t (int or c_void_p), or None."""
    if ev is None:
        return None
    if hasattr(ev, "cuda_event"):
        return ctypes.c_void_p(ev.cuda_event)
    return ev if isinstance(ev, ctypes.c_void_p) else ctypes.c_void_p(int(ev))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class KVCache:
    """One layer's KV cache: FP16 originals (tier 2) and the quantized tier 1,
    as torch tensors on one device.  Shapes (head-major, per include/kvq.h):
        k16, v16   fp16  [B][Hkv][cap][128]
        k_codes    int8  [B][Hkv][cap][128]
        k_scales   fp16  [B][Hkv][cap]
        v_codes    uint8 [B][Hkv][cap/64][128][32]
        v_scales   fp16  [B][Hkv][cap][4]
        k_err, v_err float32 [B][Hkv][cap/64]
    `length` is host-side and advanced by kvq_quantize_append.
    tier2="host" keeps k16/v16 in pinned host memory that the kernels read
    in place (zero-copy over the host link), checked by kvq_tier2_location.
    key_rotation=True selects the Hadamard-rotated key codec
    (KVQ_CODEC_ROTATE_K)."""

    def __init__(self, batch, kv_heads, capacity, device="cuda", k16=None, v16=None, tier2="device",
                 key_rotation=False):
        if capacity % BLK:
            raise ValueError("capacity must be a multiple of 64")
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        if tier2 not in ("device", "host"):
            raise ValueError("tier2 must be 'device' or 'host'")
        shape = (batch, kv_heads, capacity, D)
        self.batch, self.kv_heads, self.capacity, self.length = batch, kv_heads, capacity, 0
        self.tier2 = tier2
        self.codec = KVQ_CODEC_ROTATE_K if key_rotation else KVQ_CODEC_PLAIN
        host = tier2 == "host"
        t2dev = torch.device("cpu") if host else dev
        self.k16 = k16 if k16 is not None else torch.zeros(shape, dtype=torch.float16, device=t2dev, pin_memory=host)
        self.v16 = v16 if v16 is not None else torch.zeros(shape, dtype=torch.float16, device=t2dev, pin_memory=host)
        for t in (self.k16, self.v16):
            placed = (t.device.type == "cpu" and t.is_pinned()) if host else t.device == dev
            if t.shape != shape or t.dtype != torch.float16 or not t.is_contiguous() or not placed:
                where = "pinned host memory" if host else str(dev)
                raise ValueError(f"tier-2 tensors must be contiguous fp16 {shape} in {where}")
        nbc = capacity // BLK
        self.k_codes = torch.empty(shape, dtype=torch.int8, device=dev)
        self.k_scales = torch.empty((batch, kv_heads, capacity), dtype=torch.float16, device=dev)
        self.v_codes = torch.empty((batch, kv_heads, nbc, D, BLK // 2), dtype=torch.uint8, device=dev)
        self.v_scales = torch.empty((batch, kv_heads, capacity, D // VG), dtype=torch.float16, device=dev)
        self.k_err = torch.zeros((batch, kv_heads, nbc), dtype=torch.float32, device=dev)
        self.v_err = torch.zeros((batch, kv_heads, nbc), dtype=torch.float32, device=dev)
        if host:
            with torch.cuda.device(dev):
                where = kvq_tier2_location(self)
            if where != 1:
                raise ValueError("tier 2 is not host memory the device reads in place")

    @property
    def nblocks(self):
        return (self.length + BLK - 1) // BLK

    def c_struct(self):
        return _Cache(self.batch, self.kv_heads, D, BLK, VG, self.codec, self.capacity, self.length,
                      self.k16.data_ptr(), self.v16.data_ptr(), self.k_codes.data_ptr(),
                      self.k_scales.data_ptr(), self.v_codes.data_ptr(), self.v_scales.data_ptr(),
                      self.k_err.data_ptr(), self.v_err.data_ptr())

    def tier1_bytes(self):
        out = (ctypes.c_size_t * 6)()
        _check("kvq_cache_bytes", lib().kvq_cache_bytes(ctypes.byref(self.c_struct()), out))
        return list(out)


def kvq_decode_attn_adaptive(cache: KVCache, q, sm_scale=DEFAULT_SM_SCALE, tau_k=0.0, tau_v=0.0, tau_cov=0.995,
                             tau_vc=float("inf"), tau_rank=1.0, tau_out=float("inf"), append=False, out=None,
                             cert=None, recomputed=None, kstar=None, ndisc=None, mask_out=None, workspace=None,
                             stream=None):
    """Adaptive precision with the fallback ladder (see include/kvq.h):
    INT8 scoring pass, top-K* promotion covering tau_cov of the estimated
    mass, value promotion above tau_vc, the certified decode, the ranking
    check (inconsistent above tau_rank) and the FP16 recompute of
    inconsistent heads and of heads whose certificate exceeds tau_out.
    Returns dict(out, cert, recomputed, kstar, ndisc)."""
    _check_q(cache, q)
    B, Hq = q.shape[0], q.shape[1]
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if cert is None:
        cert = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if recomputed is None:
        recomputed = torch.empty((B, Hq), dtype=torch.uint8, device=dev)
    if kstar is None:
        kstar = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    if ndisc is None:
        ndisc = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = make_workspace(cache, Hq, dev, adaptive=True)
    c = cache.c_struct()
    st = lib().kvq_decode_attn_adaptive(ctypes.byref(c), _ptr(q), Hq, sm_scale, tau_k, tau_v, tau_cov, tau_vc,
                                        tau_rank, tau_out, 1 if append else 0, _ptr(out), _ptr(cert),
                                        _ptr(recomputed), _ptr(kstar), _ptr(ndisc), _ptr(mask_out),
                                        _ptr(workspace), workspace.numel(), _stream(stream))
    _check("kvq_decode_attn_adaptive", st)
    cache.length = int(c.length)
    return dict(out=out, cert=cert, recomputed=recomputed, kstar=kstar, ndisc=ndisc)


def kvq_tier2_location(cache: KVCache) -> int:
    """0 if the cache's tier 2 is device memory, 1 if it is pinned host memory
    the device reads in place (raises KvqError otherwise)."""
    where = ctypes.c_int32(-1)
    _check("kvq_tier2_location", lib().kvq_tier2_location(ctypes.byref(cache.c_struct()), ctypes.byref(where)))
    return int(where.value)


def kvq_quantize_append(cache: KVCache, n_new: int, stream=None):
    """Quantize tokens [length, length+n_new) of cache.k16/v16 into tier 1 and
    advance cache.length (asynchronous on `stream`)."""
    c = cache.c_struct()
    _check("kvq_quantize_append", lib().kvq_quantize_append(ctypes.byref(c), int(n_new), _stream(stream)))
    cache.length = int(c.length)


def kvq_cache_reset(cache: KVCache, stream=None):
    """Empty the cache for reuse (asynchronous on `stream`): zero the block
    statistics and set length to 0."""
    c = cache.c_struct()
    _check("kvq_cache_reset", lib().kvq_cache_reset(ctypes.byref(c), _stream(stream)))
    cache.length = int(c.length)


def _check_q(cache, q):
    if q.dtype != torch.float16 or not q.is_contiguous() or q.dim() != 3 or q.shape[0] != cache.batch \
            or q.shape[2] != D:
        raise ValueError("q must be a contiguous fp16 tensor [B][Hq][128]")


def kvq_bounds(cache: KVCache, q, sm_scale=DEFAULT_SM_SCALE, tau_k=0.0, tau_v=0.0, want=("kb", "vb", "mask"),
               stream=None):
    """Per-block key bound, value bound and fallback mask, each
    [B][Hkv][nblocks] (float32, float32, uint8); entries not in `want` are None."""
    _check_q(cache, q)
    nb = cache.nblocks
    dev = q.device
    kb = torch.empty((cache.batch, cache.kv_heads, nb), dtype=torch.float32, device=dev) if "kb" in want else None
    vb = torch.empty((cache.batch, cache.kv_heads, nb), dtype=torch.float32, device=dev) if "vb" in want else None
    mask = torch.empty((cache.batch, cache.kv_heads, nb), dtype=torch.uint8, device=dev) if "mask" in want else None
    c = cache.c_struct()
    _check("kvq_bounds", lib().kvq_bounds(ctypes.byref(c), _ptr(q), q.shape[1], sm_scale, tau_k, tau_v,
                                          _ptr(kb), _ptr(vb), _ptr(mask), _stream(stream)))
    return kb, vb, mask


def kvq_decode_workspace_bytes(cache: KVCache, q_heads: int) -> int:
    return int(lib().kvq_decode_workspace_bytes(ctypes.byref(cache.c_struct()), int(q_heads)))


def kvq_adaptive_workspace_bytes(cache: KVCache, q_heads: int) -> int:
    return int(lib().kvq_adaptive_workspace_bytes(ctypes.byref(cache.c_struct()), int(q_heads)))


def kvq_append_decode_noalloc(cache: KVCache, q, sm_scale=DEFAULT_SM_SCALE, tau_k=0.0, tau_v=0.0, out=None,
                              mask_out=None, stream=None):
    """kvq_append_decode with its split partials in the library's static
    device scratch (no workspace; the library call allocates nothing).  Pass
    `out` to keep the binding from allocating it."""
    _check_q(cache, q)
    if out is None:
        out = torch.empty_like(q)
    c = cache.c_struct()
    st = lib().kvq_append_decode_noalloc(ctypes.byref(c), _ptr(q), q.shape[1], sm_scale, tau_k, tau_v, _ptr(out),
                                         _ptr(mask_out), _stream(stream))
    _check("kvq_append_decode_noalloc", st)
    cache.length = int(c.length)
    return out


def make_workspace(cache: KVCache, q_heads: int, device=None, adaptive=False):
    """A zero-filled workspace for the decode entry points (reusable across
    calls); adaptive=True sizes it for kvq_decode_attn_adaptive too."""
    n = (kvq_adaptive_workspace_bytes if adaptive else kvq_decode_workspace_bytes)(cache, q_heads)
    if n == 0:
        raise ValueError("invalid cache shape or q_heads")
    return torch.zeros(n, dtype=torch.uint8, device=device or cache.k_codes.device)


def kvq_decode_attn(cache: KVCache, q, sm_scale=DEFAULT_SM_SCALE, tau_k=0.0, tau_v=0.0, out=None,
                    mask_out=None, workspace=None, stream=None, kernel=KERNEL_AUTO, splits=0, split_done=None):
    """Certified decode attention: q [B][Hq][128] fp16 -> out [B][Hq][128] fp16.
    mask_out (optional uint8 [B][Hkv][nblocks]) receives the fallback masks.
    split_done (optional: a torch.cuda.Event already recorded once so that it
    exists, or a raw hipEvent_t) is recorded between the split-K kernel and
    the merge kernel."""
    _check_q(cache, q)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = make_workspace(cache, q.shape[1], q.device)
    c = cache.c_struct()
    st = lib().kvq_decode_attn_ex(ctypes.byref(c), _ptr(q), q.shape[1], sm_scale, tau_k, tau_v, _ptr(out),
                                  _ptr(mask_out), _ptr(workspace), workspace.numel(), _stream(stream),
                                  int(kernel), int(splits),
                                  _event(split_done))
    _check("kvq_decode_attn", st)
    return out


def kvq_append_decode(cache: KVCache, q, sm_scale=DEFAULT_SM_SCALE, tau_k=0.0, tau_v=0.0, out=None,
                      mask_out=None, workspace=None, stream=None, kernel=KERNEL_AUTO, splits=0, split_done=None):
    """One decode step: quantize token cache.length (its fp16 rows already in
    cache.k16/v16) and attend over cache.length+1 tokens, in one launch of the
    matrix-core kernel; advances cache.length.  Same arguments and results as
    kvq_quantize_append(cache, 1) followed by kvq_decode_attn."""
    _check_q(cache, q)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = make_workspace(cache, q.shape[1], q.device)
    c = cache.c_struct()
    st = lib().kvq_append_decode_ex(ctypes.byref(c), _ptr(q), q.shape[1], sm_scale, tau_k, tau_v, _ptr(out),
                                    _ptr(mask_out), _ptr(workspace), workspace.numel(), _stream(stream),
                                    int(kernel), int(splits),
                                    _event(split_done))
    _check("kvq_append_decode", st)
    cache.length = int(c.length)
    return out


def kvq_decode_attn_cert(cache: KVCache, q, sm_scale=DEFAULT_SM_SCALE, tau_k=0.0, tau_v=0.0,
                         tau_out=float("inf"), append=False, out=None, cert=None, recomputed=None,
                         mask_out=None, workspace=None, stream=None):
    """Certified decode with a per-head output certificate (float32 [B][Hq])
    and recompute on FP16 of the heads whose certificate exceeds tau_out
    (recomputed: uint8 [B][Hq], 1 for those heads).  With append, token
    cache.length is quantized first and cache.length advances.  Returns
    (out, cert, recomputed)."""
    _check_q(cache, q)
    B, Hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if cert is None:
        cert = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if recomputed is None:
        recomputed = torch.empty((B, Hq), dtype=torch.uint8, device=q.device)
    if workspace is None:
        workspace = make_workspace(cache, Hq, q.device)
    c = cache.c_struct()
    st = lib().kvq_decode_attn_cert(ctypes.byref(c), _ptr(q), Hq, sm_scale, tau_k, tau_v, tau_out,
                                    1 if append else 0, _ptr(out), _ptr(cert), _ptr(recomputed),
                                    _ptr(mask_out), _ptr(workspace), workspace.numel(), _stream(stream))
    _check("kvq_decode_attn_cert", st)
    cache.length = int(c.length)
    return out, cert, recomputed
