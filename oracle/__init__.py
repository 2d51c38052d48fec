"""CPU oracle for certified quantized-KV decode attention (numpy front end).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  The
arithmetic lives in kvq_oracle.c (plain C loops, fp64) and follows
"Runtime-Certified Bounded-Error Quantized Attention", technical summary,
Methodology 1 (tiered INT8-key / INT4-value storage with FP16 originals) and
Methodology 2 (key and value error terms computed online).  The readings of
the page used here are spelled out in kvq_oracle.c's header.

All fp16 arrays are numpy float16 (IEEE binary16); layouts are those of the
header of kvq_oracle.c.
"""
import ctypes
import os

import numpy as np

from . import build as _build

D = 128
BLK = 64
VG = 32

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.kvqo_max_threads.argtypes = []
        L.kvqo_max_threads.restype = ctypes.c_int
        L.kvqo_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.kvqo_f16_to_f64.restype = ctypes.c_double
        L.kvqo_f32_to_f16.argtypes = [f32]
        L.kvqo_f32_to_f16.restype = ctypes.c_uint16
        L.kvqo_f32_to_f16_array.argtypes = [P, P, i64]
        L.kvqo_f32_to_f16_array.restype = None
        L.kvqo_tree128.argtypes = [P]
        L.kvqo_tree128.restype = ctypes.c_double
        L.kvqo_qnorm.argtypes = [P]
        L.kvqo_qnorm.restype = f32
        L.kvqo_group_qnorm.argtypes = [P, i32, i32, i32, i32]
        L.kvqo_group_qnorm.restype = f32
        L.kvqo_key_bound.argtypes = [f32, f32, f32]
        L.kvqo_key_bound.restype = f32
        L.kvqo_quant_k_row.argtypes = [P, P, P, P]
        L.kvqo_quant_k_row.restype = None
        L.kvqo_quant_v_row.argtypes = [P, P, P, P]
        L.kvqo_quant_v_row.restype = None
        L.kvqo_quantize_cache.argtypes = [i32, i32, i64, i64, P, P, P, P, P, P, P, P, i32]
        L.kvqo_quantize_cache.restype = None
        L.kvqo_bounds.argtypes = [i32, i32, i32, i64, i64, P, f32, f32, f32, P, P, P, P, P]
        L.kvqo_bounds.restype = None
        L.kvqo_attention.argtypes = [i32, i32, i32, i64, i64, P, f32, f32, f32,
                                     P, P, P, P, P, P, P, P, P, P, i32]
        L.kvqo_attention.restype = None
        L.kvqo_certificate.argtypes = [i32, i32, i32, i64, i64, P, f32, f32, f32, ctypes.c_double,
                                       P, P, P, P, P, P, P, P, P, P, P, P, P, i32]
        L.kvqo_certificate.restype = None
        L.kvqo_certify_masked.argtypes = [i32, i32, i32, i64, i64, P, f32, P, ctypes.c_double, P,
                                          P, P, P, P, P, P, P, P, P, P, P, P, P, i32]
        L.kvqo_certify_masked.restype = None
        dbl = ctypes.c_double
        L.kvqo_adaptive.argtypes = [i32, i32, i32, i64, i64, P, f32, f32, f32, dbl, dbl, dbl, dbl] + [P] * 20 + [i32]
        L.kvqo_quant_k_row_rot.argtypes = [P, P, P, P]
        L.kvqo_quant_k_row_rot.restype = None
        L.kvqo_adaptive.restype = None
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------- scalars

def max_threads() -> int:
    return int(lib().kvqo_max_threads())


def f16_bits_to_f64(bits: int) -> float:
    return lib().kvqo_f16_to_f64(int(bits) & 0xFFFF)


def f32_to_f16_bits(x: float) -> int:
    return int(lib().kvqo_f32_to_f16(float(np.float32(x))))


def f32_to_f16_array(x):
    """float32 array -> uint16 fp16 bit patterns (RNE)."""
    x = _c(x, np.float32)
    out = np.zeros(x.shape, np.uint16)
    lib().kvqo_f32_to_f16_array(_p(x), _p(out), x.size)
    return out


def tree128(v) -> float:
    v = _c(v, np.float64)
    assert v.shape == (D,)
    return lib().kvqo_tree128(_p(v))


def qnorm(q) -> float:
    q = _c(q, np.float16)
    assert q.shape == (D,)
    return float(np.float32(lib().kvqo_qnorm(_p(q))))


def key_bound(sm: float, qn: float, kerr: float) -> float:
    return float(np.float32(lib().kvqo_key_bound(sm, qn, kerr)))


def quant_k_row(x):
    """Returns (codes int8[128], scale float16, err float32)."""
    x = _c(x, np.float16)
    codes = np.zeros(D, np.int8)
    scale = np.zeros(1, np.float16)
    err = np.zeros(1, np.float32)
    lib().kvqo_quant_k_row(_p(x), _p(codes), _p(scale), _p(err))
    return codes, scale[0], err[0]


def quant_k_row_rot(x):
    """The rotated key codec on one row: (codes int8[128] of u = H x / 16,
    scale float16, err float32 = ||x - x~||)."""
    x = _c(x, np.float16)
    codes = np.zeros(D, np.int8)
    scale = np.zeros(1, np.float16)
    err = np.zeros(1, np.float32)
    lib().kvqo_quant_k_row_rot(_p(x), _p(codes), _p(scale), _p(err))
    return codes, scale[0], err[0]


def quant_v_row(x):
    """Returns (codes int8[128] in [-7,7], scales float16[4], err float32)."""
    x = _c(x, np.float16)
    codes = np.zeros(D, np.int8)
    scales = np.zeros(4, np.float16)
    err = np.zeros(1, np.float32)
    lib().kvqo_quant_v_row(_p(x), _p(codes), _p(scales), _p(err))
    return codes, scales, err[0]


# ----------------------------------------------------------------- cache

class Cache:
    """The oracle's own quantized cache (tier 1) for fp16 tier-2 arrays.
    key_rotation: the keys are quantized after the Hadamard rotation
    (kvqo_quant_k_row_rot) and read back through its inverse."""

    def __init__(self, k16, v16, length, key_rotation=False):
        k16 = _c(k16, np.float16)
        v16 = _c(v16, np.float16)
        B, Hkv, cap, d = k16.shape
        assert d == D and cap % BLK == 0 and v16.shape == k16.shape and 0 <= length <= cap
        self.B, self.Hkv, self.cap, self.length = B, Hkv, cap, int(length)
        self.key_rotation = bool(key_rotation)
        self.k16, self.v16 = k16, v16
        nb = cap // BLK
        self.k_codes = np.zeros((B, Hkv, cap, D), np.int8)
        self.k_scales = np.zeros((B, Hkv, cap), np.float16)
        self.v_codes = np.zeros((B, Hkv, nb, D, BLK // 2), np.uint8)
        self.v_scales = np.zeros((B, Hkv, cap, D // VG), np.float16)
        self.k_err = np.zeros((B, Hkv, nb), np.float32)
        self.v_err = np.zeros((B, Hkv, nb), np.float32)
        lib().kvqo_quantize_cache(B, Hkv, cap, self.length, _p(k16), _p(v16), _p(self.k_codes),
                                  _p(self.k_scales), _p(self.v_codes), _p(self.v_scales),
                                  _p(self.k_err), _p(self.v_err), int(self.key_rotation))

    @property
    def nblocks(self):
        return (self.length + BLK - 1) // BLK

    def v_codes_unpacked(self):
        """int8 [B][Hkv][cap][128] in [-8, 7] read back from the packed layout."""
        vc = self.v_codes  # [B][Hkv][nb][D][32]
        lo = (vc & 0x0F).astype(np.int16)
        hi = (vc >> 4).astype(np.int16)
        tok = np.stack([lo, hi], axis=-1).reshape(self.B, self.Hkv, -1, D, BLK)  # [..nb, D, 64]
        tok = np.where(tok >= 8, tok - 16, tok).astype(np.int8)
        return tok.transpose(0, 1, 2, 4, 3).reshape(self.B, self.Hkv, -1, D)

    def bounds(self, q, sm, tau_k, tau_v):
        """kb, vb float32 and mask uint8, each [B][Hkv][nblocks]."""
        q = _c(q, np.float16)
        B, Hq, d = q.shape
        assert B == self.B and d == D and Hq % self.Hkv == 0
        nb = self.nblocks
        kb = np.zeros((B, self.Hkv, nb), np.float32)
        vb = np.zeros((B, self.Hkv, nb), np.float32)
        mask = np.zeros((B, self.Hkv, nb), np.uint8)
        lib().kvqo_bounds(B, Hq, self.Hkv, self.cap, self.length, _p(q), sm, tau_k, tau_v,
                          _p(self.k_err), _p(self.v_err), _p(kb), _p(vb), _p(mask))
        return kb, vb, mask

    def attention(self, q, sm, tau_k, tau_v):
        """fp64 output [B][Hq][128] and mask uint8 [B][Hkv][nblocks]."""
        q = _c(q, np.float16)
        B, Hq, d = q.shape
        assert B == self.B and d == D and Hq % self.Hkv == 0
        out = np.zeros((B, Hq, D), np.float64)
        mask = np.zeros((B, self.Hkv, max(self.nblocks, 1)), np.uint8)
        lib().kvqo_attention(B, Hq, self.Hkv, self.cap, self.length, _p(q), sm, tau_k, tau_v,
                             _p(self.k16), _p(self.v16), _p(self.k_codes), _p(self.k_scales),
                             _p(self.v_codes), _p(self.v_scales), _p(self.k_err), _p(self.v_err),
                             _p(out), _p(mask), int(self.key_rotation))
        return out, mask[:, :, : self.nblocks]


    def certificate(self, q, sm, tau_k, tau_v, tau_out=float("inf")):
        """Per-head certificate and rung-3 recompute (see kvqo_certificate):
        dict of out (fp64 [B][Hq][128], recomputed heads dense), cert, e_key,
        e_val (fp64 [B][Hq]) and recomputed (uint8 [B][Hq])."""
        q = _c(q, np.float16)
        B, Hq, d = q.shape
        assert B == self.B and d == D and Hq % self.Hkv == 0
        r = {k: np.zeros((B, Hq), np.float64) for k in ("cert", "e_key", "e_val")}
        r["out"] = np.zeros((B, Hq, D), np.float64)
        r["recomputed"] = np.zeros((B, Hq), np.uint8)
        lib().kvqo_certificate(B, Hq, self.Hkv, self.cap, self.length, _p(q), sm, tau_k, tau_v,
                               float(tau_out), _p(self.k16), _p(self.v16), _p(self.k_codes),
                               _p(self.k_scales), _p(self.v_codes), _p(self.v_scales), _p(self.k_err),
                               _p(self.v_err), _p(r["out"]), _p(r["cert"]), _p(r["e_key"]),
                               _p(r["e_val"]), _p(r["recomputed"]), int(self.key_rotation))
        return r


    def certify_masked(self, q, sm, masks, tau_out=float("inf"), force=None):
        """As certificate, under fallback masks given by the caller (uint8
        [B][Hkv][nblocks]) instead of the bounds' masks, with the FP16
        recompute also forced where force (uint8 [B][Hq], optional) is set."""
        q = _c(q, np.float16)
        B, Hq, d = q.shape
        assert B == self.B and d == D and Hq % self.Hkv == 0
        nb = self.nblocks
        m = np.zeros((B, self.Hkv, max(nb, 1)), np.uint8)
        m[:, :, :nb] = np.asarray(masks, np.uint8)[:, :, :nb]
        f = None if force is None else _c(np.asarray(force, np.uint8).reshape(B, Hq), np.uint8)
        r = {k: np.zeros((B, Hq), np.float64) for k in ("cert", "e_key", "e_val")}
        r["out"] = np.zeros((B, Hq, D), np.float64)
        r["recomputed"] = np.zeros((B, Hq), np.uint8)
        lib().kvqo_certify_masked(B, Hq, self.Hkv, self.cap, self.length, _p(q), sm, _p(m), float(tau_out),
                                  None if f is None else _p(f), _p(self.k16), _p(self.v16), _p(self.k_codes),
                                  _p(self.k_scales), _p(self.v_codes), _p(self.v_scales), _p(self.k_err),
                                  _p(self.v_err), _p(r["out"]), _p(r["cert"]), _p(r["e_key"]),
                                  _p(r["e_val"]), _p(r["recomputed"]), int(self.key_rotation))
        return r

    def adaptive(self, q, sm, tau_k, tau_v, tau_cov, tau_vc=float("inf"), tau_rank=1.0, tau_out=float("inf")):
        """Adaptive precision with the ranking check and rungs 1-3 (see
        kvqo_adaptive): dict of out, cert, e_key, e_val, recomputed (as
        certificate), masks (uint8 [B][Hkv][NB], bounds OR promotions), lhat
        and lfp (fp64 [B][Hq][NB], natural-log block masses from the INT8 and
        FP16 keys), kstar (int32 [B][Hq]), ndisc and npairs (int64 [B][Hq])
        and inconsistent (uint8 [B][Hq])."""
        q = _c(q, np.float16)
        B, Hq, d = q.shape
        assert B == self.B and d == D and Hq % self.Hkv == 0
        nb = (self.length + BLK - 1) // BLK
        r = {k: np.zeros((B, Hq), np.float64) for k in ("cert", "e_key", "e_val")}
        r["out"] = np.zeros((B, Hq, D), np.float64)
        r["recomputed"] = np.zeros((B, Hq), np.uint8)
        r["masks"] = np.zeros((B, self.Hkv, max(nb, 1)), np.uint8)
        r["lhat"] = np.zeros((B, Hq, max(nb, 1)), np.float64)
        r["lfp"] = np.zeros((B, Hq, max(nb, 1)), np.float64)
        r["kstar"] = np.zeros((B, Hq), np.int32)
        r["ndisc"] = np.zeros((B, Hq), np.int64)
        r["npairs"] = np.zeros((B, Hq), np.int64)
        r["inconsistent"] = np.zeros((B, Hq), np.uint8)
        lib().kvqo_adaptive(B, Hq, self.Hkv, self.cap, self.length, _p(q), sm, tau_k, tau_v, float(tau_cov),
                            float(tau_vc), float(tau_rank), float(tau_out), _p(self.k16), _p(self.v16),
                            _p(self.k_codes), _p(self.k_scales), _p(self.v_codes), _p(self.v_scales),
                            _p(self.k_err), _p(self.v_err), _p(r["out"]), _p(r["cert"]), _p(r["e_key"]),
                            _p(r["e_val"]), _p(r["recomputed"]), _p(r["masks"]), _p(r["lhat"]), _p(r["lfp"]),
                            _p(r["kstar"]), _p(r["ndisc"]), _p(r["npairs"]), _p(r["inconsistent"]),
                            int(self.key_rotation))
        for k in ("masks", "lhat", "lfp"):
            r[k] = r[k][..., :nb]
        return r


def tau_for_fraction(values, frac):
    """Tolerance that makes about `frac` of `values` exceed it: the midpoint
    between the sorted values around rank N - max(1, round(frac*N)).
    Non-finite values always exceed any finite tolerance and are ignored."""
    v = np.sort(np.asarray(values, np.float64).ravel())
    v = v[np.isfinite(v)]
    n = v.size
    if n == 0:
        return float("inf")
    k = max(1, int(round(frac * n)))
    if k >= n:
        return 0.0
    lo, hi = v[n - k - 1], v[n - k]
    return float(np.float32((lo + hi) / 2.0))
