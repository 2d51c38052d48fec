"""Host-side checks of the C ABI that need no GPU: the library loads and
exports every entry point declared in include/kvq.h, sizes are right, and
invalid arguments are rejected with the documented status before any GPU
work is enqueued (the pointers below are never dereferenced)."""
import ctypes
import math
import os
import re

import pytest

import quantized_decode_attention_kvq_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, CAPACITY, ALIGNMENT, WORKSPACE = 0, -1, -2, -3, -4, -5


def declared_functions():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", src))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"kvq_quantize_append", "kvq_bounds", "kvq_decode_attn"} <= names
    L = kvq.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(kvq.EXPORTS) == names


FAKE = 0x10000  # 64 KiB-aligned fake device address, never dereferenced


def cache(B=2, H=4, cap=256, length=0, **kw):
    c = kvq._Cache(B, H, 128, 64, 32, 0, cap, length, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def L():
    return kvq.lib()


def test_cache_bytes():
    out = (ctypes.c_size_t * 6)()
    assert L().kvq_cache_bytes(ctypes.byref(cache(B=2, H=4, cap=256)), out) == OK
    rows = 2 * 4 * 256
    assert list(out) == [rows * 128, rows * 2, rows * 64, rows * 8, rows // 64 * 4, rows // 64 * 4]


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, UNSUPPORTED), ("block_tokens", 32, UNSUPPORTED), ("v_group", 16, UNSUPPORTED),
    ("batch", 0, INVALID), ("kv_heads", 0, INVALID), ("capacity", 100, INVALID), ("length", 300, INVALID),
    ("length", -1, INVALID),
])
def test_shape_validation(field, value, status):
    out = (ctypes.c_size_t * 6)()
    assert L().kvq_cache_bytes(ctypes.byref(cache(**{field: value})), out) == status


def test_append_validation():
    c = cache(cap=256, length=200)
    assert L().kvq_quantize_append(ctypes.byref(c), 57, None) == CAPACITY
    assert L().kvq_quantize_append(ctypes.byref(c), -1, None) == INVALID
    assert L().kvq_quantize_append(ctypes.byref(c), 0, None) == OK and c.length == 200
    c = cache(k_codes=FAKE + 8)
    assert L().kvq_quantize_append(ctypes.byref(c), 1, None) == ALIGNMENT
    c = cache(v16=None)
    assert L().kvq_quantize_append(ctypes.byref(c), 1, None) == INVALID


def test_reset_validation():
    # every case fails before anything is enqueued, and length is kept
    for kw, status in [({"batch": 0}, INVALID), ({"capacity": 100}, INVALID), ({"head_dim": 64}, UNSUPPORTED),
                       ({"k_err": None}, INVALID), ({"v_err": None}, INVALID),
                       ({"k_err": FAKE + 2}, ALIGNMENT), ({"v_err": FAKE + 1}, ALIGNMENT)]:
        c = cache(cap=256, length=100, **kw)
        assert L().kvq_cache_reset(ctypes.byref(c), None) == status, kw
        assert c.length == 100
    assert L().kvq_cache_reset(None, None) == INVALID


@pytest.mark.parametrize("q_heads,tk,tv,status", [
    (3, 0.0, 0.0, INVALID),           # not a multiple of kv_heads (4)
    (4 * 17, 0.0, 0.0, UNSUPPORTED),  # G = 17 > 16
    (8, math.nan, 0.0, INVALID),
    (8, 0.0, -1.0, INVALID),
])
def test_query_validation(q_heads, tk, tv, status):
    c = cache(length=100)
    assert L().kvq_bounds(ctypes.byref(c), FAKE, q_heads, 0.1, tk, tv, None, None, None, None) == status
    assert L().kvq_decode_attn(ctypes.byref(c), FAKE, q_heads, 0.1, tk, tv, FAKE, None, FAKE, 1 << 30,
                               None) == status


def test_decode_workspace_validation():
    c = cache(length=100)
    need = L().kvq_decode_workspace_bytes(ctypes.byref(c), 8)
    assert need > 0
    assert L().kvq_decode_attn(ctypes.byref(c), FAKE, 8, 0.1, 0.0, 0.0, FAKE, None, FAKE, need - 1,
                               None) == WORKSPACE
    assert L().kvq_decode_attn(ctypes.byref(c), FAKE, 8, 0.1, 0.0, 0.0, FAKE, None, None, need,
                               None) == WORKSPACE
    assert L().kvq_decode_attn(ctypes.byref(c), FAKE, 8, math.inf, 0.0, 0.0, FAKE, None, FAKE, need,
                               None) == INVALID
    assert L().kvq_decode_attn(ctypes.byref(c), FAKE + 2, 8, 0.1, 0.0, 0.0, FAKE, None, FAKE, need,
                               None) == ALIGNMENT
    assert L().kvq_decode_workspace_bytes(ctypes.byref(c), 7) == 0


def test_status_strings():
    for s in (OK, INVALID, UNSUPPORTED, CAPACITY, ALIGNMENT, WORKSPACE, -6):
        assert L().kvq_status_str(s)
    assert L().kvq_last_hip_error() == 0


@pytest.mark.parametrize("field", ["k16", "v16"])
def test_tier2_location_rejects_null_pointers(field):
    where = ctypes.c_int32(7)
    assert L().kvq_tier2_location(ctypes.byref(cache(**{field: None})), ctypes.byref(where)) == INVALID
    assert where.value == 7
    assert L().kvq_tier2_location(None, ctypes.byref(where)) == INVALID
    assert L().kvq_tier2_location(ctypes.byref(cache()), None) == INVALID


def _adaptive(c, ws_bytes, cert=FAKE, tau_cov=0.9, tau_vc=math.inf, tau_rank=0.5, kstar=None):
    return L().kvq_decode_attn_adaptive(ctypes.byref(c), FAKE, 8, 0.1, 0.0, 0.0, tau_cov, tau_vc, tau_rank,
                                        math.inf, 0, FAKE, cert, None, kstar, None, None, FAKE, ws_bytes, None)


def test_adaptive_validation():
    c = cache(length=100)
    base = L().kvq_decode_workspace_bytes(ctypes.byref(c), 8)
    need = L().kvq_adaptive_workspace_bytes(ctypes.byref(c), 8)
    assert need > base > 0
    assert L().kvq_adaptive_workspace_bytes(ctypes.byref(c), 7) == 0
    assert _adaptive(c, need - 1) == WORKSPACE
    assert _adaptive(c, need, cert=None) == INVALID
    for kw in (dict(tau_cov=math.nan), dict(tau_cov=-0.5), dict(tau_vc=math.nan), dict(tau_rank=-1.0)):
        assert _adaptive(c, need, **kw) == INVALID, kw
    assert _adaptive(c, need, kstar=FAKE + 2) == ALIGNMENT
    # more than 8192 blocks per sequence
    big = cache(B=1, H=1, cap=8194 * 64, length=8193 * 64 + 1)
    assert _adaptive(big, L().kvq_adaptive_workspace_bytes(ctypes.byref(big), 8)) == UNSUPPORTED


def test_codec_validation():
    out = (ctypes.c_size_t * 6)()
    assert L().kvq_cache_bytes(ctypes.byref(cache(codec=1)), out) == OK
    assert L().kvq_cache_bytes(ctypes.byref(cache(codec=2)), out) == UNSUPPORTED
    assert L().kvq_quantize_append(ctypes.byref(cache(codec=-1)), 1, None) == UNSUPPORTED


def test_library_matches_sources(monkeypatch):
    # the loaded library was built from the present sources; one built from
    # other sources is refused rather than loaded
    assert kvq._build.is_current()
    monkeypatch.setattr(kvq._build, "source_hash", lambda: "0" * 64)
    assert not kvq._build.is_current()
    monkeypatch.setattr(kvq, "_lib", None)
    with pytest.raises(RuntimeError, match="not built from the present sources"):
        kvq.lib()
