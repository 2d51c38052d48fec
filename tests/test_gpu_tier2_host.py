"""Tier 2 in pinned host memory (the placement Methodology 1 gives the FP16
originals): kvq_tier2_location reports it, and every kernel reads it in
place -- the bulk and fused appends (tier-1 bytes bitwise against the
oracle), the decode's fallback tiles (masks bitwise, outputs within 2e-3),
and the certified decode with its FP16 recompute (certificates and flags
against the oracle).  The device-memory cache on the same inputs gives the
same tier-1 bytes and masks.
Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1
(tiered storage with deterministic fallback) and Methodology 3 (rung 3).
"""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, assert_tier1_equal, gpu_cache, normwise_err, oracle_cache, small, taus_for

pytestmark = pytest.mark.gpu


def host_cache(d, T):
    B, Hkv, cap, _ = d["k16"].shape
    c = kvq.KVCache(B, Hkv, cap, tier2="host")
    c.k16.copy_(d["k16"])
    c.v16.copy_(d["v16"])
    if T:
        kvq.kvq_quantize_append(c, T)
    return c


def test_tier2_location_reports_device_and_host():
    w = small("llama3_8b_32k", B=1, T=128)
    d = workloads.make(w)
    print("[tier2] location query", flush=True)
    assert kvq.kvq_tier2_location(gpu_cache(d, 0)) == 0
    hc = host_cache(d, 0)
    assert kvq.kvq_tier2_location(hc) == 1
    assert kvq.make_workspace(hc, w.Hq).device.type == "cuda"  # the workspace lives with tier 1
    # pageable host memory is refused (a host-side query: nothing runs on the GPU)
    c = host_cache(d, 0)
    c.k16 = torch.zeros_like(c.k16, device="cpu", pin_memory=False)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_tier2_location(c)


@pytest.mark.parametrize("frac", ["cfg", 0.3, 0])
def test_host_tier2_fused_step_matches_oracle(frac):
    w = small("llama3_8b_32k", B=2, T=700)
    d = workloads.make(w)
    f = w.fallback_frac if frac == "cfg" else frac
    print(f"[tier2 host] fused step {w.name} B{w.B} T={w.T} frac={f}", flush=True)
    T0 = w.T - 1
    oc = oracle_cache(d, w.T)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, f)
    c = host_cache(d, T0)
    dc = gpu_cache(d, T0)
    nb = (w.T + 63) // 64
    mh = torch.full((w.B, w.Hkv, nb), 0xEE, dtype=torch.uint8, device="cuda")
    md = torch.full_like(mh, 0xEE)
    out = kvq.kvq_append_decode(c, d["q"].cuda(), SM, tk, tv, mask_out=mh)
    kvq.kvq_append_decode(dc, d["q"].cuda(), SM, tk, tv, mask_out=md)
    torch.cuda.synchronize()
    assert_tier1_equal(c, oc, w.T)
    ref, omask = oc.attention(q, SM, tk, tv)
    np.testing.assert_array_equal(mh.cpu().numpy(), omask)
    np.testing.assert_array_equal(md.cpu().numpy(), omask)
    err = normwise_err(out.float().cpu().numpy(), ref)
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"host tier 2 vs oracle {err.max():.3e}"


def test_host_tier2_certified_recompute():
    w = small("stress_fallback", B=2, T=600)
    d = workloads.make(w)
    print(f"[tier2 host] certified decode {w.name} B{w.B} T={w.T}", flush=True)
    oc = oracle_cache(d, w.T)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, w.fallback_frac)
    ref = oc.certificate(q, SM, tk, tv, -1.0)  # every head recomputed on FP16
    c = host_cache(d, w.T)
    out, cert, rec = kvq.kvq_decode_attn_cert(c, d["q"].cuda(), SM, tk, tv, -1.0)
    torch.cuda.synchronize()
    np.testing.assert_allclose(cert.cpu().numpy().astype(np.float64), ref["cert"], rtol=1e-3, atol=1e-9)
    np.testing.assert_array_equal(rec.cpu().numpy(), ref["recomputed"])
    err = normwise_err(out.float().cpu().numpy(), ref["out"])
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"recompute from host tier 2 {err.max():.3e}"
