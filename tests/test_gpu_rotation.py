"""The Hadamard-rotated key codec (KVQ_CODEC_ROTATE_K) on the GPU against the
oracle: tier-1 bytes bitwise (bulk and ragged appends, rows with a large
outlier channel, a non-finite row), masks bitwise and outputs within 2e-3
for the decode, the fused append-and-decode and the certified decode
(certificates within 1e-3), and the adaptive decode bracketed like the plain
codec; the VALU kernel refuses rotated caches.  Codec: the Walsh-Hadamard
transform before scalar quantization of the KQV scheme in "Statistical
Inference and Quality Measures of KV Cache Quantisations Inspired by
TurboQuant" (technical summary, quantisation schemes), read as a rotation of
the keys alone; bounds and fallback as "Runtime-Certified Bounded-Error
Quantized Attention", Methodology 1-3.
"""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, assert_tier1_equal, gpu_cache, normwise_err, oracle_cache, small, taus_for

pytestmark = pytest.mark.gpu


def _planted(w):
    d = workloads.make(w)
    k = d["k16"].clone()
    # a few rows with one very large channel, one row holding Inf
    k[0, 0, 5, 17] = 900.0
    k[0, 0, 70, 3] = -4000.0
    k[-1, -1, 100, 127] = 60000.0
    k[0, 0, 130, 9] = float("inf")
    d["k16"] = k
    return d


@pytest.mark.parametrize("chunks", [None, [1, 63, 64, 5, 300, 67]])
def test_rotated_append_bitwise(chunks):
    w = small("llama3_8b_32k", B=2, T=500)
    d = _planted(w)
    print(f"[rotation] append chunks={chunks}", flush=True)
    c = gpu_cache(d, w.T, append_chunks=chunks, key_rotation=True)
    assert_tier1_equal(c, oracle_cache(d, w.T, key_rotation=True), w.T)


@pytest.mark.parametrize("name,kw", [("llama3_8b_32k", dict(B=2, T=900)), ("llama3_70b_128k", dict(B=1, T=1100)),
                                     ("single_head", dict(T=1000)), ("stress_fallback", dict(B=2, T=600))])
@pytest.mark.parametrize("frac", [0, "cfg", None])
def test_rotated_decode_matches_oracle(name, kw, frac):
    w = small(name, **kw)
    d = workloads.make(w)
    f = w.fallback_frac if frac == "cfg" else frac
    print(f"[rotation] decode {name} T={w.T} frac={f}", flush=True)
    oc = oracle_cache(d, w.T, key_rotation=True)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, f)
    c = gpu_cache(d, w.T, key_rotation=True)
    nb = (w.T + 63) // 64
    mask = torch.full((w.B, w.Hkv, nb), 0xEE, dtype=torch.uint8, device="cuda")
    out = kvq.kvq_decode_attn(c, d["q"].cuda(), SM, tk, tv, mask_out=mask)
    torch.cuda.synchronize()
    ref, omask = oc.attention(q, SM, tk, tv)
    np.testing.assert_array_equal(mask.cpu().numpy(), omask)
    err = normwise_err(out.float().cpu().numpy(), ref)
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"{err.max():.3e}"


@pytest.mark.parametrize("T0", [0, 63, 64, 700])
def test_rotated_fused_step(T0):
    w = small("llama3_8b_32k", B=2, T=T0 + 1)
    d = _planted(w) if T0 >= 200 else workloads.make(w)
    print(f"[rotation] fused step T0={T0}", flush=True)
    oc = oracle_cache(d, T0 + 1, key_rotation=True)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, w.fallback_frac)
    c = gpu_cache(d, T0, key_rotation=True)
    out = kvq.kvq_append_decode(c, d["q"].cuda(), SM, tk, tv)
    torch.cuda.synchronize()
    assert_tier1_equal(c, oc, T0 + 1)
    ref, _ = oc.attention(q, SM, tk, tv)
    got = out.float().cpu().numpy()
    # heads of the group holding the Inf key row are NaN in both (dense semantics)
    bad = ~np.isfinite(ref).all(axis=-1)
    np.testing.assert_array_equal(~np.isfinite(got).all(axis=-1), bad)
    err = normwise_err(got[~bad], ref[~bad])
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"{err.max():.3e}"


@pytest.mark.parametrize("tau_out", [float("inf"), -1.0])
def test_rotated_certificate(tau_out):
    w = small("llama3_8b_32k", B=2, T=800)
    d = workloads.make(w)
    print(f"[rotation] certificate tau_out={tau_out}", flush=True)
    oc = oracle_cache(d, w.T, key_rotation=True)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, w.fallback_frac)
    ref = oc.certificate(q, SM, tk, tv, tau_out)
    c = gpu_cache(d, w.T, key_rotation=True)
    out, cert, rec = kvq.kvq_decode_attn_cert(c, d["q"].cuda(), SM, tk, tv, tau_out)
    torch.cuda.synchronize()
    np.testing.assert_allclose(cert.cpu().numpy().astype(np.float64), ref["cert"], rtol=1e-3, atol=1e-9)
    np.testing.assert_array_equal(rec.cpu().numpy(), ref["recomputed"])
    err = normwise_err(out.float().cpu().numpy(), ref["out"])
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"{err.max():.3e}"


@pytest.mark.parametrize("append", [False, True])
def test_rotated_adaptive_bracketed(append):
    w = small("llama3_8b_32k_niah", B=2, T=900)
    d = workloads.make(w)
    print(f"[rotation] adaptive append={append}", flush=True)
    oc = oracle_cache(d, w.T, key_rotation=True)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, w.fallback_frac)
    lo = oc.adaptive(q, SM, tk, tv, 0.995 - 1e-5, tau_rank=0.3)
    hi = oc.adaptive(q, SM, tk, tv, 0.995 + 1e-5, tau_rank=0.3)
    ref = oc.adaptive(q, SM, tk, tv, 0.995, tau_rank=0.3)
    c = gpu_cache(d, w.T - 1 if append else w.T, key_rotation=True)
    nb = (w.T + 63) // 64
    mask = torch.full((w.B, w.Hkv, nb), 0xEE, dtype=torch.uint8, device="cuda")
    g = kvq.kvq_decode_attn_adaptive(c, d["q"].cuda(), SM, tk, tv, 0.995, tau_rank=0.3, mask_out=mask,
                                     append=append)
    torch.cuda.synchronize()
    assert c.length == w.T
    if append:
        assert_tier1_equal(c, oc, w.T)
    m = mask.cpu().numpy()
    assert np.all((lo["masks"] & 1) <= (m & 1)) and np.all((m & 1) <= (hi["masks"] & 1))
    # every group against the oracle under the GPU's masks and recompute
    # decisions (fp32 and fp64 promotions may legitimately differ at ties)
    out = g["out"].float().cpu().numpy()
    rec = g["recomputed"].cpu().numpy()
    under = oc.certify_masked(q, SM, m, float("inf"), force=rec)
    err = normwise_err(out, under["out"])
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"{err.max():.3e}"
    np.testing.assert_allclose(g["cert"].cpu().numpy().astype(np.float64), under["cert"], rtol=1e-3, atol=1e-9)


def test_valu_kernel_refuses_rotated_cache():
    w = small("llama3_8b_32k", B=1, T=128)
    d = workloads.make(w)
    c = gpu_cache(d, w.T, key_rotation=True)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_decode_attn(c, d["q"].cuda(), SM, 1.0, 1.0, kernel=kvq.KERNEL_VALU)


def test_rotation_cuts_key_fallback_at_fixed_tau():
    w = small("llama3_8b_32k", B=2, T=2048)
    d = workloads.make(w)
    print("[rotation] fallback share at a fixed tau", flush=True)
    plain = gpu_cache(d, w.T)
    rot = gpu_cache(d, w.T, key_rotation=True)
    q = d["q"].cuda()
    kb, _, _ = kvq.kvq_bounds(plain, q, SM, 0.0, 0.0, want=("kb",))
    tk = float(np.quantile(kb.cpu().numpy(), 0.95))
    _, _, mp = kvq.kvq_bounds(plain, q, SM, tk, float("inf"), want=("mask",))
    _, _, mr = kvq.kvq_bounds(rot, q, SM, tk, float("inf"), want=("mask",))
    torch.cuda.synchronize()
    assert (mr.cpu().numpy() & 1).mean() < 0.5 * (mp.cpu().numpy() & 1).mean()
