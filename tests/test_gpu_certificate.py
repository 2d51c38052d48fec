"""kvq_decode_attn_cert against the oracle: per-head certificates (relative
1e-3: the decode accumulates the attention masses in fp32, the oracle in
fp64), recompute flags (bitwise, with tau_out set where no certificate is
near it), masks (bitwise) and outputs (within 2e-3; dense for recomputed
heads), with and without the fused append, across group sizes and fallback
regimes.
Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology 2
(two-term error decomposition) and Methodology 3 (rung 3, per-head FP16
recompute).
"""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, gpu_cache, normwise_err, oracle_cache, small, taus_for

pytestmark = pytest.mark.gpu

CERT_RTOL = 1e-3


def _tau_out_between(cert):
    """A tolerance in the widest relative gap of the middle of the sorted
    certificates, so that no certificate sits near it."""
    c = np.sort(np.asarray(cert, np.float64).ravel())
    n = len(c)
    lo, hi = n // 4, max(n // 4 + 1, 3 * n // 4)
    gaps = [(c[i + 1] / max(c[i], 1e-30), i) for i in range(lo, min(hi, n - 1))]
    r, i = max(gaps)
    assert r > 1 + 4 * CERT_RTOL, "no usable gap between certificates"
    return float(np.sqrt(c[i] * c[i + 1]))


def _check(w, d, T, frac, tau_out, append):
    print(f"[cert] {w.name} B{w.B} Hq{w.Hq} T={T} frac={frac} tau_out={tau_out} append={append}", flush=True)
    oc = oracle_cache(d, T)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, frac)
    base = oc.certificate(q, SM, tk, tv)
    if tau_out == "between":
        tau_out = _tau_out_between(base["cert"])
    ref = oc.certificate(q, SM, tk, tv, tau_out)
    c = gpu_cache(d, T - 1 if append else T)
    nb = (T + 63) // 64
    mask = torch.full((w.B, w.Hkv, nb), 0xEE, dtype=torch.uint8, device="cuda")
    out, cert, rec = kvq.kvq_decode_attn_cert(c, d["q"].cuda(), SM, tk, tv, tau_out, append=append, mask_out=mask)
    torch.cuda.synchronize()
    assert c.length == T
    _, _, omask = oc.bounds(q, SM, tk, tv)
    np.testing.assert_array_equal(mask.cpu().numpy(), omask)
    cg = cert.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(cg, ref["cert"], rtol=CERT_RTOL, atol=1e-9)
    np.testing.assert_array_equal(rec.cpu().numpy(), ref["recomputed"])
    err = normwise_err(out.float().cpu().numpy(), ref["out"])
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"output vs oracle {err.max():.3e}"
    return ref


@pytest.mark.parametrize("name,kw", [("llama3_8b_32k", dict(B=2, T=900)), ("llama3_70b_128k", dict(B=1, T=1100)),
                                     ("stress_fallback", dict(B=2, T=700)), ("single_head", dict(T=1024))])
@pytest.mark.parametrize("frac", [0.02, 0.3, None])
def test_certificate_matches_oracle(name, kw, frac):
    w = small(name, **kw)
    _check(w, workloads.make(w), w.T, frac, float("inf"), False)


@pytest.mark.parametrize("name,kw", [("llama3_8b_32k", dict(B=2, T=900)), ("llama3_70b_128k", dict(B=1, T=1100)),
                                     ("stress_fallback", dict(B=2, T=700))])
def test_recompute_of_flagged_heads(name, kw):
    w = small(name, **kw)
    ref = _check(w, workloads.make(w), w.T, 0.02, "between", False)
    assert 0 < ref["recomputed"].sum() < ref["recomputed"].size


def test_every_head_recomputed():
    w = small("llama3_8b_32k", B=2, T=500)
    ref = _check(w, workloads.make(w), w.T, 0.05, -1.0, False)
    assert ref["recomputed"].all()


@pytest.mark.parametrize("T0", [0, 63, 64, 200])
def test_certificate_with_fused_append(T0):
    w = small("llama3_8b_32k", B=2, T=T0 + 1)
    _check(w, workloads.make(w), T0 + 1, 0.05, "between" if T0 >= 63 else float("inf"), True)


def test_certificate_replays_are_stable():
    """Two certified calls on the same cache: same certificates, flags and
    outputs up to fp16 rounding of the output."""
    w = small("llama3_8b_32k", B=2, T=600)
    d = workloads.make(w)
    c = gpu_cache(d, w.T)
    q = d["q"].cuda()
    o1, c1, r1 = kvq.kvq_decode_attn_cert(c, q, SM, 1.0, 0.2, 3.0)
    o2, c2, r2 = kvq.kvq_decode_attn_cert(c, q, SM, 1.0, 0.2, 3.0)
    torch.cuda.synchronize()
    np.testing.assert_allclose(c1.cpu().numpy(), c2.cpu().numpy(), rtol=1e-5)
    np.testing.assert_array_equal(r1.cpu().numpy(), r2.cpu().numpy())
    assert normwise_err(o1.float().cpu().numpy(), o2.float().cpu().numpy()).max() <= 2.0 ** -10
