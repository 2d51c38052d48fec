"""kvq_append_decode (one launch per decode step: quantize-on-append of the
new token inside the matrix-core decode kernel) against the two-call
sequence kvq_quantize_append(1) + kvq_decode_attn and against the oracle:
tier-1 bytes, block statistics and masks bitwise, outputs within 2e-3 of the
oracle and within fp16 rounding of the two-call result.  The new token sits
at every kind of position in its block (first, second, odd, even, last of a
half, last of the block), in certified and in fallback blocks (planted
spikes make its own block fall back on K, V or both).
Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1-2.
"""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, assert_tier1_equal, gpu_cache, normwise_err, oracle_cache, small, taus_for

pytestmark = pytest.mark.gpu


def _run(w, d, T0, frac, kernel=kvq.KERNEL_AUTO):
    print(f"[fused] {w.name} B{w.B} Hq{w.Hq} T0={T0} frac={frac} kernel={kernel}", flush=True)
    T1 = T0 + 1
    A = gpu_cache(d, T0)
    Bc = gpu_cache(d, T0)
    oc = oracle_cache(d, T1)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, frac)
    nb = (T1 + 63) // 64
    ma = torch.full((w.B, w.Hkv, nb), 0xEE, dtype=torch.uint8, device="cuda")
    mb = torch.full_like(ma, 0xEE)
    qd = d["q"].cuda()
    out_a = kvq.kvq_append_decode(A, qd, SM, tk, tv, mask_out=ma, kernel=kernel)
    kvq.kvq_quantize_append(Bc, 1)
    out_b = kvq.kvq_decode_attn(Bc, qd, SM, tk, tv, mask_out=mb, kernel=kernel)
    torch.cuda.synchronize()
    assert A.length == T1 and Bc.length == T1
    assert_tier1_equal(A, oc, T1)
    assert_tier1_equal(Bc, oc, T1)
    ref, omask = oc.attention(q, SM, tk, tv)
    np.testing.assert_array_equal(ma.cpu().numpy(), omask)
    np.testing.assert_array_equal(mb.cpu().numpy(), omask)
    err = normwise_err(out_a.float().cpu().numpy(), ref)
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"fused vs oracle {err.max():.3e}"
    assert normwise_err(out_a.float().cpu().numpy(), out_b.float().cpu().numpy()).max() <= 2.0 ** -10
    return omask


@pytest.mark.parametrize("T0", [0, 1, 2, 31, 32, 63, 64, 65, 95, 126, 127, 2000])
@pytest.mark.parametrize("frac", [0, "cfg", None])
def test_fused_step_positions(T0, frac):
    w = small("llama3_8b_32k", B=2, T=T0 + 1)
    f = w.fallback_frac if frac == "cfg" else frac
    _run(w, workloads.make(w), T0, f)


@pytest.mark.parametrize("spike", ["k", "v", "kv"])
@pytest.mark.parametrize("T0", [64, 97, 190])
def test_fused_step_new_token_falls_back(spike, T0):
    # a spike in the new token's own rows makes its block's bound exceed tau
    w = small("llama3_8b_32k", B=2, T=T0 + 1)
    d = workloads.make(w)
    if "k" in spike:
        d["k16"][:, :, T0, 5] = 3000.0
    if "v" in spike:
        d["v16"][:, :, T0, 77] = -3000.0
    m = _run(w, d, T0, 0.5)
    assert np.all(m[:, :, T0 // 64] & (1 if "k" in spike else 2))


@pytest.mark.parametrize("name,kw", [("llama3_70b_128k", dict(B=1, T=700)), ("single_head", dict(T=300)),
                                     ("stress_fallback", dict(B=2, T=500))])
def test_fused_step_group_sizes(name, kw):
    w = small(name, **kw)
    _run(w, workloads.make(w), w.T - 1, w.fallback_frac)


def test_fused_step_valu_kernel_appends_separately():
    w = small("llama3_8b_32k", B=2, T=300)
    _run(w, workloads.make(w), w.T - 1, w.fallback_frac, kernel=kvq.KERNEL_VALU)


def test_fused_step_capacity():
    w = small("llama3_8b_32k", B=1, T=128)
    d = workloads.make(w)
    c = gpu_cache(d, 128)  # full: capacity 128
    with pytest.raises(kvq.KvqError):
        kvq.kvq_append_decode(c, d["q"].cuda(), SM, 0.0, 0.0)
    assert c.length == 128
