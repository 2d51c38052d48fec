"""kvq_append_decode_noalloc (the decode step with its split partials in the
library's static device scratch, for callers that cannot allocate) against
kvq_append_decode with a workspace, through the C ABI, and against the
oracle: tier-1 bytes and masks bitwise, outputs within 2e-3 of the oracle
and within fp16 rounding of the workspace path.  Two calls in a row, the
second on a smaller cache, share the scratch."""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, assert_tier1_equal, gpu_cache, normwise_err, oracle_cache, small, taus_for

pytestmark = pytest.mark.gpu


def _step(name, kw):
    w = small(name, **kw)
    print(f"[noalloc] {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} T{w.T}", flush=True)
    d = workloads.make(w)
    T0 = w.T - 1
    oc = oracle_cache(d, w.T)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, w.fallback_frac or 0.05)
    A = gpu_cache(d, T0)
    Bc = gpu_cache(d, T0)
    nb = (w.T + 63) // 64
    ma = torch.full((w.B, w.Hkv, nb), 0xEE, dtype=torch.uint8, device="cuda")
    mb = torch.full_like(ma, 0xEE)
    qd = d["q"].cuda()
    out_a = torch.empty_like(qd)
    out_b = torch.full_like(qd, float("nan"))
    kvq.kvq_append_decode(A, qd, SM, tk, tv, out=out_a, mask_out=ma)
    kvq.kvq_append_decode_noalloc(Bc, qd, SM, tk, tv, out=out_b, mask_out=mb)
    torch.cuda.synchronize()
    assert A.length == w.T and Bc.length == w.T
    assert_tier1_equal(Bc, oc, w.T)
    ref, omask = oc.attention(q, SM, tk, tv)
    np.testing.assert_array_equal(mb.cpu().numpy(), omask)
    np.testing.assert_array_equal(ma.cpu().numpy(), omask)
    ob = out_b.float().cpu().numpy()
    err = normwise_err(ob, ref)
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"noalloc vs oracle {err.max():.3e}"
    assert normwise_err(ob, out_a.float().cpu().numpy()).max() <= 2.0 ** -10


def test_noalloc_two_calls_second_smaller():
    _step("llama3_8b_32k", dict(B=4, T=3000))
    _step("stress_fallback", dict(B=1, T=500))


def test_noalloc_rejects_partials_beyond_the_scratch():
    # 1024 (batch, KV head) groups of 16 query heads: one split each already
    # needs 1024 * 16 * 524 bytes, more than KVQ_SCRATCH_BYTES
    B, Hkv, G, cap = 128, 8, 16, 64
    k16 = torch.zeros((B, Hkv, cap, 128), dtype=torch.float16, device="cuda")
    c = kvq.KVCache(B, Hkv, cap, device="cuda", k16=k16, v16=torch.zeros_like(k16))
    kvq.kvq_quantize_append(c, 10)
    q = torch.zeros((B, Hkv * G, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append_decode_noalloc(c, q, SM, 0.0, 0.0, out=torch.empty_like(q))
    assert e.value.status == -5
    assert c.length == 10  # nothing was enqueued
