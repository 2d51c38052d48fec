"""kvq_cache_reset: a cache filled with one sequence, reset, and filled with
another gives the tier-1 bytes of a fresh cache holding the second sequence
(bitwise, against the oracle), zero statistics past its last block, and the
oracle's masks and outputs (within 2e-3) for the decode and the fused append
+ decode.  Also captured into a graph (the fill is a kernel, not a memset).
Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1
(per-block error annotations of the compressed tier, started over for a new
sequence)."""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, assert_tier1_equal, normwise_err, oracle_cache, small, taus_for

pytestmark = pytest.mark.gpu


def _check_stats_zero_past(c, T):
    nb = (T + 63) // 64
    assert not c.k_err[:, :, nb:].any() and not c.v_err[:, :, nb:].any(), "statistics past the last block"


@pytest.mark.parametrize("T1,T2", [(1500, 300), (300, 1500), (1000, 64), (1000, 65), (129, 1)])
def test_reset_then_append_equals_fresh(T1, T2):
    w = small("llama3_8b_32k", B=2, T=max(T1, T2) + 1)
    print(f"[reset] T1={T1} T2={T2}", flush=True)
    da = workloads.make(w.scaled(seed=11))
    db = workloads.make(w.scaled(seed=12))
    c = kvq.KVCache(w.B, w.Hkv, w.cap, device="cuda", k16=da["k16"].cuda(), v16=da["v16"].cuda())
    kvq.kvq_quantize_append(c, T1)
    torch.cuda.synchronize()
    # the second sequence's originals into the same tier 2, then reset
    c.k16.copy_(db["k16"])
    c.v16.copy_(db["v16"])
    kvq.kvq_cache_reset(c)
    assert c.length == 0
    torch.cuda.synchronize()
    assert not c.k_err.any() and not c.v_err.any()
    kvq.kvq_quantize_append(c, T2 - 1)
    oc = oracle_cache(db, T2)
    q = db["q"].cuda()
    tk, tv = taus_for(oc, db["q"].numpy(), 0.05)
    ref, omask = oc.attention(db["q"].numpy(), SM, tk, tv)
    mask = torch.full((w.B, w.Hkv, (T2 + 63) // 64), 0xEE, dtype=torch.uint8, device="cuda")
    out = kvq.kvq_append_decode(c, q, SM, tk, tv, mask_out=mask)
    torch.cuda.synchronize()
    assert c.length == T2
    assert_tier1_equal(c, oc, T2)
    _check_stats_zero_past(c, T2)
    np.testing.assert_array_equal(mask.cpu().numpy(), omask)
    err = normwise_err(out.float().cpu().numpy(), ref)
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"{err.max():.3e}"


def test_reset_captured_in_graph():
    # reset + bulk append + fused step captured together, replayed on a cache
    # that every replay leaves full
    w = small("llama3_8b_32k", B=2, T=700)
    print("[reset graph]", flush=True)
    d = workloads.make(w.scaled(seed=13))
    oc = oracle_cache(d, w.T)
    tk, tv = taus_for(oc, d["q"].numpy(), 0.05)
    ref, omask = oc.attention(d["q"].numpy(), SM, tk, tv)
    c = kvq.KVCache(w.B, w.Hkv, w.cap, device="cuda", k16=d["k16"].cuda(), v16=d["v16"].cuda())
    q = d["q"].cuda()
    ws = kvq.make_workspace(c, w.Hq)
    out = torch.zeros_like(q)

    def seq(stream):
        kvq.kvq_cache_reset(c, stream)
        kvq.kvq_quantize_append(c, w.T - 1, stream)
        kvq.kvq_append_decode(c, q, SM, tk, tv, out=out, workspace=ws, stream=stream)

    seq(torch.cuda.current_stream())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        seq(torch.cuda.current_stream())
    for rep in range(3):
        c.k_err.fill_(7.0)  # stale statistics that the reset must clear
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        c.length = w.T
        assert_tier1_equal(c, oc, w.T)
        _check_stats_zero_past(c, w.T)
        err = normwise_err(out.float().cpu().numpy(), ref)
        assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"replay {rep}: {err.max():.3e}"
