"""kvq_decode_attn_adaptive against the oracle: INT8 scoring pass, top-K*
promotion, value promotion, ranking check and rung-3 recompute.

The promotions and the ranking are decisions the GPU takes on fp32 block
masses and the oracle on fp64 ones, so near the boundary either side of a
tie is correct.  The checks therefore bracket the GPU: its masks must lie
between the oracle's masks at tau_cov - DELTA (and tau_vc * (1 + DELTA)) and
at tau_cov + DELTA (tau_vc * (1 - DELTA)), DELTA = 1e-5 in cumulative mass
(fp32 sums of at most a few thousand block masses are good to about 1e-6);
its promoted counts likewise; its discordant-pair counts may differ from the
oracle's by at most the pairs the oracle finds within EPS of a tie, and its
flags must match wherever that margin cannot cross tau_rank.  Every group's
outputs (2e-3) and certificates (1e-3 relative) are then compared with the
oracle evaluated under the GPU's own masks and recompute decisions
(certify_masked), so that no group goes unchecked where the two sides' fp32
and fp64 promotions legitimately differ.  The
planted needle case (an outlier channel the query ignores reorders two
blocks under INT8) must be flagged and recomputed to dense attention.
Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology 3
("Adaptive Top-K Selection", "Ranking-Consistency Check", rungs 1-3).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, assert_tier1_equal, gpu_cache, normwise_err, oracle_cache, small, taus_for

pytestmark = pytest.mark.gpu

INF = float("inf")
DELTA = 1e-5  # cumulative-mass margin of the promotion bracket
EPS = 1e-3    # natural-log margin of a near tie in the ranking check


def _near_ties(a, b, eps):
    n = len(a)
    if n < 2:
        return 0
    da = np.abs(a[:, None] - a[None, :]) < eps
    db = np.abs(b[:, None] - b[None, :]) < eps
    near = np.triu(da | db, 1)
    return int(near.sum())


def _run(name, d, w, T, frac, tau_cov, tau_vc=INF, tau_rank=1.0, tau_out=INF, append=False, exact=False):
    print(f"[adaptive] {name} B{w.B} Hq{w.Hq} T={T} frac={frac} cov={tau_cov} vc={tau_vc} rank={tau_rank} "
          f"out={tau_out} append={append}", flush=True)
    oc = oracle_cache(d, T)
    q = d["q"].numpy()
    tk, tv = taus_for(oc, q, frac) if frac != "inf" else (INF, INF)
    ref = oc.adaptive(q, SM, tk, tv, tau_cov, tau_vc, tau_rank, tau_out)
    lo = oc.adaptive(q, SM, tk, tv, max(tau_cov - DELTA, 0.0) if tau_cov > 0 else 0.0,
                     tau_vc * (1 + DELTA), tau_rank, tau_out)
    hi = oc.adaptive(q, SM, tk, tv, tau_cov + DELTA if tau_cov > 0 else 0.0, tau_vc * (1 - DELTA), tau_rank, tau_out)
    c = gpu_cache(d, T - 1 if append else T)
    nb = (T + 63) // 64
    mask = torch.full((w.B, w.Hkv, nb), 0xEE, dtype=torch.uint8, device="cuda")
    g = kvq.kvq_decode_attn_adaptive(c, d["q"].cuda(), SM, tk, tv, tau_cov, tau_vc, tau_rank, tau_out,
                                     append=append, mask_out=mask)
    torch.cuda.synchronize()
    assert c.length == T
    if append:
        # the scoring pass appended the token: tier 1 as the oracle quantized it
        assert_tier1_equal(c, oc, T)
    m = mask.cpu().numpy()
    # promotions bracketed by the oracle at the nudged tolerances (per bit)
    for bit in (1, 2):
        assert np.all((lo["masks"] & bit) <= (m & bit)), f"bit {bit}: GPU misses a promotion"
        assert np.all((m & bit) <= (hi["masks"] & bit)), f"bit {bit}: GPU promotes too much"
    ks = g["kstar"].cpu().numpy()
    assert np.all(lo["kstar"] <= ks) and np.all(ks <= hi["kstar"])
    same = np.all(m == ref["masks"], axis=-1)  # [B][Hkv]: groups decided alike
    print(f"  groups with the oracle's masks: {same.mean():.3f}", flush=True)
    if exact:
        assert same.all()
    # ranking check where the head promotes the oracle's set
    nd = g["ndisc"].cpu().numpy()
    rec = g["recomputed"].cpu().numpy()
    checked = 0
    for b in range(w.B):
        for h in range(w.Hq):
            kv = h // w.G
            if not same[b, kv] or ks[b, h] != ref["kstar"][b, h]:
                continue
            k = ks[b, h]
            P = np.argsort(-ref["lhat"][b, h], kind="stable")[:k]
            near = _near_ties(ref["lhat"][b, h][P], ref["lfp"][b, h][P], EPS)
            assert abs(int(nd[b, h]) - int(ref["ndisc"][b, h])) <= near, (b, h, nd[b, h], ref["ndisc"][b, h], near)
            npairs = k * (k - 1) // 2
            lo_flag = npairs > 0 and ref["ndisc"][b, h] - near > tau_rank * npairs
            hi_flag = npairs > 0 and ref["ndisc"][b, h] + near > tau_rank * npairs
            if lo_flag == hi_flag and tau_out == INF:
                assert rec[b, h] == int(lo_flag), (b, h)
            checked += 1
    assert checked > 0
    # every group: outputs and certificates against the oracle under the
    # GPU's masks, recomputing exactly the heads the GPU recomputed
    out = g["out"].float().cpu().numpy()
    cert = g["cert"].cpu().numpy().astype(np.float64)
    under = oc.certify_masked(q, SM, m, INF, force=rec)
    err = normwise_err(out, under["out"])
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, (np.unravel_index(err.argmax(), err.shape), err.max())
    np.testing.assert_allclose(cert, under["cert"], rtol=1e-3, atol=1e-9)
    # the certificate rung under those masks: heads clear of tau_out by the
    # certificate's tolerance take the oracle's decision
    if tau_out != INF:
        assert np.all(rec[under["cert"] > tau_out * (1 + 1e-3)] == 1)
    return ref, g


@pytest.mark.parametrize("tau_cov", [0.5, 0.9, 0.995])
def test_adaptive_matches_oracle(tau_cov):
    w = small("llama3_8b_32k", B=2, T=900)
    _run(w.name, workloads.make(w), w, w.T, w.fallback_frac, tau_cov, tau_rank=0.3)


@pytest.mark.parametrize("name,kw,tau_vc", [("single_head", dict(T=1024), INF),
                                            ("stress_fallback", dict(B=2, T=700), 1e-3),
                                            ("llama3_70b_128k", dict(B=1, T=1300), 1e-4),
                                            ("llama3_8b_32k", dict(B=1, Hkv=2, Hq=6, T=1000), INF),    # G = 3
                                            ("llama3_8b_32k", dict(B=1, Hkv=2, Hq=32, T=1000), INF)])  # G = 16
def test_adaptive_group_sizes_and_value_promotion(name, kw, tau_vc):
    w = small(name, **kw)
    _run(name, workloads.make(w), w, w.T, w.fallback_frac, 0.9, tau_vc=tau_vc, tau_rank=0.2)


@pytest.mark.parametrize("T", [777, 641])  # the appended token inside a block / opening one
def test_adaptive_with_append_and_certificate_recompute(T):
    w = small("llama3_8b_32k", B=2, T=T)
    _run(w.name, workloads.make(w), w, w.T, w.fallback_frac, 0.9, tau_rank=0.5, tau_out=5.0, append=True)


def test_zero_coverage_is_the_certified_decode():
    w = small("llama3_8b_32k", B=2, T=600)
    d = workloads.make(w)
    ref, g = _run(w.name, d, w, w.T, w.fallback_frac, 0.0, exact=True)
    assert not g["kstar"].cpu().numpy().any() and not g["ndisc"].cpu().numpy().any()
    c = gpu_cache(d, w.T)
    oc = oracle_cache(d, w.T)
    tk, tv = taus_for(oc, d["q"].numpy(), w.fallback_frac)
    out, cert, _ = kvq.kvq_decode_attn_cert(c, d["q"].cuda(), SM, tk, tv)
    torch.cuda.synchronize()
    assert normwise_err(g["out"].float().cpu().numpy(), out.float().cpu().numpy()).max() <= 2.0 ** -10
    np.testing.assert_allclose(g["cert"].cpu().numpy(), cert.cpu().numpy(), rtol=1e-5)


def test_full_coverage_reads_every_key_as_fp16():
    w = small("stress_fallback", B=1, T=500)
    ref, g = _run(w.name, workloads.make(w), w, w.T, "inf", 1.5)
    assert (ref["masks"] & 1).all()


@pytest.mark.parametrize("outlier", [True, False])
def test_planted_ranking_inconsistency(outlier):
    T = 640
    k16 = np.zeros((1, 1, T, 128), np.float16)
    for blk, tok, k0, k1 in ((2, 5, 9.6, 254.0), (6, 40, 9.9, 508.0), (4, 17, 7.0, 0.0)):
        k16[0, 0, blk * 64 + tok, 0] = k0
        if outlier:
            k16[0, 0, blk * 64 + tok, 1] = k1
    v16 = np.random.default_rng(77).standard_normal((1, 1, T, 128)).astype(np.float16)
    q = np.zeros((1, 1, 128), np.float16)
    q[0, 0, 0] = 10.0
    d = {"k16": torch.from_numpy(k16), "v16": torch.from_numpy(v16), "q": torch.from_numpy(q)}
    w = workloads.WORKLOADS["single_head"].scaled(T=T)
    ref, g = _run("planted needles", d, w, T, "inf", 0.95, tau_rank=0.2, exact=True)
    assert g["kstar"].cpu().numpy()[0, 0] == 3
    nd = int(g["ndisc"].cpu().numpy()[0, 0])
    rec = int(g["recomputed"].cpu().numpy()[0, 0])
    if outlier:
        assert nd == 1 and rec == 1
        dense = oracle_cache(d, T).attention(q, SM, 0.0, 0.0)[0]
        assert normwise_err(g["out"].float().cpu().numpy(), dense).max() <= OUT_TOL
    else:
        assert nd == 0 and rec == 0


def test_empty_cache():
    w = small("llama3_8b_32k", B=2, T=64)
    d = workloads.make(w)
    c = gpu_cache(d, 0)
    print("[adaptive] empty cache", flush=True)
    g = kvq.kvq_decode_attn_adaptive(c, d["q"].cuda(), SM, 1.0, 1.0, 0.9, tau_rank=0.1)
    torch.cuda.synchronize()
    assert not g["out"].float().cpu().numpy().any()
    assert not g["kstar"].cpu().numpy().any() and not g["recomputed"].cpu().numpy().any()
    assert not g["ndisc"].cpu().numpy().any()


@pytest.mark.parametrize("kw,tau_cov,kmin,kmax", [
    (dict(B=1, T=80000), 0.9999, 1025, 2048),                  # up to 8 elements per thread
    (dict(B=1, Hkv=1, Hq=4, T=140000), 1.5, 2049, 1 << 30),   # chunks of 2048 one after another
])
def test_ranking_check_over_many_promoted_blocks(kw, tau_cov, kmin, kmax):
    # heads promoting more than 256 blocks: the discordant pairs are counted
    # by the merge sorts instead of pair by pair
    w = small("llama3_8b_32k", **kw)
    ref, g = _run(w.name, workloads.make(w), w, w.T, w.fallback_frac, tau_cov, tau_rank=0.3)
    ks = g["kstar"].cpu().numpy()
    assert kmin <= ks.max() <= kmax


def test_selection_beyond_the_register_path():
    # more than 2048 blocks per head: the selection keeps its block masses in
    # LDS instead of registers
    w = small("llama3_8b_32k", B=1, Hkv=2, Hq=8, T=140000)
    ref, g = _run(w.name, workloads.make(w), w, w.T, w.fallback_frac, 0.99, tau_rank=0.3)
    assert (w.T + 63) // 64 > 2048 and g["kstar"].cpu().numpy().max() > 0
