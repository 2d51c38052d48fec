"""Pins for the oracle's adaptive precision: the INT8 scoring pass, top-K*
coverage promotion (rung 1), value promotion (rung 2), the ranking-
consistency check and the recompute of inconsistent heads (rung 3).  CPU only.

Method: "Runtime-Certified Bounded-Error Quantized Attention", technical
summary, Methodology 3 ("Adaptive Top-K Selection", "Ranking-Consistency
Check", the four-rung fallback ladder) and Key Contributions ("Adaptive
Precision", "Ranking-Consistency Check").  What pins it:
  - the block log-masses equal scipy's logsumexp over the dequantized (and
    the FP16) logits of each block;
  - the promoted set of a head is the smallest set of blocks covering tau_cov
    of the INT8 mass, found by enumerating every subset on a 10-block cache;
  - the discordant share equals (1 - Kendall's tau) / 2 from scipy;
  - special cases: tau_cov = 0 and tau_vc = inf give the plain decode;
    tau_cov = 1 puts every key block on FP16 (SDPA over the FP16 keys);
    tau_vc = 0 promotes every value block with a nonzero error;
  - a planted case whose INT8 scores reorder two needle blocks (an outlier
    channel the query ignores coarsens their scales) is flagged
    inconsistent and recomputed to dense attention; the same needles without
    the outlier are consistent;
  - promotions grow with tau_cov, and the certificate still bounds the dense
    error under the adaptive masks.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle
import workloads

SM = float(np.float32(1 / math.sqrt(128)))
INF = float("inf")


def case(name, **kw):
    w = workloads.WORKLOADS[name].scaled(**kw)
    d = workloads.make(w, "cpu")
    return w, d["q"].numpy(), d["k16"].numpy(), d["v16"].numpy()


def sdpa64(q, k, v, G, T):
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, :, None, :]
    kt = torch.from_numpy(np.asarray(k[:, :, :T], np.float64)).repeat_interleave(G, dim=1).contiguous()
    vt = torch.from_numpy(np.asarray(v[:, :, :T], np.float64)).repeat_interleave(G, dim=1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SM)
    return o[:, :, 0, :].numpy()


def dequant(cache):
    k = cache.k_codes.astype(np.float64) * cache.k_scales.astype(np.float64)[..., None]
    vc = cache.v_codes_unpacked().astype(np.float64)
    vs = np.repeat(cache.v_scales.astype(np.float64), 32, axis=-1)
    return k, vc * vs


def top_set(lhat_row, k):
    return np.argsort(-lhat_row, kind="stable")[:k]


# ---------------------------------------------------------- scoring pass

@pytest.mark.parametrize("name,kw", [("llama3_8b_32k", dict(B=2, T=700)), ("single_head", dict(T=1000))])
def test_block_logmass_is_a_block_logsumexp(name, kw):
    w, q, k16, v16 = case(name, **kw)
    c = oracle.Cache(k16, v16, w.T)
    r = c.adaptive(q, SM, INF, INF, 0.5)
    khat, _ = dequant(c)
    nb = c.nblocks
    for b in range(w.B):
        for h in range(w.Hq):
            kv = h // w.G
            for keys, got in ((khat, r["lhat"]), (k16.astype(np.float64), r["lfp"])):
                lg = SM * keys[b, kv, :w.T] @ q[b, h].astype(np.float64)
                lg = np.concatenate([lg, np.full(nb * 64 - w.T, -np.inf)]).reshape(nb, 64)
                np.testing.assert_allclose(got[b, h], scipy.special.logsumexp(lg, axis=1), rtol=0, atol=1e-11)


# ---------------------------------------------------------------- rung 1

@pytest.mark.parametrize("tau_cov", [0.2, 0.5, 0.8, 0.95, 0.999])
def test_promoted_set_is_the_smallest_cover(tau_cov):
    # 10 blocks, one head: enumerate every subset
    w, q, k16, v16 = case("single_head", T=640)
    c = oracle.Cache(k16, v16, w.T)
    r = c.adaptive(q, SM, INF, INF, tau_cov)
    lh = r["lhat"][0, 0]
    m = np.exp(lh - scipy.special.logsumexp(lh))
    nb = m.size
    assert nb == 10 and len(set(m.tolist())) == nb  # no ties
    best = None
    for k in range(1, nb + 1):
        sets = [(sum(m[list(s)]), s) for s in itertools.combinations(range(nb), k)]
        cover = [x for x in sets if x[0] >= tau_cov]
        if cover:
            best = set(max(cover)[1])
            break
    promoted = set(np.nonzero(r["masks"][0, 0] & 1)[0].tolist())
    assert r["kstar"][0, 0] == len(best)
    assert promoted == best


def test_zero_coverage_is_the_plain_decode():
    w, q, k16, v16 = case("llama3_8b_32k", B=2, T=900)
    c = oracle.Cache(k16, v16, w.T)
    kb, vb, _ = c.bounds(q, SM, 0.0, 0.0)
    tk, tv = oracle.tau_for_fraction(kb, 0.05), oracle.tau_for_fraction(vb, 0.05)
    r = c.adaptive(q, SM, tk, tv, 0.0)
    out, mask = c.attention(q, SM, tk, tv)
    np.testing.assert_array_equal(r["masks"], mask)
    np.testing.assert_allclose(r["out"], out, rtol=0, atol=1e-12)
    assert not r["kstar"].any() and not r["inconsistent"].any() and not r["npairs"].any()
    ref = c.certificate(q, SM, tk, tv)
    np.testing.assert_allclose(r["cert"], ref["cert"], rtol=1e-14, atol=0)


def test_full_coverage_puts_every_key_on_fp16():
    w, q, k16, v16 = case("stress_fallback", B=1, T=600)
    c = oracle.Cache(k16, v16, w.T)
    _, vb, _ = c.bounds(q, SM, 0.0, 0.0)
    tv = oracle.tau_for_fraction(vb, 0.2)
    r = c.adaptive(q, SM, INF, tv, 1.0)
    assert (r["masks"] & 1).all()
    _, vhat = dequant(c)
    vmix = vhat.copy()
    for h in range(w.Hkv):
        for blk in range(c.nblocks):
            if r["masks"][0, h, blk] & 2:
                vmix[0, h, blk * 64:blk * 64 + 64] = v16[0, h, blk * 64:blk * 64 + 64]
    ref = sdpa64(q, k16, vmix, w.G, w.T)
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)


def test_promotions_grow_with_coverage():
    w, q, k16, v16 = case("llama3_8b_32k", B=1, T=2000)
    c = oracle.Cache(k16, v16, w.T)
    prev = None
    for tau_cov in (0.1, 0.5, 0.9, 0.99, 0.999):
        r = c.adaptive(q, SM, INF, INF, tau_cov)
        if prev is not None:
            assert np.all(r["kstar"] >= prev["kstar"])
            assert np.all((r["masks"] & 1) >= (prev["masks"] & 1))
        prev = r


# ---------------------------------------------------------------- rung 2

def test_value_promotion_extremes():
    w, q, k16, v16 = case("llama3_8b_32k", B=1, T=900)
    c = oracle.Cache(k16, v16, w.T)
    r_inf = c.adaptive(q, SM, INF, INF, 0.0, tau_vc=INF)
    assert not (r_inf["masks"] & 2).any()
    r0 = c.adaptive(q, SM, INF, INF, 0.0, tau_vc=0.0)
    nb = c.nblocks
    has_err = c.v_err[:, :, :nb] > 0
    np.testing.assert_array_equal((r0["masks"] & 2) != 0, has_err)
    prev = 0
    for tau_vc in (1e-2, 1e-3, 1e-4, 1e-5):
        n = int((c.adaptive(q, SM, INF, INF, 0.0, tau_vc=tau_vc)["masks"] & 2).sum())
        assert n >= prev
        prev = n


# -------------------------------------------------------- ranking check

def test_discordant_share_is_kendall_tau():
    w, q, k16, v16 = case("llama3_8b_32k", B=1, T=1500)
    c = oracle.Cache(k16, v16, w.T)
    r = c.adaptive(q, SM, INF, INF, 0.9)
    checked = 0
    for h in range(w.Hq):
        k = r["kstar"][0, h]
        P = top_set(r["lhat"][0, h], k)
        assert r["npairs"][0, h] == k * (k - 1) // 2
        if k < 2:
            continue
        a, b = r["lhat"][0, h][P], r["lfp"][0, h][P]
        assert len(set(a.tolist())) == k and len(set(b.tolist())) == k
        tau = scipy.stats.kendalltau(a, b).statistic
        assert r["ndisc"][0, h] / r["npairs"][0, h] == pytest.approx((1 - tau) / 2, abs=1e-12)
        checked += 1
    assert checked > 0


def planted_needles(outlier):
    """One head, 10 blocks, q = 10 e_0.  Needle keys with k_0 = 9.6, 9.9 and
    7.0 in blocks 2, 6 and 4; the rest of the keys are 0.  With `outlier`,
    the first two needles also hold 254 and 508 in channel 1, which the query
    ignores: their INT8 scales become 2 and 4, so the INT8 k_0 are 10 and 8
    and the two blocks change places in the INT8 ranking."""
    T = 640
    k16 = np.zeros((1, 1, T, 128), np.float16)
    for blk, tok, k0, k1 in ((2, 5, 9.6, 254.0), (6, 40, 9.9, 508.0), (4, 17, 7.0, 0.0)):
        k16[0, 0, blk * 64 + tok, 0] = k0
        if outlier:
            k16[0, 0, blk * 64 + tok, 1] = k1
    v16 = np.random.default_rng(77).standard_normal((1, 1, T, 128)).astype(np.float16)
    q = np.zeros((1, 1, 128), np.float16)
    q[0, 0, 0] = 10.0
    return q, k16, v16, T


@pytest.mark.parametrize("outlier", [True, False])
def test_planted_ranking_inconsistency(outlier):
    q, k16, v16, T = planted_needles(outlier)
    c = oracle.Cache(k16, v16, T)
    r = c.adaptive(q, SM, INF, INF, 0.95, tau_rank=0.2)
    assert r["kstar"][0, 0] == 3
    assert set(np.nonzero(r["masks"][0, 0] & 1)[0].tolist()) == {2, 4, 6}
    assert r["npairs"][0, 0] == 3
    if outlier:
        # FP16 ranks block 6 over block 2, INT8 the reverse: one of three pairs
        assert r["ndisc"][0, 0] == 1 and r["inconsistent"][0, 0] == 1 and r["recomputed"][0, 0] == 1
        ref = sdpa64(q, k16, v16, 1, T)
        np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)
    else:
        assert r["ndisc"][0, 0] == 0 and r["inconsistent"][0, 0] == 0 and r["recomputed"][0, 0] == 0
    # a tolerance at or above the discordant share never flags
    r1 = c.adaptive(q, SM, INF, INF, 0.95, tau_rank=1.0 / 3.0)
    assert r1["inconsistent"][0, 0] == 0


# ------------------------------------------------- certificate under promotion

@pytest.mark.parametrize("name,kw", [("llama3_8b_32k", dict(B=1, T=900)), ("stress_fallback", dict(B=1, T=700))])
def test_certificate_bounds_dense_error_under_promotion(name, kw):
    w, q, k16, v16 = case(name, **kw)
    c = oracle.Cache(k16, v16, w.T)
    kb, vb, _ = c.bounds(q, SM, 0.0, 0.0)
    tk, tv = oracle.tau_for_fraction(kb, 0.02), oracle.tau_for_fraction(vb, 0.02)
    r = c.adaptive(q, SM, tk, tv, 0.9, tau_vc=1e-3)
    dense = sdpa64(q, k16, v16, w.G, w.T)
    err = np.max(np.abs(r["out"] - dense), axis=-1)
    assert np.all(err <= r["cert"] * (1 + 1e-9) + 1e-12)
