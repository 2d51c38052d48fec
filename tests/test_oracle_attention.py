"""Pins for the oracle's bounds, fallback masks and fp64 attention (CPU only).

They check what the mathematics fixes, independently of the oracle's own
code: the Cauchy-Schwarz key bound really bounds the logit perturbation
(tight for a query parallel to the error), the value bound equals the
observed error, tau = 0 reproduces dense attention (torch SDPA in fp64),
tau = +inf is plain quantized attention, and closed forms for T = 1, q = 0 and
identical tokens.  Method: "Runtime-Certified Bounded-Error Quantized
Attention", Methodology 2 (key term from the per-token score perturbation,
value term from per-block reconstruction error, computed online from scales
and query norms) and Key Contributions ("Deterministic Recovery": fallback to
the exact dense output).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

SM = float(np.float32(1 / math.sqrt(128)))


def small_case(name="stress_fallback", **kw):
    w = workloads.WORKLOADS[name].scaled(**kw)
    d = workloads.make(w, "cpu")
    return w, d["q"].numpy(), d["k16"].numpy(), d["v16"].numpy()


def dequant(cache):
    k = cache.k_codes.astype(np.float64) * cache.k_scales.astype(np.float64)[..., None]
    vc = cache.v_codes_unpacked().astype(np.float64)
    vs = np.repeat(cache.v_scales.astype(np.float64), 32, axis=-1)
    return k, vc * vs


def sdpa64(q, k, v, G, T):
    """Reference dense attention: torch SDPA in fp64 on the CPU."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, :, None, :]        # [B,Hq,1,D]
    kt = torch.from_numpy(np.asarray(k[:, :, :T], np.float64))
    vt = torch.from_numpy(np.asarray(v[:, :, :T], np.float64))
    kt = kt.repeat_interleave(G, dim=1).contiguous()
    vt = vt.repeat_interleave(G, dim=1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SM)
    return o[:, :, 0, :].numpy()


def normwise(a, ref):
    den = np.max(np.abs(ref), axis=-1)
    return np.max(np.abs(a - ref), axis=-1) / np.where(den == 0, 1, den)


# ------------------------------------------------------------ bounds

def test_key_bound_dominates_observed_logit_error():
    w, q, k16, v16 = small_case(B=2, T=640)
    cache = oracle.Cache(k16, v16, w.T)
    kb, vb, _ = cache.bounds(q, SM, 0.0, 0.0)
    khat, vhat = dequant(cache)
    worst_ratio = 0.0
    for b in range(w.B):
        for hq in range(w.Hq):
            h = hq // w.G
            qv = q[b, hq].astype(np.float64)
            for blk in range(cache.nblocks):
                t0, t1 = blk * 64, min(w.T, blk * 64 + 64)
                e = k16[b, h, t0:t1].astype(np.float64) - khat[b, h, t0:t1]
                obs = SM * np.max(np.abs(e @ qv))
                assert obs <= kb[b, h, blk]
                if kb[b, h, blk] > 0:
                    worst_ratio = max(worst_ratio, obs / kb[b, h, blk])
                # value bound is exactly the observed max error of the block
                ev = np.max(np.abs(v16[b, h, t0:t1].astype(np.float64) - vhat[b, h, t0:t1]))
                assert vb[b, h, blk] == np.float32(ev)
    assert 0 < worst_ratio < 1


def test_key_bound_is_tight_for_parallel_query():
    rng = np.random.default_rng(2)
    k16 = np.zeros((1, 1, 64, 128), np.float16)
    k16[0, 0, :64] = rng.standard_normal((64, 128)).astype(np.float16)
    v16 = np.zeros_like(k16)
    cache = oracle.Cache(k16, v16, 64)
    khat, _ = dequant(cache)
    e = k16[0, 0].astype(np.float64) - khat[0, 0]
    t = int(np.argmax(np.linalg.norm(e, axis=1)))
    q = (e[t] / np.max(np.abs(e[t])) * 8).astype(np.float16)[None, None, :]
    kb, _, _ = cache.bounds(q, SM, 0.0, 0.0)
    # exact logit perturbation with rationals
    obs = abs(sum(Fraction(float(a)) * (Fraction(float(x)) - Fraction(float(k))) for a, x, k in
                  zip(q[0, 0], k16[0, 0, t], khat[0, 0, t]))) * Fraction(SM)
    ratio = float(obs) / float(kb[0, 0, 0])
    assert 1 - 2 ** -15 <= ratio <= 1


def test_key_bound_arithmetic_matches_hand_value():
    # ((sm*qn)*kerr)*(1+2^-16) with exactly representable operands
    assert oracle.key_bound(0.5, 4.0, 0.25) == 0.5 * (1 + 2 ** -16)
    assert oracle.key_bound(1.0, 0.0, np.inf) != oracle.key_bound(1.0, 0.0, np.inf)  # NaN


def test_group_query_norm_is_max_over_the_group():
    w, q, k16, v16 = small_case(B=1, T=64)
    cache = oracle.Cache(k16, v16, 64)
    kb, _, _ = cache.bounds(q, SM, 0.0, 0.0)
    for h in range(w.Hkv):
        qn = max(oracle.qnorm(q[0, h * w.G + g]) for g in range(w.G))
        assert kb[0, h, 0] == np.float32(np.float32(np.float32(SM * qn) * cache.k_err[0, h, 0]) *
                                         np.float32(1 + 2 ** -16))


def test_masks_are_monotone_in_tau():
    w, q, k16, v16 = small_case(B=2, T=1000)
    cache = oracle.Cache(k16, v16, w.T)
    kb, vb, _ = cache.bounds(q, SM, 0.0, 0.0)
    taus = np.quantile(kb, [0.0, 0.2, 0.5, 0.9, 0.99, 1.0])
    prev = None
    for t in taus:
        _, _, m = cache.bounds(q, SM, float(t), float(t))
        if prev is not None:
            assert np.all((m & ~prev) == 0)  # a larger tolerance never adds a fallback
        prev = m
    _, _, m = cache.bounds(q, SM, np.inf, np.inf)
    assert not m.any()
    _, _, m = cache.bounds(q, SM, 0.0, 0.0)
    assert np.array_equal(m & 1, (kb > 0).astype(np.uint8)) and np.array_equal(m >> 1, (vb > 0).astype(np.uint8))


# ------------------------------------------------------------ attention special cases

@pytest.mark.parametrize("name,T", [("single_head", 1000), ("stress_fallback", 333), ("llama3_8b_32k", 129)])
def test_tau_zero_is_dense_attention(name, T):
    kw = dict(T=T) if name == "single_head" else dict(T=T, B=2)
    w, q, k16, v16 = small_case(name, **kw)
    cache = oracle.Cache(k16, v16, w.T)
    out, mask = cache.attention(q, SM, 0.0, 0.0)
    ref = sdpa64(q, k16, v16, w.G, w.T)
    assert np.max(normwise(out, ref)) <= 1e-12


def test_tau_inf_is_plain_quantized_attention():
    w, q, k16, v16 = small_case(B=2, T=700)
    cache = oracle.Cache(k16, v16, w.T)
    out, mask = cache.attention(q, SM, np.inf, np.inf)
    assert not mask.any()
    khat, vhat = dequant(cache)
    ref = sdpa64(q, khat, vhat, w.G, w.T)
    assert np.max(normwise(out, ref)) <= 1e-12
    # and the quantized output is measurably different from dense
    dense = sdpa64(q, k16, v16, w.G, w.T)
    assert np.max(normwise(out, dense)) > 1e-4


def test_mixed_fallback_matches_blockwise_substitution():
    w, q, k16, v16 = small_case(B=1, T=500)
    cache = oracle.Cache(k16, v16, w.T)
    kb, vb, _ = cache.bounds(q, SM, 0.0, 0.0)
    tk = oracle.tau_for_fraction(kb, 0.3)
    tv = oracle.tau_for_fraction(vb, 0.3)
    out, mask = cache.attention(q, SM, tk, tv)
    assert 0 < (mask & 1).sum() < mask.size and 0 < (mask >> 1).sum() < mask.size
    khat, vhat = dequant(cache)
    kmix, vmix = khat.copy(), vhat.copy()
    for h in range(w.Hkv):
        for blk in range(cache.nblocks):
            sl = slice(blk * 64, blk * 64 + 64)
            if mask[0, h, blk] & 1:
                kmix[0, h, sl] = k16[0, h, sl]
            if mask[0, h, blk] & 2:
                vmix[0, h, sl] = v16[0, h, sl]
    ref = sdpa64(q, kmix, vmix, w.G, w.T)
    assert np.max(normwise(out, ref)) <= 1e-12


def test_closed_form_single_token():
    w, q, k16, v16 = small_case("single_head", T=1)
    cache = oracle.Cache(k16, v16, 1)
    out, _ = cache.attention(q, SM, np.inf, np.inf)
    _, vhat = dequant(cache)
    assert np.array_equal(out[0, 0], vhat[0, 0, 0])
    out, _ = cache.attention(q, SM, 0.0, 0.0)
    assert np.array_equal(out[0, 0], v16[0, 0, 0].astype(np.float64))


def test_closed_form_zero_query_is_mean_value():
    w, q, k16, v16 = small_case("single_head", T=333)
    q = np.zeros_like(q)
    cache = oracle.Cache(k16, v16, w.T)
    out, mask = cache.attention(q, SM, 0.0, np.inf)
    assert not (mask & 1).any()  # ||q|| = 0: the key bound is 0 everywhere
    _, vhat = dequant(cache)
    assert np.max(np.abs(out[0, 0] - vhat[0, 0, : w.T].mean(0))) <= 1e-14


def test_closed_form_identical_tokens():
    w, q, k16, v16 = small_case("single_head", T=200)
    k16[:, :, : w.T] = k16[:, :, :1]
    v16[:, :, : w.T] = v16[:, :, :1]
    cache = oracle.Cache(k16, v16, w.T)
    out, _ = cache.attention(q, SM, np.inf, np.inf)
    _, vhat = dequant(cache)
    assert np.max(np.abs(out[0, 0] - vhat[0, 0, 0])) <= 1e-13 * np.max(np.abs(vhat[0, 0, 0]))


def test_empty_cache_gives_zero_output():
    w, q, k16, v16 = small_case("single_head", T=64)
    cache = oracle.Cache(k16, v16, 0)
    out, mask = cache.attention(q, SM, 0.0, 0.0)
    assert not out.any() and mask.size == 0


def test_nonfinite_input_falls_back_to_dense_semantics():
    w, q, k16, v16 = small_case("single_head", T=256)
    k16[0, 0, 70, 5] = np.inf
    v16[0, 0, 130, 100] = np.nan
    cache = oracle.Cache(k16, v16, w.T)
    assert cache.k_err[0, 0, 1] == np.inf and cache.v_err[0, 0, 2] == np.inf
    _, _, m = cache.bounds(q, SM, np.inf, np.inf)
    assert m[0, 0, 1] & 1 and m[0, 0, 2] & 2  # +inf bound is never certified
    out, _ = cache.attention(q, SM, 0.0, 0.0)
    ref = sdpa64(q, k16, v16, w.G, w.T)
    assert np.array_equal(np.isnan(out), np.isnan(ref))


# ------------------------------------------------------------ cache statistics

def test_block_statistics_are_max_over_valid_tokens():
    w, q, k16, v16 = small_case("single_head", T=150)
    cache = oracle.Cache(k16, v16, w.T)
    for blk in range(cache.nblocks):
        ks, vs = [], []
        for t in range(blk * 64, min(w.T, blk * 64 + 64)):
            ks.append(oracle.quant_k_row(k16[0, 0, t])[2])
            vs.append(oracle.quant_v_row(v16[0, 0, t])[2])
        assert cache.k_err[0, 0, blk] == max(ks) and cache.v_err[0, 0, blk] == max(vs)
    # nibbles of tokens >= length inside the last written block are zero
    vc = cache.v_codes_unpacked()[0, 0]
    assert not vc[w.T: cache.nblocks * 64].any()
    assert vc[: w.T].min() >= -7 and vc[: w.T].max() <= 7
