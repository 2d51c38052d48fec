"""Pins for the oracle's per-head output certificate and its rung-3
recompute (CPU only).

The certificate claims max_j |o_dense - o^| <= cert for every head, where
o_dense is dense attention over the FP16 keys and values and o^ the decode
output.  These tests check that claim against an independent dense
reference (torch SDPA in fp64) on workloads with outliers, spikes and every
fallback regime; the total-variation lemma behind the key term by brute
force and at its extremal case; the value term in closed form for q = 0
(uniform weights, so every block's mass is its share of the tokens); zero
certificates when every block falls back; and the recompute rung (heads over
tau_out come out dense).  Method: "Runtime-Certified Bounded-Error Quantized
Attention", Methodology 2 (two-term error decomposition: a key term from
the per-token score perturbation through the total variation of the softmax,
a value term from per-block reconstruction errors weighted by attention
mass) and Methodology 3 (rung 3, per-head fallback to FP16).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

SM = float(np.float32(1 / math.sqrt(128)))


def case(name, seed_shift=0, **kw):
    w = workloads.WORKLOADS[name].scaled(**kw)
    d = workloads.make(w, "cpu")
    return w, d["q"].numpy(), d["k16"].numpy(), d["v16"].numpy()


def sdpa64(q, k16, v16, G, T):
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    kt = torch.from_numpy(k16[:, :, :T].astype(np.float64)).repeat_interleave(G, dim=1).contiguous()
    vt = torch.from_numpy(v16[:, :, :T].astype(np.float64)).repeat_interleave(G, dim=1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SM)
    return o[:, :, 0, :].numpy()


def taus(cache, q, frac):
    kb, vb, _ = cache.bounds(q, SM, 0.0, 0.0)
    if frac is None:
        return float("inf"), float("inf")
    return oracle.tau_for_fraction(kb, frac), oracle.tau_for_fraction(vb, frac)


# --------------------------------------------------------------- the lemma

def test_total_variation_lemma():
    """Logit moves within [-D, D] change a softmax by at most tanh(D/2) in
    total variation, and the two-level move (+D on a set of mass
    1/(1+e^D), -D elsewhere) attains it."""
    rng = np.random.default_rng(7)
    for _ in range(2000):
        n = int(rng.integers(2, 40))
        dd = float(rng.uniform(0, 4))
        s = rng.normal(0, 3, n)
        delta = rng.uniform(-dd, dd, n)
        if rng.random() < 0.3:
            delta = np.where(rng.random(n) < 0.5, dd, -dd)
        p = np.exp(s - s.max()); p /= p.sum()
        ph = np.exp(s + delta - (s + delta).max()); ph /= ph.sum()
        tv = 0.5 * np.abs(p - ph).sum()
        assert tv <= math.tanh(dd / 2) + 1e-12
    # extremal: two tokens, masses a = 1/(1+e^D) and 1-a, moves +D and -D
    for dd in [0.1, 0.5, 1.0, 2.0, 5.0]:
        a = 1 / (1 + math.exp(dd))
        p = np.array([a, 1 - a])
        ph = p * np.exp([dd, -dd]); ph /= ph.sum()
        assert 0.5 * np.abs(p - ph).sum() == pytest.approx(math.tanh(dd / 2), rel=1e-12)


# ------------------------------------------------------- the bound holds

@pytest.mark.parametrize("name,kw", [("stress_fallback", dict(B=2, T=700)),
                                     ("llama3_8b_32k", dict(B=2, T=900)),
                                     ("llama3_70b_128k", dict(B=1, T=1100)),
                                     ("single_head", dict(T=1024))])
@pytest.mark.parametrize("frac", [0.0001, 0.02, 0.3, None])
def test_certificate_bounds_the_dense_error(name, kw, frac):
    w, q, k16, v16 = case(name, **kw)
    oc = oracle.Cache(k16, v16, w.T)
    tk, tv = taus(oc, q, frac)
    r = oc.certificate(q, SM, tk, tv)
    out, _ = oc.attention(q, SM, tk, tv)
    np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-14)  # no recompute at tau_out = inf
    assert not r["recomputed"].any()
    dense = sdpa64(q, k16, v16, w.G, w.T)
    err = np.abs(dense - out).max(-1)
    assert np.all(np.isfinite(r["cert"]))
    assert np.all(err <= r["cert"] * (1 + 1e-9) + 1e-12), (err / r["cert"]).max()
    np.testing.assert_allclose(r["cert"], r["e_key"] + r["e_val"], rtol=0, atol=0)
    assert np.all(r["e_key"] >= 0) and np.all(r["e_val"] >= 0)


def test_certificate_bounds_planted_spikes():
    """Spikes in certified blocks' neighbours and a query aligned with a key
    error: the dense error stays under the certificate."""
    w, q, k16, v16 = case("llama3_8b_32k", B=1, T=400)
    k16 = k16.copy(); v16 = v16.copy(); q = q.copy()
    k16[0, :, 130, 7] = np.float16(60.0)
    v16[0, :, 131, 9] = np.float16(-40.0)
    q[0, :, 7] = np.float16(9.0)
    oc = oracle.Cache(k16, v16, w.T)
    for frac in [0.01, 0.2]:
        tk, tv = taus(oc, q, frac)
        r = oc.certificate(q, SM, tk, tv)
        dense = sdpa64(q, k16, v16, w.G, w.T)
        err = np.abs(dense - r["out"]).max(-1)
        assert np.all(err <= r["cert"] * (1 + 1e-9) + 1e-12)


# ------------------------------------------------------- closed forms

def test_value_term_closed_form_for_zero_query():
    """q = 0: every logit is 0 and moves by 0, so the key term is 0 and the
    weights are uniform; the value term is sum over value-certified blocks of
    (tokens in block / T) * v_err."""
    w, q, k16, v16 = case("stress_fallback", B=2, T=333)
    q = np.zeros_like(q)
    oc = oracle.Cache(k16, v16, w.T)
    kb, vb, _ = oc.bounds(q, SM, 0.0, 0.0)
    tv = oracle.tau_for_fraction(vb, 0.2)
    r = oc.certificate(q, SM, 1.0, tv)
    _, _, mask = oc.bounds(q, SM, 1.0, tv)
    assert np.all(r["e_key"] == 0)
    nb = oc.nblocks
    ntok = np.array([min(64, w.T - 64 * i) for i in range(nb)], np.float64)
    for b in range(w.B):
        for hq in range(w.Hq):
            h = hq // w.G
            cert_v = ~(mask[b, h] >> 1 & 1).astype(bool)
            want = float(np.sum(ntok[cert_v] / w.T * oc.v_err[b, h, :nb][cert_v].astype(np.float64)))
            assert r["e_val"][b, hq] == pytest.approx(want, rel=1e-12, abs=1e-300)
    dense = sdpa64(q, k16, v16, w.G, w.T)
    assert np.all(np.abs(dense - r["out"]).max(-1) <= r["e_val"] * (1 + 1e-9) + 1e-12)


def test_everything_falls_back_gives_zero_certificate():
    """tau = 0: every block with a nonzero error falls back on both bounds,
    the decode is dense and both terms vanish."""
    w, q, k16, v16 = case("llama3_8b_32k", B=2, T=500)
    oc = oracle.Cache(k16, v16, w.T)
    assert np.all(oc.k_err[:, :, :oc.nblocks] > 0) and np.all(oc.v_err[:, :, :oc.nblocks] > 0)
    r = oc.certificate(q, SM, 0.0, 0.0)
    assert np.all(r["cert"] == 0)
    dense = sdpa64(q, k16, v16, w.G, w.T)
    np.testing.assert_allclose(r["out"], dense, rtol=0, atol=1e-12)


def test_certificate_is_monotone_in_the_tolerances():
    """Raising tau_k (tau_v) certifies more blocks: the key (value) term
    cannot shrink."""
    w, q, k16, v16 = case("stress_fallback", B=1, T=640)
    oc = oracle.Cache(k16, v16, w.T)
    kb, vb, _ = oc.bounds(q, SM, 0.0, 0.0)
    prev = None
    for frac in [0.5, 0.2, 0.05, 0.01]:
        tk, tv = oracle.tau_for_fraction(kb, frac), oracle.tau_for_fraction(vb, frac)
        r = oc.certificate(q, SM, tk, tv)
        if prev is not None:
            assert np.all(r["e_key"] >= prev["e_key"] - 1e-15)
        prev = r


# ------------------------------------------------------- rung 3

def test_recompute_rung_gives_dense_heads():
    w, q, k16, v16 = case("llama3_8b_32k", B=2, T=800)
    oc = oracle.Cache(k16, v16, w.T)
    tk, tv = taus(oc, q, 0.02)
    base = oc.certificate(q, SM, tk, tv)
    c = np.sort(base["cert"].ravel())
    tau_out = float((c[len(c) // 2 - 1] + c[len(c) // 2]) / 2)
    r = oc.certificate(q, SM, tk, tv, tau_out)
    np.testing.assert_array_equal(r["recomputed"], (base["cert"] > tau_out).astype(np.uint8))
    assert 0 < r["recomputed"].sum() < r["recomputed"].size
    dense = sdpa64(q, k16, v16, w.G, w.T)
    sel = r["recomputed"].astype(bool)
    np.testing.assert_allclose(r["out"][sel], dense[sel], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(r["out"][~sel], base["out"][~sel])
    np.testing.assert_array_equal(r["cert"], base["cert"])


# ------------------------------------------- under masks given by the caller

def _sdpa64_kv(q, k, v, G):
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(G, dim=1).contiguous()
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(G, dim=1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SM)[:, :, 0, :].numpy()


def test_certify_masked_against_sdpa():
    """certify_masked under caller masks: all blocks on FP16 is dense SDPA
    with a zero certificate; all blocks certified is SDPA over the
    dequantized keys (codes x scale) and values (nibbles x group scale);
    keys on FP16 with certified values is SDPA over FP16 keys and
    dequantized values; the bounds' own masks reproduce certificate(); a
    forced head comes out dense."""
    w, q, k16, v16 = case("llama3_8b_32k", B=2, T=333)
    oc = oracle.Cache(k16, v16, w.T)
    T, nb = w.T, oc.nblocks
    kq = oc.k_codes[:, :, :T].astype(np.float64) * oc.k_scales[:, :, :T, None].astype(np.float64)
    vq = oc.v_codes_unpacked()[:, :, :T].astype(np.float64) * \
        np.repeat(oc.v_scales[:, :, :T].astype(np.float64), 32, axis=-1)
    k, v = k16[:, :, :T], v16[:, :, :T]
    shape = (w.B, w.Hkv, nb)
    for bits, kk, vv in [(3, k, v), (0, kq, vq), (1, k, vq), (2, kq, v)]:
        r = oc.certify_masked(q, SM, np.full(shape, bits, np.uint8))
        np.testing.assert_allclose(r["out"], _sdpa64_kv(q, kk, vv, w.G), rtol=0, atol=1e-12)
        if bits == 3:
            assert np.all(r["cert"] == 0)
        assert not r["recomputed"].any()
    tk, tv = taus(oc, q, 0.1)
    _, _, m = oc.bounds(q, SM, tk, tv)
    r = oc.certify_masked(q, SM, m)
    c = oc.certificate(q, SM, tk, tv)
    for key in ("out", "cert", "e_key", "e_val", "recomputed"):
        np.testing.assert_array_equal(r[key], c[key])
    force = np.zeros((w.B, w.Hq), np.uint8)
    force[1, 5] = 1
    r = oc.certify_masked(q, SM, np.zeros(shape, np.uint8), force=force)
    assert r["recomputed"].sum() == 1 and r["recomputed"][1, 5] == 1
    np.testing.assert_allclose(r["out"][1, 5], sdpa64(q, k16, v16, w.G, T)[1, 5], rtol=0, atol=1e-12)
