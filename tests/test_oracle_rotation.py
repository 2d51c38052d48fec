"""Pins for the oracle's Hadamard-rotated key codec (outlier-aware codec).

The rotation is the Walsh-Hadamard transform applied before scalar
quantization in the KQV scheme of "Statistical Inference and Quality
Measures of KV Cache Quantisations Inspired by TurboQuant" (technical
summary, quantisation schemes), read as a rotation of the keys alone.  The
oracle quantizes u = H k / 16 with the key codec and reads keys back as
k~ = H (s c) / 8.  What pins it, with H built by scipy.linalg.hadamard
(independent of the oracle's butterflies):
  - the stored key error equals ||k - k~|| (fp32 rounding), and every code is
    the round-half-even of u / s;
  - at tau = inf the decode equals SDPA over the keys k~; at tau = 0 it is
    dense attention, as with the plain codec;
  - the key bound still dominates the observed logit error for random
    queries and is tight for a query along k - k~;
  - a row with one large outlier channel gets a much smaller key error
    rotated than plain, and on the 32k workload's outlier channels the
    rotation lowers the key errors and the fallback share at a fixed tau;
  - non-finite rows still fall back (error +inf).
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import workloads

SM = float(np.float32(1 / math.sqrt(128)))
H = scipy.linalg.hadamard(128).astype(np.float64)


def case(name, **kw):
    w = workloads.WORKLOADS[name].scaled(**kw)
    d = workloads.make(w, "cpu")
    return w, d["q"].numpy(), d["k16"].numpy(), d["v16"].numpy()


def rot_keys(c):
    """k~ = H (s c) / 8 for every row of an oracle cache built with the rotation."""
    sc = c.k_codes.astype(np.float64) * c.k_scales.astype(np.float64)[..., None]
    return sc @ H.T / 8.0


def sdpa64(q, k, v, G, T):
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, :, None, :]
    kt = torch.from_numpy(np.asarray(k[:, :, :T], np.float64)).repeat_interleave(G, dim=1).contiguous()
    vt = torch.from_numpy(np.asarray(v[:, :, :T], np.float64)).repeat_interleave(G, dim=1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SM)[:, :, 0, :].numpy()


def dequant_v(c):
    vc = c.v_codes_unpacked().astype(np.float64)
    return vc * np.repeat(c.v_scales.astype(np.float64), 32, axis=-1)


def test_key_error_and_codes_of_the_rotated_codec():
    w, q, k16, v16 = case("llama3_8b_32k", B=1, T=512)
    c = oracle.Cache(k16, v16, w.T, key_rotation=True)
    k = k16[:, :, :w.T].astype(np.float64)
    kt = rot_keys(c)[:, :, :w.T]
    # per-token error ||k - k~||; the block statistic is its max
    err = np.linalg.norm(k - kt, axis=-1)
    blk = err.reshape(1, w.Hkv, -1, 64).max(-1)
    np.testing.assert_allclose(c.k_err[:, :, : blk.shape[-1]], blk, rtol=2 ** -22, atol=0)
    # codes: round half to even of u / s, u = H k / 16
    u = k @ H.T / 16.0
    s = c.k_scales[:, :, :w.T].astype(np.float64)[..., None]
    codes = c.k_codes[:, :, :w.T].astype(np.float64)
    assert np.all(np.abs(u / s - codes) <= 0.5)
    assert np.all(np.abs(codes) <= 127) and np.abs(codes).max() == 127


def test_tau_inf_is_attention_over_the_rotated_keys():
    w, q, k16, v16 = case("llama3_8b_32k", B=1, T=700)
    c = oracle.Cache(k16, v16, w.T, key_rotation=True)
    out, mask = c.attention(q, SM, float("inf"), float("inf"))
    assert not mask.any()
    ref = sdpa64(q, rot_keys(c), dequant_v(c), w.G, w.T)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_tau_zero_is_dense_attention():
    w, q, k16, v16 = case("stress_fallback", B=1, T=500)
    c = oracle.Cache(k16, v16, w.T, key_rotation=True)
    out, _ = c.attention(q, SM, 0.0, 0.0)
    ref = sdpa64(q, k16, v16, w.G, w.T)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_key_bound_dominates_and_is_tight():
    w, q, k16, v16 = case("llama3_8b_32k", B=1, T=640)
    c = oracle.Cache(k16, v16, w.T, key_rotation=True)
    k = k16[0, :, :w.T].astype(np.float64)
    diff = k - rot_keys(c)[0, :, :w.T]
    kb, _, _ = c.bounds(q, SM, 0.0, 0.0)
    G = w.G
    for h in range(w.Hkv):
        obs = np.abs(SM * diff[h] @ q[0, h * G:(h + 1) * G].astype(np.float64).T).max(-1)
        assert np.all(obs.reshape(-1, 64).max(-1) <= kb[0, h])
    # a query along the worst token's error: the bound is attained up to rounding
    t = int(np.argmax(np.linalg.norm(diff[0], axis=-1)))
    qa = np.zeros((1, w.Hq, 128), np.float16)
    qa[0, 0] = (diff[0, t] / np.abs(diff[0, t]).max() * 4).astype(np.float16)
    kb1, _, _ = c.bounds(qa, SM, 0.0, 0.0)
    obs = abs(SM * diff[0, t] @ qa[0, 0].astype(np.float64))
    ratio = obs / kb1[0, 0, t // 64]
    assert 0.99 <= ratio <= 1.0


def test_rotation_shrinks_the_error_of_an_outlier_row():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(128).astype(np.float16)
    x[17] = np.float16(300.0)
    for rot, fn in ((False, "kvqo_quant_k_row"), (True, "kvqo_quant_k_row_rot")):
        codes = np.zeros(128, np.int8)
        scale = np.zeros(1, np.uint16)
        err = np.zeros(1, np.float32)
        getattr(oracle.lib(), fn)(oracle._p(x), oracle._p(codes), oracle._p(scale), oracle._p(err))
        if rot:
            e_rot = float(err[0])
        else:
            e_plain = float(err[0])
    assert e_rot < e_plain / 4


def test_rotation_cuts_fallback_on_outlier_channels():
    w, q, k16, v16 = case("llama3_8b_32k", B=2, T=2048)
    plain = oracle.Cache(k16, v16, w.T)
    rot = oracle.Cache(k16, v16, w.T, key_rotation=True)
    nb = plain.nblocks
    assert np.median(rot.k_err[:, :, :nb]) < 0.8 * np.median(plain.k_err[:, :, :nb])
    kb, _, _ = plain.bounds(q, SM, 0.0, 0.0)
    tk = oracle.tau_for_fraction(kb, 0.05)
    _, _, mp = plain.bounds(q, SM, tk, float("inf"))
    _, _, mr = rot.bounds(q, SM, tk, float("inf"))
    assert (mr & 1).mean() < 0.5 * (mp & 1).mean()


def test_non_finite_rows_fall_back():
    w, q, k16, v16 = case("single_head", T=256)
    k16 = k16.copy()
    k16[0, 0, 70, 3] = np.float16(np.inf)
    c = oracle.Cache(k16, v16, w.T, key_rotation=True)
    assert np.isinf(c.k_err[0, 0, 1]) and not c.k_codes[0, 0, 70].any() and c.k_scales[0, 0, 70] == 0
    _, mask = c.attention(q, SM, 1e30, 1e30)
    assert mask[0, 0, 1] & 1
