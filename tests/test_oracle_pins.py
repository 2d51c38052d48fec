"""Pins of the oracle's certificate, value promotion and rotated codec that a
plausible slip in each would fail.

- The per-head certificate ("Runtime-Certified Bounded-Error Quantized
  Attention", technical summary, Methodology 2, Two-Term Error
  Decomposition) against the hand derivation in
  tests/golden/certificate_cases.json: a planted three-block cache with two
  heads of different norms, whose quantization errors and block masses have
  closed forms.  It fixes Delta from each head's own norm, the factor 1/2 in
  tanh(Delta/2), both branches of R = 2*max(7S + eta, A) and the
  mass-weighted value term.
- Rung 2 of the fallback ladder (Methodology 3, "promote values"): a value
  tile is promoted when the block's estimated mass times its value error
  exceeds tau_vc.  A planted cache has a high-error block of negligible mass
  (not promoted), a low-error block of large mass (promoted) and an
  error-free block of large mass (not promoted), so that a rule on the error
  alone or on the mass alone fails.
- The rotated key codec (Walsh-Hadamard transform before scalar quantization,
  "Statistical Inference and Quality Measures of KV Cache Quantisations
  Inspired by TurboQuant", quantisation schemes): rows whose rotated values
  u = H k / 16 are exact half-integers, so the rounding direction at a tie is
  pinned to round-half-even.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "certificate_cases.json")))


def _row(spec):
    r = np.zeros(128, np.float16)
    for j, v in spec.items():
        r[int(j)] = v
    return r


@pytest.mark.parametrize("case", sorted(GOLD["cases"]))
def test_certificate_hand_cases(case):
    su = GOLD["setup"]
    B, Hkv, Hq, cap, T = 1, 1, 2, 192, 150
    k16 = np.zeros((B, Hkv, cap, 128), np.float16)
    v16 = np.zeros_like(k16)
    for b, (kr, vr) in enumerate(zip(su["k_rows"], su["v_rows"][case])):
        k16[0, 0, 64 * b: min(64 * b + 64, T)] = _row(kr)
        v16[0, 0, 64 * b: min(64 * b + 64, T)] = _row(vr)
    q = np.zeros((B, Hq, 128), np.float16)
    q[0, 0] = _row(su["q"]["head0"])
    q[0, 1] = _row(su["q"]["head1"])
    c = oracle.Cache(k16, v16, T)
    np.testing.assert_array_equal(c.k_err[0, 0], np.float32(GOLD["kerr"]))
    kb, vb, mask = c.bounds(q, su["sm"], su["tau_k"], su["tau_v"])
    np.testing.assert_array_equal(kb[0, 0], np.float32(GOLD["key_bounds"]))
    np.testing.assert_array_equal(mask[0, 0], GOLD["masks"])
    r = c.certificate(q, su["sm"], su["tau_k"], su["tau_v"])
    heads = GOLD["cases"][case]["heads"]
    for h in range(2):
        g = heads[f"head{h}"]
        np.testing.assert_allclose(r["e_key"][0, h], g["e_key"], rtol=1e-12, atol=0)
        np.testing.assert_allclose(r["e_val"][0, h], g["e_val"], rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(r["cert"][0, h], g["cert"], rtol=1e-12, atol=0)
    # the two heads differ only in their own norm (4 and 2): a group norm
    # would give head 1 head 0's key term
    assert r["e_key"][0, 1] < 0.51 * r["e_key"][0, 0]


def _rung2_cache():
    # keys [x_i, 127, 0...]: scale 1, exact codes, so the scoring pass's block
    # log-masses are ln 64 + sm * x_i; q = e_0, sm = 1/8
    T = 192
    k16 = np.zeros((1, 1, T, 128), np.float16)
    v16 = np.zeros_like(k16)
    for b, x in enumerate([-80.0, 0.0, 0.0]):
        k16[0, 0, 64 * b: 64 * b + 64, 0] = x
        k16[0, 0, 64 * b: 64 * b + 64, 1] = 127.0
    # values: block 0 (70, 5): scale 10, v_err 5; block 1 (7, 0.125): scale 1,
    # v_err 0.125; block 2 (7, 1): exact, v_err 0
    for b, (a, e) in enumerate([(70.0, 5.0), (7.0, 0.125), (7.0, 1.0)]):
        v16[0, 0, 64 * b: 64 * b + 64, 0] = a
        v16[0, 0, 64 * b: 64 * b + 64, 1] = e
    q = np.zeros((1, 1, 128), np.float16)
    q[0, 0, 0] = 1.0
    return oracle.Cache(k16, v16, T), q


@pytest.mark.parametrize("tau_vc,expect", [
    # masses (e^-10, 1, 1) / (2 + e^-10): products m*v_err = 1.1e-4, 0.0625, 0
    (0.03, [0, 2, 0]),     # only the large-mass, small-error block
    (1e-3, [0, 2, 0]),
    (5e-5, [2, 2, 0]),     # the small-mass, large-error block joins
    (0.07, [0, 0, 0]),
])
def test_value_promotion_weighs_error_by_mass(tau_vc, expect):
    c, q = _rung2_cache()
    np.testing.assert_array_equal(c.v_err[0, 0, :3], np.float32([5.0, 0.125, 0.0]))
    r = c.adaptive(q, 0.125, float("inf"), float("inf"), tau_cov=0.0, tau_vc=tau_vc)
    m = np.exp(r["lhat"][0, 0] - np.log(np.exp(r["lhat"][0, 0]).sum()))
    np.testing.assert_allclose(m, np.array([math.exp(-10), 1.0, 1.0]) / (2 + math.exp(-10)), rtol=1e-12)
    np.testing.assert_array_equal(r["masks"][0, 0], expect)
    assert r["kstar"][0, 0] == 0


@pytest.mark.parametrize("a,b,half", [(1036.0, 996.0, 2.5), (1044.0, 988.0, 3.5), (996.0, 1036.0, -2.5),
                                      (988.0, 1044.0, -3.5), (1028.0, 1004.0, 1.5)])
def test_rotated_codec_rounds_exact_ties_to_even(a, b, half):
    # k = a e_0 + b e_1: u = H k / 16 is (a + b)/16 = 127 on even channels and
    # (a - b)/16 = `half` on odd ones (column 1 of the Sylvester matrix
    # alternates in sign), so the scale is f16(127/127) = 1 and every odd
    # quotient is an exact tie
    k = np.zeros(128, np.float16)
    k[0], k[1] = a, b
    codes, scale, err = oracle.quant_k_row_rot(k)
    assert float(scale) == 1.0
    assert np.all(codes[0::2] == 127)
    even = 2 * round(half / 2)  # the even neighbour of the tie
    assert abs(even - half) == 0.5
    np.testing.assert_array_equal(codes[1::2], np.full(64, even, np.int8))
    # |u - s c| = 0.5 on the 64 odd channels: ||k - k~|| = sqrt(2 * 64 * 0.25)
    assert err == np.float32(math.sqrt(32.0))
