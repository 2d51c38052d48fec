"""Pins for the oracle's codec (CPU only).

Each test checks the oracle against something other than itself: hand
derivations (tests/golden/hand_cases.json), exact rational arithmetic with
Python's fractions (round() on a Fraction rounds half to even), numpy's IEEE
fp16 conversion, and closed forms.  The codec follows "Runtime-Certified
Bounded-Error Quantized Attention", Methodology 1 (INT8 keys, INT4 values,
scales, per-block error annotations).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


# ------------------------------------------------------------ independent helpers

def f16_rne_of_fraction(r: Fraction) -> float:
    """Nearest binary16 to a non-negative rational, ties to even (textbook:
    pick the binade, divide by its quantum, round half to even)."""
    assert r >= 0
    if r == 0:
        return 0.0
    e = math.frexp(float(r))[1] - 1
    while Fraction(2) ** e > r:
        e -= 1
    while Fraction(2) ** (e + 1) <= r:
        e += 1
    quantum = Fraction(2) ** (max(e, -14) - 10)
    m = round(r / quantum)
    val = m * quantum
    if val > 65504:
        return math.inf
    return float(val)


def fp16_values_positive_finite():
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16)


def row(values, at=None):
    x = np.zeros(128, np.float16)
    if at is None:
        x[: len(values)] = values
    else:
        for k, v in at.items():
            x[int(k)] = v
    return x


# ------------------------------------------------------------ fp16 primitives

def test_f16_decode_matches_numpy_for_every_pattern():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_bits_to_f64(int(b)) for b in bits[::7]])
    r = ref[::7]
    both_nan = np.isnan(got) & np.isnan(r)
    assert np.array_equal(got[~both_nan], r[~both_nan])


def test_f32_to_f16_matches_numpy_rne():
    rng = np.random.default_rng(7)
    # random binary32 patterns across the whole range, plus every fp16 value and
    # every midpoint between adjacent fp16 values (the tie cases)
    rnd = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    xs = np.concatenate([rnd, h.astype(np.float32), mids, -mids, np.float32([65504, 65519.99, 65520, 1e9])])
    got = oracle.f32_to_f16_array(xs)
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    nan = np.isnan(xs)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


@pytest.mark.parametrize("div,which", [(127, "k"), (7, "v")])
def test_scale_bruteforce_every_fp16_absmax(div, which):
    """s = f16(f32(a)/div) equals the fp16 nearest to the exact rational a/div
    for every positive finite fp16 absmax a."""
    vals = fp16_values_positive_finite()
    step = 1  # all 31,743 values
    for a in vals[::step]:
        x = row([a])
        if which == "k":
            _, s, _ = oracle.quant_k_row(x)
        else:
            _, s4, _ = oracle.quant_v_row(x)
            s = s4[0]
        ref = f16_rne_of_fraction(Fraction(float(a)) / div)
        assert float(s) == ref, (float(a), float(s), ref)


# ------------------------------------------------------------ codes vs exact rationals

def _exact_codes(x, s, lim):
    if s == 0:
        return [0] * len(x)
    return [max(-lim, min(lim, round(Fraction(float(v)) / Fraction(float(s))))) for v in x]


def test_k_codes_are_rne_of_exact_quotient_random_rows():
    rng = np.random.default_rng(11)
    for trial in range(300):
        scale = 10.0 ** rng.uniform(-6, 4)
        x = (rng.standard_normal(128) * scale).astype(np.float16)
        if trial % 3 == 0:  # plant exact ties: multiples of s/2 with s a power of two
            s = np.float16(2.0 ** int(rng.integers(-8, 4)))
            n = rng.integers(-126, 126, size=128)
            x = (s * (n + 0.5)).astype(np.float16)
            x[0] = np.float16(127 * float(s))
        codes, s, err = oracle.quant_k_row(x)
        assert list(codes) == _exact_codes(x, s, 127)
        e = [Fraction(float(v)) - Fraction(float(s)) * int(c) for v, c in zip(x, codes)]
        exact = math.sqrt(float(sum(t * t for t in e)))
        assert abs(float(err) - exact) <= 2 * np.spacing(np.float32(exact))


def test_v_codes_are_rne_of_exact_quotient_random_rows():
    rng = np.random.default_rng(12)
    for trial in range(300):
        scale = 10.0 ** rng.uniform(-6, 4)
        x = (rng.standard_normal(128) * scale).astype(np.float16)
        if trial % 3 == 0:
            s = np.float16(2.0 ** int(rng.integers(-8, 4)))
            n = rng.integers(-7, 7, size=128)
            x = (s * (n + 0.5)).astype(np.float16)
            for g in range(4):
                x[32 * g] = np.float16(7 * float(s))
        codes, s4, err = oracle.quant_v_row(x)
        worst = Fraction(0)
        for g in range(4):
            xs = x[32 * g: 32 * g + 32]
            a = max(abs(Fraction(float(v))) for v in xs)
            assert float(s4[g]) == f16_rne_of_fraction(a / 7)
            cg = _exact_codes(xs, s4[g], 7)
            assert list(codes[32 * g: 32 * g + 32]) == cg
            for v, c in zip(xs, cg):
                worst = max(worst, abs(Fraction(float(v)) - Fraction(float(s4[g])) * c))
        assert float(err) == float(worst)  # exact, order-free


def test_subnormal_scale_clamp_path():
    # a = 178*2^-24 (an fp16 subnormal): a/127 is 1.40 quanta of 2^-24, so s
    # rounds down to one quantum and a/s = 178 exceeds 127: the clamp binds.
    a = np.float16(178 * 2.0 ** -24)
    codes, s, _ = oracle.quant_k_row(row([a, -a]))
    ref_s = f16_rne_of_fraction(Fraction(float(a)) / 127)
    assert float(s) == ref_s
    q = Fraction(float(a)) / Fraction(ref_s)
    assert q > 127
    assert codes[0] == 127 and codes[1] == -127
    # below 127*2^-25 the scale underflows to 0 and every code is 0
    tiny = np.float16(63 * 2.0 ** -24)
    codes, s, err = oracle.quant_k_row(row([tiny]))
    assert float(s) == 0 and not codes.any() and float(err) == float(tiny)


# ------------------------------------------------------------ hand cases

@pytest.mark.parametrize("case", GOLD["k_rows"], ids=lambda c: c["name"])
def test_hand_k_rows(case):
    codes, s, err = oracle.quant_k_row(row(case["x"]))
    assert int(np.float16(s).view(np.uint16)) == case["scale_bits"]
    n = len(case["codes"])
    assert list(codes[:n]) == case["codes"] and not codes[n:].any()
    assert float(err) == float(np.float32(math.sqrt(case["err_sq"])))


@pytest.mark.parametrize("case", GOLD["v_rows"], ids=lambda c: c["name"])
def test_hand_v_rows(case):
    x = row(case["x"]) if "x" in case else row(None, case["x_at"])
    codes, s4, err = oracle.quant_v_row(x)
    assert [int(b) for b in np.asarray(s4, np.float16).view(np.uint16)] == case["scale_bits"]
    if "codes" in case:
        n = len(case["codes"])
        assert list(codes[:n]) == case["codes"] and not codes[n:].any()
    else:
        expect = np.zeros(128, np.int8)
        for k, c in case["codes_at"].items():
            expect[int(k)] = c
        assert np.array_equal(codes, expect)
    assert float(err) == case["err"]


def test_hand_nibble_packing():
    c0, c1 = GOLD["nibble_packing"]["codes_token0_token1"]
    s = 1.0  # a=7 -> s=1 for both tokens
    v16 = np.zeros((1, 1, 64, 128), np.float16)
    v16[0, 0, 0, 0] = c0 * s
    v16[0, 0, 0, 1] = 7
    v16[0, 0, 1, 0] = c1 * s
    v16[0, 0, 1, 1] = 7
    k16 = np.zeros_like(v16)
    cache = oracle.Cache(k16, v16, 2)
    assert cache.v_codes[0, 0, 0, 0, 0] == GOLD["nibble_packing"]["byte"]
    # channel 1 holds 7 for both tokens: 0x77
    assert cache.v_codes[0, 0, 0, 1, 0] == 0x77
    assert not cache.v_codes[0, 0, 0, 2:].any()


# ------------------------------------------------------------ the pinned fp64 tree

def test_tree128_exact_when_partial_sums_are_exact():
    v = np.arange(128, dtype=np.float64)
    assert oracle.tree128(v) == 127 * 128 / 2


def test_tree128_cross_run_order_is_pinned():
    # Runs of 8 terms are summed first; run sums then pair at term strides
    # 64, 32, 16, 8.  Put A=1+2^-52 (odd significand) at term 0, +2^-53 at
    # term 64 and -2^-53 at term 8.  Pinned tree: (A + 2^-53) is a tie that
    # rounds to even -> 1+2^-51; then + (-2^-53) is again a tie between
    # 1+2^-52 (odd) and 1+2^-51 (even) -> 1+2^-51.  Summing in index order
    # instead gives (A - 2^-53) -> 1 then 1 + 2^-53 -> 1.
    v = np.zeros(128)
    v[0] = 1 + 2.0 ** -52
    v[64] = 2.0 ** -53
    v[8] = -(2.0 ** -53)
    assert oracle.tree128(v) == 1 + 2.0 ** -51
    assert math.fsum(v) == 1 + 2.0 ** -52  # exact sum differs from both


def test_tree128_in_run_order_is_pinned():
    # Within a run: strides 1, 2, 4.  (x0 + x1) = (1+2^-52) + 2^-53 -> 1+2^-51
    # (tie, even); (x2 + x3) = -2^-53; sum: 1 + 1.5*2^-52 -> tie -> 1+2^-51.
    # Pairing strides 4, 2, 1 instead would give (x0+x2) -> 1 first, then 1.
    v = np.zeros(128)
    v[0] = 1 + 2.0 ** -52
    v[1] = 2.0 ** -53
    v[2] = -(2.0 ** -53)
    assert oracle.tree128(v) == 1 + 2.0 ** -51


def test_tree128_close_to_exact_sum():
    rng = np.random.default_rng(5)
    for _ in range(200):
        v = rng.standard_normal(128) ** 2
        t = oracle.tree128(v)
        assert abs(t - math.fsum(v)) <= 8 * 2.0 ** -53 * math.fsum(v)


def test_qnorm_closed_forms():
    q = np.zeros(128, np.float16)
    q[5], q[77] = 3, 4
    assert oracle.qnorm(q) == 5.0
    assert oracle.qnorm(np.zeros(128, np.float16)) == 0.0
    q = np.full(128, 0.5, np.float16)
    assert oracle.qnorm(q) == float(np.float32(math.sqrt(32)))
    rng = np.random.default_rng(3)
    for _ in range(200):
        q = rng.standard_normal(128).astype(np.float16)
        exact = math.sqrt(math.fsum(float(x) ** 2 for x in q))
        assert abs(oracle.qnorm(q) - exact) <= np.spacing(np.float32(exact))


# ------------------------------------------------------------ non-finite inputs

def test_nonfinite_rows_force_infinite_error():
    x = row([1.0, 2.0])
    x[9] = np.inf
    codes, s, err = oracle.quant_k_row(x)
    assert not codes.any() and float(s) == 0 and err == np.inf
    x = row([1.0, 2.0])
    x[40] = np.nan
    codes, s4, err = oracle.quant_v_row(x)
    assert err == np.inf and float(s4[1]) == 0 and not codes[32:64].any()
    assert list(codes[:2]) == [4, 7] and float(s4[0]) == f16_rne_of_fraction(Fraction(2, 7))
