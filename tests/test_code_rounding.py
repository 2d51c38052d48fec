"""The rounding argument behind the append kernels' codes, checked on the CPU.

The kernels form a code as the integer nearest x * r, with r an estimate of
1/s within an ulp (v_rcp_f32), in one rounding: fma(x, r, 1.5 * 2^23) leaves
that integer in the sum's low bits.  They rely on three facts, for fp16 x and
a codec scale s = f16(f32(absmax) / lim) with |x| <= absmax:
  - the estimate is round_half_even(x / s), clamped to [-lim, lim], except at
    an exact tie, where it is one of the two neighbours;
  - the residual x - c * s is exact in fp32 (one fma);
  - at a tie |x - c * s| = s / 2 exactly, and moving an odd code one step
    toward x gives the even one.
Here fp32 arithmetic is emulated exactly with float64 (products of an fp16
and an fp32 value, and their sum with 1.5 * 2^23, fit 53 bits) and numpy's
round-to-nearest-even conversions.  Method: "Runtime-Certified Bounded-Error
Quantized Attention", Methodology 1 (INT8 keys, INT4 values, absmax scales).
"""
import numpy as np
import pytest

BIAS = 12582912.0  # 1.5 * 2^23


def _all_fp16_positive():
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def _cases(lim, rng):
    am = _all_fp16_positive()
    am = np.concatenate([am[:2048], rng.choice(am, 6000, replace=False)])  # every subnormal scale, then a sample
    s = (am.astype(np.float32) / np.float32(lim)).astype(np.float16).astype(np.float64)
    keep = s > 0
    am, s = am[keep], s[keep]
    xs, ss = [], []
    for a, sc in zip(am, s):
        c = np.arange(-lim - 1, lim + 1, dtype=np.float64)
        t = (c + 0.5) * sc
        with np.errstate(over="ignore"):
            ties = t.astype(np.float16).astype(np.float64)
        ties = ties[(ties == t) & (np.abs(ties) <= a)]
        up = np.nextafter(ties.astype(np.float16), np.float16(np.inf)).astype(np.float64)
        dn = np.nextafter(ties.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
        rnd = rng.uniform(-a, a, 24).astype(np.float16).astype(np.float64)
        x = np.concatenate([ties, up, dn, rnd, [a, -a, 0.0]])
        x = x[np.abs(x) <= a]
        xs.append(x)
        ss.append(np.full(x.shape, sc))
    return np.concatenate(xs), np.concatenate(ss)


@pytest.mark.parametrize("lim", [127, 7])
def test_single_rounding_code_is_the_rounded_quotient_except_at_ties(lim):
    rng = np.random.default_rng(lim)
    x, s = _cases(lim, rng)
    q = x / s  # exact enough: a half-integer quotient is exact in fp64, others lie >= 2^-14 from one
    exact = np.clip(np.rint(q), -lim, lim)
    tie = (q - np.floor(q)) == 0.5
    r0 = (np.float32(1.0) / s.astype(np.float32))
    for r in (r0, np.nextafter(r0, np.float32(np.inf)), np.nextafter(r0, np.float32(0))):
        cb = (x * r.astype(np.float64) + BIAS).astype(np.float32).astype(np.float64)  # fma(x, r, BIAS)
        c = np.clip(cb - BIAS, -lim, lim)
        assert np.all(c[~tie] == exact[~tie])
        lo, hi = np.clip(np.floor(q[tie]), -lim, lim), np.clip(np.ceil(q[tie]), -lim, lim)
        assert np.all((c[tie] == lo) | (c[tie] == hi))
        # the residual is exact in fp32 and reaches s/2 only at ties or clamped quotients
        e = x - c * s
        assert np.all(e.astype(np.float32).astype(np.float64) == e)
        half = np.abs(e) == s / 2
        inside = np.abs(q) <= lim + 0.5
        assert np.all(tie[half] | ~inside[half])
        assert np.all(np.abs(e[inside]) <= s[inside] / 2)
        # the tie pass: an odd code at |e| = s/2 moves one step toward x, clamped again
        odd = (c % 2) != 0
        fixed = np.where(half & odd, np.clip(c + np.sign(e), -lim, lim), c)
        assert np.all(fixed == exact)
    assert tie.sum() > 100  # the planted halfway points are there


def test_quotients_stay_within_the_bound_of_the_argument():
    # |x / s| <= 190.5 for every scale of both codecs, subnormal ones included
    am = _all_fp16_positive()
    for lim in (127, 7):
        s = (am.astype(np.float32) / np.float32(lim)).astype(np.float16).astype(np.float64)
        ratio = am[s > 0] / s[s > 0]
        assert ratio.max() <= 190.5
