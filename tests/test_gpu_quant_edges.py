"""GPU quantize-on-append on planted rounding cases, bitwise against the
oracle: elements exactly halfway between two codes (round half to even),
one fp16 ulp either side of such ties, scales that are not powers of two,
subnormal scales where the clamp to +-127 / +-7 binds, zero rows and rows
holding Inf or NaN.  The workloads' random data almost never hit these, and
the kernel derives codes from a reciprocal estimate corrected by an exact
residual, so every branch of that correction is exercised here.
Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_kvq_amd as kvq
from kvq_testlib import assert_tier1_equal

pytestmark = pytest.mark.gpu


def _f16_exact(x):
    return np.float16(x).astype(np.float64) == x


def _planted_rows(rng, n, lim, group):
    """n rows of 128 fp16 values; each `group`-channel group has an absmax
    lim*s for a scale s = m*2^e with a short mantissa, so that f16(absmax/lim)
    is s exactly and many halfway points (c + 1/2)*s are fp16 values."""
    rows = np.zeros((n, 128), np.float64)
    for r in range(n):
        for g0 in range(0, 128, group):
            kind = rng.integers(0, 10)
            if kind == 0:
                continue  # zero group: scale 0, codes 0
            if kind == 1:
                # subnormal scale: absmax a with a/f16(a/lim) > lim + 1/2
                a = float(rng.integers(lim + 1, 4 * lim)) * 2.0 ** -24
                vals = rng.uniform(-a, a, group)
                vals[rng.integers(0, group)] = a * rng.choice([-1, 1])
                rows[r, g0:g0 + group] = vals
                continue
            m = int(rng.integers(1, 16))
            e = int(rng.integers(-12, 0))
            s = m * 2.0 ** e
            a = lim * s
            vals = []
            for _ in range(group):
                c = int(rng.integers(-lim, lim))
                t = (c + 0.5) * s
                pick = rng.integers(0, 4)
                if pick == 0 and _f16_exact(t):
                    vals.append(t)                                   # exact tie
                elif pick == 1:
                    u = np.float16(t)
                    vals.append(float(np.nextafter(u, np.float16(np.inf))))   # just above
                elif pick == 2:
                    u = np.float16(t)
                    vals.append(float(np.nextafter(u, np.float16(-np.inf))))  # just below
                else:
                    vals.append(float(np.float16(rng.uniform(-a, a))))
            vals = np.clip(np.array(vals), -a, a)
            vals[rng.integers(0, group)] = a * rng.choice([-1, 1])
            rows[r, g0:g0 + group] = vals
    out = rows.astype(np.float16)
    # a few rows with non-finite entries
    out[rng.integers(0, n), rng.integers(0, 128)] = np.float16(np.inf)
    out[rng.integers(0, n), rng.integers(0, 128)] = np.float16(np.nan)
    return out


@pytest.mark.parametrize("chunks", [[640], [1, 63, 64, 5, 300, 207]])
def test_planted_rounding_cases_bitwise(chunks):
    rng = np.random.default_rng(20260521)
    T = sum(chunks)
    print(f"[planted ties] T={T} chunks={chunks}", flush=True)
    k = _planted_rows(rng, T, 127, 128)
    v = _planted_rows(rng, T, 7, 32)
    k16 = np.zeros((1, 1, 640, 128), np.float16)
    v16 = np.zeros_like(k16)
    k16[0, 0, :T], v16[0, 0, :T] = k, v
    # ties are really present
    assert np.count_nonzero(k16 != 0) > 1000
    c = kvq.KVCache(1, 1, 640, k16=torch.from_numpy(k16).cuda(), v16=torch.from_numpy(v16).cuda())
    for n in chunks:
        kvq.kvq_quantize_append(c, n)
    oc = oracle.Cache(k16, v16, T)
    assert_tier1_equal(c, oc, T)
