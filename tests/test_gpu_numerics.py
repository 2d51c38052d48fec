"""The decode's P.V numerics at their edges, against the fp64 oracle
(output within 2e-3 normwise, masks bitwise): keys and values scaled by
powers of ten on 32k-token groups shaped like the Llama-3-8B workload (small
value scales put p * s_v near the fp16 subnormal range; large key scales
make the softmax nearly one-hot), and a 128k-token needle 17 nats above a
haystack whose values carry a per-channel mean offset: the haystack's
weights are near exp(-17) of the needle's and carry about 7% of the output
(normwise), so a numerator that dropped them would be off by 35 times the
bar.  Method: "Runtime-Certified
Bounded-Error Quantized Attention", Methodology 1-2 (the output is the
attention over the certified tiles and the FP16 fallback tiles)."""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, gpu_cache, oracle_cache, small, taus_for

pytestmark = pytest.mark.gpu

# The output is fp16: its own rounding adds up to half an fp16 spacing, which
# below 2^-14 (subnormals) is 2^-25 absolute, so rows whose largest output is
# about 1e-5 (keys x1e-2, values x1e-3: a nearly uniform softmax over small
# values) lose up to 2.3e-3 normwise to the format alone.  The bar is the
# 2e-3 normwise bound plus one fp16 subnormal spacing.
SUBNORMAL_STEP = 2.0 ** -24

KERNELS = [("auto", kvq.KERNEL_AUTO), ("table", kvq.KERNEL_MFMA_TABLE), ("valu", kvq.KERNEL_VALU)]


def _run(d, T, frac, kern):
    oc = oracle_cache(d, T)
    qn = d["q"].numpy()
    tk, tv = taus_for(oc, qn, frac)
    ref, omask = oc.attention(qn, SM, tk, tv)
    gc = gpu_cache(d, T - 1)
    B, Hkv = d["k16"].shape[:2]
    mask = torch.full((B, Hkv, (T + 63) // 64), 0xEE, dtype=torch.uint8, device="cuda")
    out = kvq.kvq_append_decode(gc, d["q"].cuda(), SM, tk, tv, mask_out=mask, kernel=kern)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(mask.cpu().numpy(), omask)
    o = out.float().cpu().numpy().astype(np.float64)
    # normwise error with the format's absolute term taken out
    den = np.abs(ref).max(axis=-1)
    err = np.maximum(np.abs(o - ref).max(axis=-1) - SUBNORMAL_STEP, 0.0) / np.where(den == 0, 1.0, den)
    return err, omask


@pytest.mark.parametrize("kname,kern", KERNELS)
@pytest.mark.parametrize("ks,vs", [(1e-2, 1.0), (1e2, 1.0), (1.0, 1e-2), (1.0, 1e-3), (1.0, 1e2), (1e-2, 1e-3)])
def test_magnitude_sweep(ks, vs, kname, kern):
    w = small("llama3_8b_32k", B=1)
    print(f"[numerics] keys x{ks} values x{vs} kernel {kname}", flush=True)
    d = workloads.make(w)
    d["k16"] = (d["k16"].float() * ks).half()
    d["v16"] = (d["v16"].float() * vs).half()
    assert torch.isfinite(d["k16"]).all() and torch.isfinite(d["v16"]).all()
    err, m = _run(d, w.T, 0.01, kern)
    print(f"  max normwise err {err.max():.3e}, fallback k {np.mean(m & 1):.4f} v {np.mean(m >> 1):.4f}", flush=True)
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"{err.max():.3e}"


@pytest.mark.parametrize("kname,kern", KERNELS)
@pytest.mark.parametrize("G", [1, 8])
def test_needle_over_offset_haystack(G, kname, kern):
    T = 131072
    print(f"[numerics] needle 17 nats over a {T}-token haystack, G={G}, kernel {kname}", flush=True)
    d = workloads.needle_over_haystack(T, SM, G=G)
    oc = oracle_cache(d, T)
    ref, _ = oc.attention(d["q"].numpy(), SM, float("inf"), float("inf"))
    # the haystack's share of the output: what a numerator that drops the
    # small weights would lose
    hay = np.abs(ref - d["v16"][0, 0, d["needle"]].float().numpy()[None, None, :]).max() / np.abs(ref).max()
    print(f"  haystack share of the output (normwise) {hay:.3e}", flush=True)
    assert hay > 4 * OUT_TOL  # the case is sensitive to the haystack's weights
    for frac in (0.0, 0.01):
        err, m = _run(d, T, frac, kern)
        print(f"  frac {frac}: max normwise err {err.max():.3e}, fallback blocks {int((m != 0).sum())}", flush=True)
        assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"frac {frac}: {err.max():.3e}"


@pytest.mark.parametrize("kname,kern", KERNELS)
def test_query_dynamic_range(kname, kern):
    """Queries far from N(0,1): outlier channels 50x and 300x the rest, heads
    scaled by 1e-3 and 1e2, a head that is zero but for one channel, and a
    zero head.  The fp16 query enters the products exactly, so a head's
    largest channel does not cost its small ones precision (a fixed-point
    query with 16 bits against max|q| did: 2.6e-3 here)."""
    w = small("llama3_8b_32k", B=2)
    print(f"[numerics] query dynamic range, kernel {kname}", flush=True)
    d = workloads.make(w)
    q = d["q"].float()
    g = torch.Generator().manual_seed(7)
    for b in range(w.B):
        for h in range(w.Hq):
            c = torch.randperm(128, generator=g)[:2]
            q[b, h, c[0]] *= 50.0
            if h % 4 == 1:
                q[b, h, c[1]] *= 300.0
    q[0, 2] *= 1e-3
    q[1, 3] *= 1e2
    q[0, 5] = 0.0
    q[0, 5, 17] = 3.0
    q[1, 6] = 0.0
    d["q"] = q.half()
    assert torch.isfinite(d["q"]).all()
    err, m = _run(d, w.T, 0.01, kern)
    print(f"  max normwise err {err.max():.3e}, fallback k {np.mean(m & 1):.4f} v {np.mean(m >> 1):.4f}", flush=True)
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"{err.max():.3e}"
