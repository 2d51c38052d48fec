"""The matrix-core decode's two variants against the oracle: the streaming
one (tiles of each split's first blocks copied before their masks are known,
the rest of the group's work cut into equal ranges, the appended token's
block taken by the last split) and the general one (every mask formed
first), on the paths where they differ.  Masks bitwise, outputs within 2e-3
of the oracle's fp64 output and within fp16 rounding of each other.
Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology
1-2 and "Deterministic Recovery" (blocks served from the FP16 originals when
only their keys, only their values, or both fall back).
"""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, assert_tier1_equal, gpu_cache, normwise_err, oracle_cache, small, taus_for

pytestmark = pytest.mark.gpu

KERNELS = [kvq.KERNEL_AUTO, kvq.KERNEL_MFMA_TABLE]


def _both(w, d, tk, tv, T=None, splits=0, append=False):
    """Decode (or fused append + decode) with both variants and the oracle."""
    T = w.T if T is None else T
    T1 = T + 1 if append else T
    oc = oracle_cache(d, T1)
    ref, omask = oc.attention(d["q"].numpy(), SM, tk, tv)
    outs = []
    for kern in KERNELS:
        print(f"  kernel={kern} T={T} append={append} splits={splits} tk={tk:.4g} tv={tv:.4g}", flush=True)
        gc = gpu_cache(d, T)
        nb = (T1 + 63) // 64
        mask = torch.full((w.B, w.Hkv, nb), 0xEE, dtype=torch.uint8, device="cuda")
        call = kvq.kvq_append_decode if append else kvq.kvq_decode_attn
        out = call(gc, d["q"].cuda(), SM, tk, tv, mask_out=mask, kernel=kern, splits=splits)
        torch.cuda.synchronize()
        if append:
            assert_tier1_equal(gc, oc, T1)
        np.testing.assert_array_equal(mask.cpu().numpy(), omask)
        o = out.float().cpu().numpy()
        err = normwise_err(o, ref)
        assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"kernel {kern}: {err.max():.3e}"
        outs.append(o)
    assert normwise_err(outs[0], outs[1]).max() <= 2.0 ** -10
    return omask


@pytest.mark.parametrize("kind", ["k", "v", "kv", "mixed"])
def test_fallback_kinds(kind):
    # keys alone (16-token steps of FP16 keys), values alone (16-token steps
    # of FP16 values with the rows' key codes packed), both (8-token steps)
    w = small("stress_fallback", B=2, T=1500)
    print(f"[stream fallback {kind}]", flush=True)
    d = workloads.make(w)
    oc = oracle_cache(d, w.T)
    tk, tv = taus_for(oc, d["q"].numpy(), 0.15)
    if kind == "k":
        tv = float("inf")
    elif kind == "v":
        tk = float("inf")
    elif kind == "kv":
        tk = tv = 0.0
    m = _both(w, d, tk, tv)
    assert m.any()


@pytest.mark.parametrize("splits", [2, 3, 5])
def test_speculative_blocks_fall_back(splits):
    # spikes in the first blocks of every split's home range make the tiles
    # the streaming variant copied before the masks were known unusable
    w = small("llama3_8b_32k", B=1, T=4000)
    print(f"[stream speculative fallback] splits={splits}", flush=True)
    d = workloads.make(w)
    nb = (w.T + 63) // 64
    bps = (nb + splits - 1) // splits
    for s in range(splits):
        for j, blk in enumerate(range(s * bps, min(s * bps + 8, nb))):
            t = blk * 64 + 7
            if t >= w.T:
                continue
            if j % 3 == 0:
                d["k16"][:, :, t, 9] = 3000.0
            if j % 3 == 1:
                d["v16"][:, :, t, 40] = -3000.0
            if j % 4 == 3:
                d["k16"][:, :, t, 3] = 3000.0
                d["v16"][:, :, t, 3] = 3000.0
    # a spike quantizes the rest of its row to 0, so its block's key bound is
    # about sm * |q| * |k| ~ 10 (and the value bound hundreds), while the
    # other blocks stay below 3
    m = _both(w, d, 5.0, 2.0, splits=splits)
    assert (m[0, :, 0] & 1).all() and (m[0, :, 1] & 2).all()


@pytest.mark.parametrize("T", [2048 * 64, 2048 * 64 + 1])
def test_streaming_limit(T):
    # 2048 blocks: the streaming variant's largest sequence; one token more
    # goes to the general variant under KVQ_KERNEL_AUTO
    w = small("llama3_8b_32k", B=1, Hkv=1, Hq=4, T=T)
    print(f"[stream limit] T={T}", flush=True)
    d = workloads.make(w)
    oc = oracle_cache(d, w.T)
    tk, tv = taus_for(oc, d["q"].numpy(), 0.01)
    _both(w, d, tk, tv)


@pytest.mark.parametrize("T0", [64 + 15, 64 + 16, 64 + 31, 64 + 32, 64 + 47, 64 + 48, 64 + 63])
@pytest.mark.parametrize("spike", ["v", "k"])
def test_fused_append_into_fallback_block(T0, spike):
    # the appended token lies in a block that falls back on its values (its
    # key codes are patched into the packed layout of a 16-token step) or on
    # its keys, at the boundaries of the 16-token steps
    w = small("llama3_8b_32k", B=2, T=T0 + 1)
    print(f"[stream fused fallback] T0={T0} spike={spike}", flush=True)
    d = workloads.make(w)
    if spike == "v":
        d["v16"][:, :, T0, 77] = -3000.0
    else:
        d["k16"][:, :, T0, 5] = 3000.0
    # the spike quantizes the rest of its key row (value group) to 0: key
    # bound about 10, value bound about 2, against below 2 and 0.4 elsewhere
    m = _both(w, d, 5.0, 1.0, T=T0, append=True)
    assert np.all(m[:, :, T0 // 64] & (2 if spike == "v" else 1))


@pytest.mark.parametrize("T0,splits", [(64, 2), (128, 3), (700, 11), (1999, 0)])
def test_fused_append_split_layouts(T0, splits):
    # the appended token's block alone in the last split, or sharing it
    w = small("llama3_8b_32k", B=2, T=T0 + 1)
    print(f"[stream fused splits] T0={T0} splits={splits}", flush=True)
    d = workloads.make(w)
    oc = oracle_cache(d, T0 + 1)
    tk, tv = taus_for(oc, d["q"].numpy(), 0.05)
    _both(w, d, tk, tv, T=T0, splits=splits, append=True)
