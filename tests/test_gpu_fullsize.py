"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (kvq_append_decode with the automatic kernel and split
choice: one fused append of the last token and decode, after a bulk
prefill).

The oracle cannot process a whole 32k- or 128k-token batch in seconds, so it
checks sampled (batch, KV head) groups one by one: the group's tier-1 bytes,
masks and output rows must match it (bitwise, bitwise, and within 2e-3).  For
every group, the masks the decode kernel used must equal kvq_bounds' masks.
Method: "Runtime-Certified Bounded-Error Quantized Attention", Methodology 1-2
and "Deterministic Recovery".
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, normwise_err, taus_for

pytestmark = pytest.mark.gpu


def _taus(kb, vb, frac):
    """The benchmark's tolerance rule: about `frac` of the blocks fall back per
    bound, chosen on the library's own bounds."""
    return (oracle.tau_for_fraction(kb.flatten().cpu().numpy(), frac),
            oracle.tau_for_fraction(vb.flatten().cpu().numpy(), frac))


def _group_oracle(d, b, h, T):
    k16 = d["k16"][b:b + 1, h:h + 1].cpu().numpy()
    v16 = d["v16"][b:b + 1, h:h + 1].cpu().numpy()
    return oracle.Cache(k16, v16, T)


def _check_group_tier1(c, oc, b, h, T):
    nb = (T + 63) // 64
    pairs = [
        ("k_codes", c.k_codes[b, h, :T], oc.k_codes[0, 0, :T]),
        ("k_scales", c.k_scales[b, h, :T].view(torch.int16), oc.k_scales[0, 0, :T].view(np.int16)),
        ("v_codes", c.v_codes[b, h, :nb], oc.v_codes[0, 0, :nb]),
        ("v_scales", c.v_scales[b, h, :T].view(torch.int16), oc.v_scales[0, 0, :T].view(np.int16)),
        ("k_err", c.k_err[b, h, :nb].view(torch.int32), oc.k_err[0, 0, :nb].view(np.int32)),
        ("v_err", c.v_err[b, h, :nb].view(torch.int32), oc.v_err[0, 0, :nb].view(np.int32)),
    ]
    for name, g, o in pairs:
        np.testing.assert_array_equal(g.cpu().numpy(), o, err_msg=f"{name} of group ({b}, {h})")


@pytest.mark.parametrize("name", ["llama3_8b_32k", "llama3_70b_128k", "stress_fallback", "single_head"])
def test_decode_full_size_sampled(name):
    w = workloads.WORKLOADS[name]
    print(f"[full size] {w}", flush=True)
    d = workloads.make(w, "cuda")
    q = d["q"].contiguous()
    # tolerances from the bounds of the full cache (as the benchmark does)
    c = kvq.KVCache(w.B, w.Hkv, w.cap, k16=d["k16"], v16=d["v16"])
    kvq.kvq_quantize_append(c, w.T)
    kb, vb, _ = kvq.kvq_bounds(c, q, SM, 0.0, 0.0, want=("kb", "vb"))
    tk, tv = _taus(kb, vb, w.fallback_frac)
    shape = kb.shape
    del c, kb, vb
    torch.cuda.empty_cache()
    # the benchmark's step on a fresh cache: prefill T-1 tokens, then one
    # fused append of token T-1 + decode (its tier-1 bytes written by the
    # decode kernel alone)
    c = kvq.KVCache(w.B, w.Hkv, w.cap, k16=d["k16"], v16=d["v16"])
    kvq.kvq_quantize_append(c, w.T - 1)
    mask = torch.full(shape, 0xEE, dtype=torch.uint8, device="cuda")
    out = kvq.kvq_append_decode(c, q, SM, tk, tv, mask_out=mask)
    assert c.length == w.T
    _, _, bmask = kvq.kvq_bounds(c, q, SM, tk, tv, want=("mask",))
    torch.cuda.synchronize()
    # every group: the masks used are the bounds' masks
    assert torch.equal(mask, bmask)
    m = mask.cpu().numpy()
    print(f"  tau=({tk:.4g}, {tv:.4g}) fallback k={np.mean(m & 1):.4f} v={np.mean(m >> 1):.4f}", flush=True)
    groups = sorted({(0, 0), (w.B - 1, w.Hkv - 1), (w.B // 2, w.Hkv // 2)})
    qn = q.cpu().numpy()
    for b, h in groups:
        oc = _group_oracle(d, b, h, w.T)
        _check_group_tier1(c, oc, b, h, w.T)
        ref, omask = oc.attention(qn[b:b + 1, h * w.G:(h + 1) * w.G], SM, tk, tv)
        np.testing.assert_array_equal(m[b:b + 1, h:h + 1], omask, err_msg=f"mask of group ({b}, {h})")
        got = out[b, h * w.G:(h + 1) * w.G].float().cpu().numpy()
        err = normwise_err(got, ref[0])
        print(f"  group ({b}, {h}): max normwise err {err.max():.3e}", flush=True)
        assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL


@pytest.mark.parametrize("rot", [False, True])
def test_bulk_quantize_full_size_sampled(rot):
    """1,048,576 new tokens x 8 KV heads in one append (plain and
    Hadamard-rotated key codec); sampled block-aligned windows of every head
    against the oracle, bitwise."""
    w = workloads.WORKLOADS["bulk_quantize"]
    print(f"[full size] {w} key_rotation={rot}", flush=True)
    d = workloads.make(w, "cuda")
    c = kvq.KVCache(w.B, w.Hkv, w.cap, k16=d["k16"], v16=d["v16"], key_rotation=rot)
    kvq.kvq_quantize_append(c, w.T)
    torch.cuda.synchronize()
    win = 2048
    starts = [0, (w.T // 2) // 64 * 64, w.T - win]
    for h in range(w.Hkv):
        for t0 in starts[h % 2:]:
            k16 = d["k16"][:, h:h + 1, t0:t0 + win].cpu().numpy()
            v16 = d["v16"][:, h:h + 1, t0:t0 + win].cpu().numpy()
            oc = oracle.Cache(k16, v16, win, key_rotation=rot)
            b0, nb = t0 // 64, win // 64
            pairs = [
                ("k_codes", c.k_codes[0, h, t0:t0 + win], oc.k_codes[0, 0]),
                ("k_scales", c.k_scales[0, h, t0:t0 + win].view(torch.int16), oc.k_scales[0, 0].view(np.int16)),
                ("v_codes", c.v_codes[0, h, b0:b0 + nb], oc.v_codes[0, 0]),
                ("v_scales", c.v_scales[0, h, t0:t0 + win].view(torch.int16), oc.v_scales[0, 0].view(np.int16)),
                ("k_err", c.k_err[0, h, b0:b0 + nb].view(torch.int32), oc.k_err[0, 0].view(np.int32)),
                ("v_err", c.v_err[0, h, b0:b0 + nb].view(torch.int32), oc.v_err[0, 0].view(np.int32)),
            ]
            for name, g, o in pairs:
                np.testing.assert_array_equal(g.cpu().numpy(), o, err_msg=f"{name} head {h} window {t0}")


def test_automatic_kernel_past_the_matrix_core_limit():
    # 1,050,000 tokens per sequence: 16,407 blocks, more than the matrix-core
    # kernel lists (128 blocks per split, 128 splits), so the automatic choice
    # is the VALU kernel, which appends with the append kernel first.  One
    # (b, kvh) group of four query heads, checked whole against the oracle.
    T = 1_050_000
    w = workloads.WORKLOADS["llama3_8b_32k"].scaled(B=1, Hkv=1, Hq=4, T=T)
    print(f"[full size] automatic kernel at {w}", flush=True)
    d = workloads.make(w, "cuda")
    q = d["q"].contiguous()
    oc = oracle.Cache(d["k16"].cpu().numpy(), d["v16"].cpu().numpy(), T)
    tk, tv = taus_for(oc, q.cpu().numpy(), w.fallback_frac)
    ref, omask = oc.attention(q.cpu().numpy(), SM, tk, tv)
    nb = (T + 63) // 64
    assert nb > 128 * 128
    c = kvq.KVCache(w.B, w.Hkv, w.cap, k16=d["k16"], v16=d["v16"])
    kvq.kvq_quantize_append(c, T - 1)
    out = torch.empty_like(q)
    mask = torch.full((1, 1, nb), 0xEE, dtype=torch.uint8, device="cuda")
    kvq.kvq_append_decode(c, q, SM, tk, tv, out=out, mask_out=mask)
    torch.cuda.synchronize()
    assert c.length == T
    _check_group_tier1(c, oc, 0, 0, T)
    np.testing.assert_array_equal(mask.cpu().numpy(), omask)
    err = normwise_err(out.float().cpu().numpy(), ref)
    assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, err.max()
    # the same decode through the VALU kernel by name gives the same bits, and
    # the matrix-core kernel refuses the sequence
    out_v = torch.empty_like(q)
    kvq.kvq_decode_attn(c, q, SM, tk, tv, out=out_v, kernel=kvq.KERNEL_VALU)
    torch.cuda.synchronize()
    assert torch.equal(out_v, out)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn(c, q, SM, tk, tv, kernel=kvq.KERNEL_MFMA)
    assert "unsupported" in str(e.value)
