"""Helpers shared by the GPU parity tests: build a device cache from seeded
inputs, build the oracle's own cache from the same inputs, and compare."""
import math

import numpy as np
import torch

import oracle
import quantized_decode_attention_kvq_amd as kvq
import workloads

SM = float(np.float32(1 / math.sqrt(128)))
OUT_TOL = 2e-3  # max |o - o_ref| / max |o_ref| per output row


def gpu_cache(data, T, device="cuda", append_chunks=None, key_rotation=False):
    """Device cache holding T tokens of data['k16'/'v16'], appended in
    `append_chunks` (default: one bulk append)."""
    k16 = data["k16"].to(device).contiguous()
    v16 = data["v16"].to(device).contiguous()
    B, Hkv, cap, _ = k16.shape
    c = kvq.KVCache(B, Hkv, cap, device=device, k16=k16, v16=v16, key_rotation=key_rotation)
    for n in (append_chunks or [T]):
        kvq.kvq_quantize_append(c, n)
    assert c.length == T
    return c


def oracle_cache(data, T, key_rotation=False):
    return oracle.Cache(data["k16"].cpu().numpy(), data["v16"].cpu().numpy(), T, key_rotation=key_rotation)


def assert_tier1_equal(gc, oc, T):
    """Bitwise equality of every defined tier-1 byte."""
    torch.cuda.synchronize()
    nb = (T + 63) // 64
    kc = gc.k_codes.cpu().numpy()
    np.testing.assert_array_equal(kc[:, :, :T], oc.k_codes[:, :, :T], err_msg="k_codes")
    ks = gc.k_scales.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(ks[:, :, :T], oc.k_scales.view(np.uint16)[:, :, :T], err_msg="k_scales")
    vc = gc.v_codes.cpu().numpy()
    np.testing.assert_array_equal(vc[:, :, :nb], oc.v_codes[:, :, :nb], err_msg="v_codes")
    vs = gc.v_scales.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(vs[:, :, :T], oc.v_scales.view(np.uint16)[:, :, :T], err_msg="v_scales")
    ke = gc.k_err.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(ke[:, :, :nb], oc.k_err.view(np.uint32)[:, :, :nb], err_msg="k_err")
    ve = gc.v_err.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(ve[:, :, :nb], oc.v_err.view(np.uint32)[:, :, :nb], err_msg="v_err")


def normwise_err(out, ref):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref), axis=-1)
    return np.max(np.abs(out - ref), axis=-1) / np.where(den == 0, 1.0, den)


def taus_for(oc, q, frac):
    """Tolerances chosen on the oracle's own bounds so that about `frac` of the
    blocks fall back on each bound (0 -> tau 0, None -> +inf)."""
    if frac is None:
        return float("inf"), float("inf")
    if frac == 0:
        return 0.0, 0.0
    kb, vb, _ = oc.bounds(q, SM, 0.0, 0.0)
    return oracle.tau_for_fraction(kb, frac), oracle.tau_for_fraction(vb, frac)


def small(name, **kw):
    return workloads.WORKLOADS[name].scaled(**kw)
