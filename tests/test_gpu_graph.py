"""A decode step (quantize-on-append of one token, certified decode, split
merge) captured in a HIP graph replays like the eager step on every replay,
with eager work and synchronisations between replays: the appended codes are
bitwise equal and the outputs agree to fp16 rounding (the decode kernel's
waves claim their steps dynamically, so accumulation order may differ).  The
library only launches kernels on the caller's stream, so it is capturable.
The fused step of several layers captured in one graph, as a decoder's
per-token graph holds them, matches the oracle on every replay: each layer's
tier-1 bytes bitwise and its output within 2e-3 (Methodology 1-2 of
"Runtime-Certified Bounded-Error Quantized Attention"); the split merge done
in the decode launch leaves its arrival counters at zero for the next layer
and the next replay."""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import OUT_TOL, SM, assert_tier1_equal, gpu_cache, normwise_err, oracle_cache, taus_for

pytestmark = pytest.mark.gpu


def _counter_bytes(c):
    # the workspace's arrival counters: one uint32 per (batch, KV head), first
    return (4 * c.batch * c.kv_heads + 255) // 256 * 256


def test_captured_step_replays_like_eager():
    w = workloads.WORKLOADS["llama3_8b_32k"].scaled(B=2, T=1000)
    d = workloads.make(w, "cuda")
    print(f"graph replay: B{w.B} Hq{w.Hq} Hkv{w.Hkv} T{w.T}", flush=True)
    q = d["q"].contiguous()
    tau_k, tau_v = 3.0, 0.3

    def step(c, ws, out, stream):
        c.length = w.T - 1
        kvq.kvq_quantize_append(c, 1, stream)
        kvq.kvq_decode_attn(c, q, SM, tau_k, tau_v, out=out, workspace=ws, stream=stream)

    # eager reference
    ce = gpu_cache(d, w.T - 1)
    wse = kvq.make_workspace(ce, w.Hq)
    out_e = torch.empty_like(q)
    step(ce, wse, out_e, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = out_e.float().cpu().numpy()
    ref_codes = ce.k_codes[:, :, :w.T].cpu().numpy()  # rows past `length` are never written

    # captured step on a second cache
    cg = gpu_cache(d, w.T - 1)
    wsg = kvq.make_workspace(cg, w.Hq)
    out_g = torch.zeros_like(q)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    step(cg, wsg, out_g, torch.cuda.current_stream())  # warm-up (cached device attributes)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        step(cg, wsg, out_g, torch.cuda.current_stream())
    for rep in range(4):
        out_g.zero_()
        wsg[_counter_bytes(cg):].fill_(0xAB)  # the partials need no contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert normwise_err(out_g.float().cpu().numpy(), ref).max() <= 2.0 ** -10, f"replay {rep}"
        np.testing.assert_array_equal(cg.k_codes[:, :, :w.T].cpu().numpy(), ref_codes, err_msg=f"replay {rep} codes")
        # eager work between replays
        step(ce, wse, out_e, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert normwise_err(out_e.float().cpu().numpy(), ref).max() <= 2.0 ** -10


@pytest.mark.parametrize("shared_ws", [False, True])
def test_captured_layers_match_oracle(shared_ws):
    # three layers' fused steps (append + decode + split merge, one kernel
    # each) in one graph, each layer its own cache and output, with one
    # workspace per layer or one shared by the layers in turn
    w = workloads.WORKLOADS["llama3_8b_32k"].scaled(B=2, T=1500)
    R = 3
    d = workloads.make(w)
    print(f"graph layers: B{w.B} Hq{w.Hq} Hkv{w.Hkv} T{w.T} R{R} shared_ws={shared_ws}", flush=True)
    oc = oracle_cache(d, w.T)
    qn = d["q"].numpy()
    tk, tv = taus_for(oc, qn, 0.05)
    ref, omask = oc.attention(qn, SM, tk, tv)
    q = d["q"].cuda()
    caches = [gpu_cache(d, w.T - 1) for _ in range(R)]
    wss = [kvq.make_workspace(caches[0], w.Hq)] * R if shared_ws else [kvq.make_workspace(c, w.Hq) for c in caches]
    outs = [torch.zeros_like(q) for _ in range(R)]
    masks = [torch.zeros((w.B, w.Hkv, (w.T + 63) // 64), dtype=torch.uint8, device="cuda") for _ in range(R)]

    def layers(stream):
        for c, ws, o, m in zip(caches, wss, outs, masks):
            c.length = w.T - 1
            kvq.kvq_append_decode(c, q, SM, tk, tv, out=o, mask_out=m, workspace=ws, stream=stream)

    layers(torch.cuda.current_stream())  # warm-up
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        layers(torch.cuda.current_stream())
    for rep in range(4):
        for o, m, c in zip(outs, masks, caches):
            o.zero_()
            m.fill_(0xEE)
            c.k_codes[:, :, w.T - 1].fill_(0x55)  # the appended row is written again
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r, (c, o, m) in enumerate(zip(caches, outs, masks)):
            c.length = w.T
            assert_tier1_equal(c, oc, w.T)
            np.testing.assert_array_equal(m.cpu().numpy(), omask, err_msg=f"replay {rep} layer {r} masks")
            err = normwise_err(o.float().cpu().numpy(), ref)
            assert np.all(np.isfinite(err)) and err.max() <= OUT_TOL, f"replay {rep} layer {r}: {err.max():.3e}"
        for wsx in wss[:1] if shared_ws else wss:
            assert not wsx[:4 * w.B * w.Hkv].any(), "arrival counters left non-zero"
        # eager work between replays: the same layers launched eagerly
        layers(torch.cuda.current_stream())
        torch.cuda.synchronize()
        for o in outs:
            assert normwise_err(o.float().cpu().numpy(), ref).max() <= OUT_TOL
