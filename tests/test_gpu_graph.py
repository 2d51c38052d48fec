"""A decode step (quantize-on-append of one token, certified decode, split
merge) captured in a HIP graph replays like the eager step on every replay,
with eager work and synchronisations between replays: the appended codes are
bitwise equal and the outputs agree to fp16 rounding (the decode kernel's
waves claim their steps dynamically, so accumulation order may differ).  The
library only launches kernels on the caller's stream, so it is capturable."""
import numpy as np
import pytest
import torch

import quantized_decode_attention_kvq_amd as kvq
import workloads
from kvq_testlib import SM, gpu_cache, normwise_err

pytestmark = pytest.mark.gpu


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
        wsg.fill_(0xAB)  # the workspace needs no contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert normwise_err(out_g.float().cpu().numpy(), ref).max() <= 2.0 ** -10, f"replay {rep}"
        np.testing.assert_array_equal(cg.k_codes[:, :, :w.T].cpu().numpy(), ref_codes, err_msg=f"replay {rep} codes")
        # eager work between replays
        step(ce, wse, out_e, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert normwise_err(out_e.float().cpu().numpy(), ref).max() <= 2.0 ** -10
