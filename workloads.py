"""Seeded synthetic inputs for the certified quantized-KV decode path.

This module only draws random inputs; it holds none of the method's
arithmetic, so both the HIP path and the CPU oracle can be fed from it.

Every input is fp16 drawn as float32 from torch's counter-based Philox
generator (or CPU Mersenne generator) seeded per workload, then rounded to
fp16 (round to nearest even).  Layouts:
    q        [B][Hq][128]
    k16, v16 [B][Hkv][cap][128]   (tier-2 originals, tokens t < T filled)

Workloads (their shapes follow Llama-3-style GQA decode):
    single_head      B1  Hq1  Hkv1  T1024   2 fixed K outlier channels x20
    llama3_8b_32k    B8  Hq32 Hkv8  T32768  4 K outlier channels x15 per KV head
    llama3_70b_128k  B4  Hq64 Hkv8  T131072 1% of tokens: K and V ~ Student-t(3)
    stress_fallback  B16 Hq32 Hkv8  T8192   10% of 64-token blocks get one K and
                                            one V element scaled x50
    bulk_quantize    B1  Hkv8  1,048,576 new tokens, 3 K outlier channels x20
    llama3_8b_32k_niah  the llama3_8b_32k shape and structure plus 8 needle
                     tokens per (batch, KV head) at seeded positions, whose
                     keys point along the sum of the group's queries with
                     staggered strengths (a retrieval-shaped attention
                     pattern standing in for needle-in-a-haystack prompts)
"""
from dataclasses import dataclass, replace

import torch

D = 128
BLK = 64


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    seed: int
    k_outlier_channels: int = 0
    k_outlier_scale: float = 1.0
    t_token_frac: float = 0.0      # fraction of tokens with Student-t(nu) K and V
    t_nu: int = 3
    spike_block_frac: float = 0.0  # fraction of 64-token blocks with one x`spike` K and V element
    spike_scale: float = 1.0
    fallback_frac: float = 0.0     # target share of blocks falling back, per bound
    needles: int = 0               # needle tokens per (batch, KV head)
    needle_dot: float = 0.0        # smallest q_h . k of the strongest needle over the group's heads

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def cap(self):
        return (self.T + BLK - 1) // BLK * BLK

    def scaled(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "single_head": Workload("single_head", 1, 1, 1, 1024, 1001, k_outlier_channels=2,
                            k_outlier_scale=20.0, fallback_frac=0.02),
    "llama3_8b_32k": Workload("llama3_8b_32k", 8, 32, 8, 32768, 1002, k_outlier_channels=4,
                              k_outlier_scale=15.0, fallback_frac=0.01),
    "llama3_70b_128k": Workload("llama3_70b_128k", 4, 64, 8, 131072, 1003, t_token_frac=0.01,
                                t_nu=3, fallback_frac=0.005),
    "stress_fallback": Workload("stress_fallback", 16, 32, 8, 8192, 1004, spike_block_frac=0.10,
                                spike_scale=50.0, fallback_frac=0.10),
    "bulk_quantize": Workload("bulk_quantize", 1, 8, 8, 1048576, 1005, k_outlier_channels=3,
                              k_outlier_scale=20.0),
    "llama3_8b_32k_niah": Workload("llama3_8b_32k_niah", 8, 32, 8, 32768, 1006, k_outlier_channels=4,
                                   k_outlier_scale=15.0, fallback_frac=0.01, needles=8,
                                   needle_dot=226.0),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def make(w: Workload, device="cpu"):
    """Returns dict(q, k16, v16) as fp16 tensors on `device` for workload `w`."""
    g = _gen(device, w.seed)
    B, Hq, Hkv, T, cap = w.B, w.Hq, w.Hkv, w.T, w.cap
    q = _normal((B, Hq, D), g, device)
    k = torch.zeros((B, Hkv, cap, D), dtype=torch.float32, device=device)
    v = torch.zeros((B, Hkv, cap, D), dtype=torch.float32, device=device)
    k[:, :, :T] = _normal((B, Hkv, T, D), g, device)
    v[:, :, :T] = _normal((B, Hkv, T, D), g, device)

    if w.k_outlier_channels:
        # per KV head, a fixed random set of channels scaled for every token
        for h in range(Hkv):
            ch = torch.randperm(D, generator=g, device=device)[: w.k_outlier_channels]
            k[:, h, :T, ch] *= w.k_outlier_scale

    if w.t_token_frac > 0:
        n = max(1, int(round(w.t_token_frac * T)))
        for b in range(B):
            for h in range(Hkv):
                tok = torch.randperm(T, generator=g, device=device)[:n]
                for dst in (k, v):
                    z = _normal((n, D), g, device)
                    chi = (_normal((w.t_nu, n, D), g, device) ** 2).sum(0) / w.t_nu
                    dst[b, h, tok] = z / chi.sqrt()

    if w.spike_block_frac > 0:
        nb = T // BLK
        n = max(1, int(round(w.spike_block_frac * nb)))
        for b in range(B):
            for h in range(Hkv):
                blocks = torch.randperm(nb, generator=g, device=device)[:n]
                for dst in (k, v):
                    t = blocks * BLK + torch.randint(0, BLK, (n,), generator=g, device=device)
                    j = torch.randint(0, D, (n,), generator=g, device=device)
                    dst[b, h, t, j] *= w.spike_scale

    if w.needles:
        # needle i of a (b, kvh): key along u, the unit sum of the group's
        # queries, scaled so that its smallest dot product with them is
        # needle_dot * (1 - i / (4 * needles))
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hkv):
                qg = q[b, h * G:(h + 1) * G]
                u = qg.sum(0)
                u = u / u.norm()
                dmin = float((qg @ u).min().clamp(min=1e-3))
                tok = torch.randperm(T, generator=g, device=device)[: w.needles]
                for i in range(w.needles):
                    k[b, h, tok[i]] = u * (w.needle_dot * (1 - i / (4 * w.needles)) / dmin)

    return dict(q=q.half(), k16=k.half(), v16=v.half())


def needle_over_haystack(T, sm, seed=2001, needle_nats=17.0, offset=1.0, G=1, device="cpu"):
    """One (batch, KV head) group of T tokens: a haystack of N(0,1) keys (so
    logits sm * q.k about N(0,1)) whose values carry a per-channel mean offset
    of +-offset (seeded signs) plus N(0, 0.25^2) noise, and one needle at a
    seeded position whose key lies along the unit sum u of the group's G
    queries, scaled so that its smallest logit over the heads is needle_nats,
    with N(0,1) values.  Returns dict(q, k16, v16, needle) as fp16 tensors of
    shapes [1][G][128], [1][1][cap][128] and the needle's position."""
    g = _gen(device, seed)
    cap = (T + BLK - 1) // BLK * BLK
    q = _normal((1, G, D), g, device)
    k = torch.zeros((1, 1, cap, D), dtype=torch.float32, device=device)
    v = torch.zeros((1, 1, cap, D), dtype=torch.float32, device=device)
    k[0, 0, :T] = _normal((T, D), g, device)
    signs = torch.where(_normal((D,), g, device) >= 0, 1.0, -1.0)
    v[0, 0, :T] = offset * signs + 0.25 * _normal((T, D), g, device)
    pos = int(torch.randint(0, T, (1,), generator=g, device=device))
    u = q[0].sum(0)
    u = u / u.norm()
    dmin = float((q[0] @ u).min().clamp(min=1e-3))
    k[0, 0, pos] = u * (needle_nats / (sm * dmin))
    v[0, 0, pos] = _normal((D,), g, device)
    return dict(q=q.half(), k16=k.half(), v16=v.half(), needle=pos)
