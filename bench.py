"""Benchmark of the certified quantized-KV decode step on one MI355X.

One step = one decode step of one attention layer for the whole batch:
kvq_append_decode, i.e. quantize-on-append of the new token of every sequence
fused into the split-K decode kernel (bounds, fallback masks, streamed tiles,
the online softmax and the merge of the splits, by the last workgroup of each
(batch, KV head) group to finish; --unfused: the append as its own kernel
first).  Inputs are resident in HBM when
the timed region starts.  Several layers' caches ("replicas") are cycled so
that consecutive steps never find their KV stream in the 256 MB Infinity
Cache, as in a real multi-layer decode; by default the steps of up to 32
layers (cycling those caches) are captured in one HIP graph, as a 32-layer
decoder's per-token graph holds its layers, and replayed.

The GPU's power management holds a lower clock for the first milliseconds of
sustained load (measured per launch: 1.6-2.4 GHz, and the decode kernel's time
follows it), so the timed steps follow 20 ms of untimed replays of the same
graph, as in a decoder that runs the step continuously.

Prints one JSON line:
  value      effective KV bandwidth of the step: algorithmic bytes / step time
             (GB/s, 1e9 B/s); tokens_per_s and pct_of_hbm_peak beside it.
  roofline   for the dominant kernel: its algorithmic bytes per launch / its
             mean launch time, against the 8 TB/s HBM3E peak.  On the
             matrix-core path the fused step is one kernel (append, decode,
             and the split merge done by the last workgroup of each group):
             its bytes are the step's, and its launch time comes from HIP
             events on the stream around a second pass of the timed loop's
             steps (queued behind a third, untimed pass, so that the span is
             the kernels' own, not the host's submission latency, and the GPU
             stays under load).  Elsewhere (VALU
             kernel, --unfused) it is the split-K kernel: the decode's bytes
             but the output, timed by events around each of the same steps
             run again eagerly (the library records one after the split-K
             kernel).  traffic: from committed rocprofv3 FETCH_SIZE /
             WRITE_SIZE runs when they match the sources.
  adaptive_step  the same step through kvq_decode_attn_adaptive (INT8
             scoring pass, top-K* promotion covering tau_cov, ranking check,
             recompute of inconsistent heads), with the promoted shares.
  certified_step  the same step through kvq_decode_attn_cert: per-head
             output certificate only, and with the FP16 recompute of the heads
             above a tau_out that flags about 1% of them (ms per step each).
  cpu_baseline  the CPU oracle (fp64, OpenMP) timed on a bounded sample of
             the same workload, same byte accounting.

Algorithmic bytes per decode, per (batch, KV head, 64-token block):
  8 (k_err, v_err) + key tile (8192 codes + 128 scale bytes, or 16384 fp16
  bytes on key fallback) + value tile (4096 nibble bytes + 512 scale bytes,
  or 16384 fp16 bytes on value fallback); plus q and out (256 B per head
  each).  Per append: the new token's fp16 K and V rows (512 B) read, its
  codes, scales and block statistics (210 B) written, per (batch, KV head).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "decode_counters.json")
APPEND_COUNTERS = os.path.join(ROOT, "profiles", "append_counters.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200,
                   help="timed steps (200 decode steps of one layer take about 16 ms at 32k)")
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llama3_8b_32k")
    p.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma", "mfma_table"])
    p.add_argument("--q-heads", type=int, default=0,
                   help="query heads (0: the workload's), for group-size comparisons")
    p.add_argument("--splits", type=int, default=0)
    p.add_argument("--replicas", type=int, default=0, help="layer caches cycled (0: enough for >= 2 GB)")
    p.add_argument("--fallback-frac", type=float, default=None,
                   help="fraction of blocks per bound that fall back (default: the workload's; 0: none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work of the oracle sample")
    p.add_argument("--taus", default=None,
                   help="explicit tolerances 'tau_k,tau_v' (inf allowed), overriding --fallback-frac")
    p.add_argument("--unfused", action="store_true",
                   help="step as two calls (kvq_quantize_append, kvq_decode_attn) instead of kvq_append_decode")
    p.add_argument("--graph", type=int, default=1,
                   help="1: replay the steps from captured HIP graphs (up to 32 layer steps in one graph); "
                        "0: eager launches")
    p.add_argument("--no-certify", action="store_true",
                   help="skip timing the step with the per-head output certificate (kvq_decode_attn_cert)")
    p.add_argument("--recompute-frac", type=float, default=0.01,
                   help="certified step with recompute: tau_out set so that about this fraction of heads is flagged")
    p.add_argument("--no-adaptive", action="store_true",
                   help="skip timing the adaptive-precision step (kvq_decode_attn_adaptive)")
    p.add_argument("--tau-cov", type=float, default=0.995, help="adaptive step: coverage of the INT8 mass")
    p.add_argument("--tau-rank", type=float, default=0.1, help="adaptive step: discordant share that flags a head")
    p.add_argument("--tau-vc", type=float, default=float("inf"), help="adaptive step: value-promotion threshold")
    p.add_argument("--key-rotation", action="store_true",
                   help="Hadamard-rotated key codec (KVQ_CODEC_ROTATE_K); tolerances from a plain-codec cache of "
                        "the same data, so the fallback shares compare at a fixed tau")
    p.add_argument("--tier2", default="device", choices=["device", "host"],
                   help="FP16 originals in HBM, or in pinned host memory read in place over the host link")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one 1 GiB device copy (reference kernel for HBM counters)")
    return p.parse_args()


def kernel_source_hash():
    import quantized_decode_attention_kvq_amd.build as b
    h = hashlib.sha256()
    for f in sorted(b.sources()):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def decode_bytes(mask, B, Hq):
    """Algorithmic bytes of one decode over blocks with fallback mask `mask`."""
    import numpy as np
    m = np.asarray(mask)
    fk = (m & 1).astype(np.int64)
    fv = ((m >> 1) & 1).astype(np.int64)
    per_unit = 8 + np.where(fk, 16384, 8320) + np.where(fv, 16384, 4608)
    return int(per_unit.sum()) + 2 * B * Hq * 256


def append_bytes(B, Hkv, n=1):
    return B * Hkv * n * (512 + 128 + 2 + 64 + 8 + 8)


def traffic_from_counters(path=PROFILE_COUNTERS, kernel=None, workload=None, nbytes=None):
    """HBM bytes per launch of the profiled kernel (the decode step, or the
    bulk append for APPEND_COUNTERS): FETCH_SIZE + WRITE_SIZE, each scaled by
    the same counter's reading on a plain 1 GiB copy, from the committed
    rocprofv3 counter runs, or None when they are absent, were taken on other
    kernel sources, or (when given) on another kernel, workload or byte
    count per launch."""
    if not os.path.exists(path):
        return None
    try:
        c = json.load(open(path))
        if c.get("kernel_source_hash") != kernel_source_hash():
            return None
        if kernel is not None and c.get("kernel") != kernel:
            return None
        if workload is not None and c.get("workload") != workload:
            return None
        if nbytes is not None and int(c.get("algorithmic_bytes_per_launch", -1)) != int(nbytes):
            return None
        return float(c["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(w, d, tau_k, tau_v, sm, target_s):
    """The oracle (as it stands) on a bounded sample: whole-context decode for
    a subset of (batch, KV head) groups, timed on the host cores."""
    import numpy as np

    import oracle

    k16 = d["k16"].cpu().numpy()
    v16 = d["v16"].cpu().numpy()
    q = d["q"].cpu().numpy()
    groups = [(b, h) for b in range(w.B) for h in range(w.Hkv)]

    def sample(n, reps=1):
        idx = groups[:n]
        ks = np.stack([k16[b, h] for b, h in idx])[:, None]
        vs = np.stack([v16[b, h] for b, h in idx])[:, None]
        qs = np.stack([q[b, h * w.G:(h + 1) * w.G] for b, h in idx])
        oc = oracle.Cache(ks, vs, w.T)  # the quantized cache (setup, untimed)
        t0 = time.perf_counter()
        for _ in range(reps):
            _, mask = oc.attention(qs, sm, tau_k, tau_v)
        dt = time.perf_counter() - t0
        return dt, mask

    dt1, _ = sample(1)
    n = int(max(1, min(len(groups), target_s / max(dt1, 1e-3))))
    dt, mask = sample(n)
    reps = 1
    if n == len(groups) and dt < 0.5 * target_s:
        # the whole workload takes less than the target: repeat it
        reps = int(max(1, round(target_s / max(dt, 1e-3))))
        dt, mask = sample(n, reps)
    nbytes = decode_bytes(mask, n, w.G) * reps
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"fp64 decode of {n} of {len(groups)} (batch, KV head) groups at T={w.T} "
                      f"({n * w.G} query heads), {reps} pass(es), {dt:.2f} s; same byte accounting as the GPU line",
            "tokens_per_s_equiv": round(reps * n / len(groups) * w.B / dt, 3)}


def bench_quantize(args, w):
    """Quantize-on-append throughput: one step appends the workload's T new
    tokens of every KV head to an empty cache (bulk prefill).  Algorithmic
    bytes per token-head: 512 fp16 K and V bytes read; 128 key codes, 2 key
    scale bytes, 64 value-code bytes and 8 value-scale bytes written; plus 8
    bytes of block statistics per block."""
    import numpy as np
    import torch

    import quantized_decode_attention_kvq_amd as kvq
    import workloads

    d = workloads.make(w, "cuda")
    c = kvq.KVCache(w.B, w.Hkv, w.cap, k16=d["k16"], v16=d["v16"], key_rotation=args.key_rotation)
    del d
    stream = torch.cuda.current_stream()
    th = w.B * w.Hkv * w.T
    nbytes = th * (512 + 128 + 2 + 64 + 8) + w.B * w.Hkv * ((w.T + 63) // 64) * 8

    def step(ev=None):
        c.length = 0
        if ev is not None:
            ev[0].record(stream)
        kvq.kvq_quantize_append(c, w.T, stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    traffic = traffic_from_counters(APPEND_COUNTERS) if not args.key_rotation else None
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    kgbs = nbytes / (k_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "quantize-on-append (bulk prefill): GB/s (% of HBM peak), tokens/s",
        "value": round(gbs, 2), "unit": "GB/s", "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.B * w.T / (ms_step * 1e-3), 1), "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16 in, int8 K / int4 V codes out, fp64 error sums",
        "data": "synthetic (seeded normal fp16 K/V with 3 K outlier channels x20)",
        "config": {"workload": f"{w.name}: {w.T} new tokens x {w.Hkv} KV heads x D128, one bulk append",
                   "bytes_per_step": nbytes, "key_codec": "rotate_k" if args.key_rotation else "plain",
                   "k_err_median": float(c.k_err.flatten()[: w.B * w.Hkv * ((w.T + 63) // 64)].median())},
        "roofline": {"kernel": "quantize_append_kernel", "bound": "hbm", "achieved": round(kgbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": nbytes, "mean_launch_ms": round(k_ms, 5)},
    }), flush=True)


GRAPH_STEPS = 32  # layer steps per captured graph: a Llama-3-8B per-token graph holds 32 layers
WARM_S = 0.02  # untimed replays before the timed steps, in seconds of sustained load


def graph_steps(args):
    return min(args.steps, GRAPH_STEPS)


def timed_steps(args, R, step, stream):
    """Milliseconds per step over exactly args.steps steps (step(i, stream)
    launches step i on layer cache i % R), after args.warmup untimed ones and
    20 ms of untimed replays (the GPU's clock settles under sustained load):
    (host wall clock between synchronisations; HIP events recorded on the
    stream around a second pass of the same steps, queued behind a third,
    untimed one that keeps them from starting before they are submitted).
    With args.graph, the steps of up to 32 layers (cycling the R layer
    caches) are captured in one HIP graph, as a decoder's per-token graph
    holds its layers, plus one graph of the remaining steps, and replayed;
    otherwise every step is launched eagerly."""
    import torch

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    if args.graph:
        side = torch.cuda.Stream()
        n_g = graph_steps(args)

        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for r in range(n):
                    step(r, torch.cuda.current_stream())
            return g
        full = capture(n_g)
        rem = args.steps % n_g
        part = capture(rem) if rem else None
        torch.cuda.synchronize()

        def run_all():
            for _ in range(args.steps // n_g):
                full.replay()
            if part is not None:
                part.replay()
        # untimed: the graph's first replay, then replays for 20 ms, so that the
        # timed steps run at the clock the GPU settles at under sustained load
        # (it holds a lower one for the first milliseconds; a decoder serving
        # tokens runs this step continuously)
        full.replay()
        torch.cuda.synchronize()
        tw = time.perf_counter()
        while time.perf_counter() - tw < WARM_S:
            full.replay()
            torch.cuda.synchronize()
    else:
        def run_all():
            for i in range(args.steps):
                step(i, stream)
        tw = time.perf_counter()
        while time.perf_counter() - tw < WARM_S:
            run_all()
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_all()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps * 1e3
    # the same steps again between HIP events, queued behind one more untimed
    # pass of them: the first event is then taken once the host has submitted
    # the steps, so the span is the kernels' own (back to back in a graph),
    # not the host's submission latency before the first one, and the GPU is
    # under load throughout (an idle spin ahead of them let its clock drop,
    # and the timed steps then ran up to 15% slower than the wall-clock pass)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    strm = torch.cuda.current_stream()
    run_all()
    e0.record(strm)
    run_all()
    e1.record(strm)
    torch.cuda.synchronize()
    return wall, e0.elapsed_time(e1) / args.steps


def bench_certified(args, w, caches, ws, q, sm, tau_k, tau_v, ms_plain):
    """The same step with the per-head output certificate: the certifying
    decode kernel, the certificate merge and, for heads above tau_out, the
    gated FP16 recompute.  Timed from captured graphs like the plain step,
    once with tau_out = inf (certificate only) and once with tau_out set so
    that about --recompute-frac of the heads are recomputed."""
    import numpy as np
    import torch

    import quantized_decode_attention_kvq_amd as kvq

    R = len(caches)
    out = torch.empty_like(q)
    cert = torch.empty((w.B, w.Hq), dtype=torch.float32, device=q.device)
    rec = torch.empty((w.B, w.Hq), dtype=torch.uint8, device=q.device)

    def cstep(i, tau_out, strm):
        c = caches[i % R]
        c.length = w.T - 1
        kvq.kvq_decode_attn_cert(c, q, sm, tau_k, tau_v, tau_out, append=True, out=out, cert=cert,
                                 recomputed=rec, workspace=ws[i % R], stream=strm)

    stream = torch.cuda.current_stream()
    cstep(0, float("inf"), stream)
    torch.cuda.synchronize()
    cv = np.sort(cert.flatten().cpu().numpy())
    k = max(1, int(round(args.recompute_frac * cv.size)))
    tau_out = float(np.float32((cv[cv.size - k - 1] + cv[cv.size - k]) / 2)) if cv.size > k else -1.0

    ms_cert = timed_steps(args, R, lambda i, strm: cstep(i, float("inf"), strm), stream)[0]
    ms_rec = timed_steps(args, R, lambda i, strm: cstep(i, tau_out, strm), stream)[0]
    cstep(0, tau_out, stream)
    torch.cuda.synchronize()
    r = rec.cpu().numpy()
    groups = r.reshape(w.B, w.Hkv, w.G).any(axis=2)
    return {
        "api": "kvq_decode_attn_cert (append=True)",
        "ms_per_step_certificate_only": round(ms_cert, 5),
        "overhead_vs_plain_step": round(ms_cert / ms_plain - 1.0, 4),
        "tau_out": tau_out,
        "heads_recomputed_frac": round(float(r.mean()), 5),
        "kv_groups_recomputed_frac": round(float(groups.mean()), 5),
        "ms_per_step_with_recompute": round(ms_rec, 5),
        "certificate_median": float(np.median(cv)),
        "certificate_max": float(cv[-1]),
    }


def bench_adaptive(args, w, caches, q, sm, tau_k, tau_v, ms_plain):
    """The same step through kvq_decode_attn_adaptive (append, INT8 scoring
    pass, selection, certifying decode with the promoted tiles, certificate
    merge, ranking check, gated FP16 recompute), timed like the plain step."""
    import numpy as np
    import torch

    import quantized_decode_attention_kvq_amd as kvq

    R = len(caches)
    out = torch.empty_like(q)
    cert = torch.empty((w.B, w.Hq), dtype=torch.float32, device=q.device)
    rec = torch.empty((w.B, w.Hq), dtype=torch.uint8, device=q.device)
    kstar = torch.empty((w.B, w.Hq), dtype=torch.int32, device=q.device)
    ndisc = torch.empty((w.B, w.Hq), dtype=torch.int32, device=q.device)
    mask = torch.empty((w.B, w.Hkv, (w.T + 63) // 64), dtype=torch.uint8, device=q.device)
    wsa = [kvq.make_workspace(c, w.Hq, adaptive=True) for c in caches]

    def astep(i, strm, mask_out=None):
        c = caches[i % R]
        c.length = w.T - 1
        kvq.kvq_decode_attn_adaptive(c, q, sm, tau_k, tau_v, args.tau_cov, args.tau_vc, args.tau_rank,
                                     append=True, out=out, cert=cert, recomputed=rec, kstar=kstar, ndisc=ndisc,
                                     mask_out=mask_out, workspace=wsa[i % R], stream=strm)

    stream = torch.cuda.current_stream()
    astep(0, stream, mask)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    ks = kstar.cpu().numpy()
    r = rec.cpu().numpy()
    ms = timed_steps(args, R, lambda i, strm: astep(i, strm), stream)[0]
    nb = m.shape[-1]
    return {
        "api": "kvq_decode_attn_adaptive (append=True)",
        "tau_cov": args.tau_cov, "tau_rank": args.tau_rank,
        "tau_vc": args.tau_vc if np.isfinite(args.tau_vc) else "inf",
        "ms_per_step": round(ms, 5),
        "overhead_vs_plain_step": round(ms / ms_plain - 1.0, 4),
        "kstar_mean_frac": round(float(ks.mean()) / nb, 5),
        "key_fp16_blocks_frac": round(float((m & 1).mean()), 5),
        "value_fp16_blocks_frac": round(float(((m >> 1) & 1).mean()), 5),
        "heads_recomputed_frac": round(float(r.mean()), 5),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU runs are not part of it (the decode path would shard over "
              "(batch, KV head) groups with no communication)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_decode_attention_kvq_amd as kvq
    import workloads

    torch.cuda.set_device(0)
    w = workloads.WORKLOADS[args.workload]
    if args.q_heads:
        w = w.scaled(Hq=args.q_heads)
    if w.name == "bulk_quantize":
        return bench_quantize(args, w)
    dev = "cuda"
    sm = kvq.DEFAULT_SM_SCALE
    kernel = {"auto": kvq.KERNEL_AUTO, "valu": kvq.KERNEL_VALU, "mfma": kvq.KERNEL_MFMA,
              "mfma_table": kvq.KERNEL_MFMA_TABLE}[args.kernel]

    d = workloads.make(w, dev)
    # layer caches: same data, distinct HBM allocations
    tier2 = 2 * d["k16"].numel() * 2
    tier1 = tier2 * 0.395
    R = args.replicas or int(max(2, np.ceil(2e9 / tier1)))
    caches = []
    for r in range(R):
        if args.tier2 == "host":
            c = kvq.KVCache(w.B, w.Hkv, w.cap, device=dev, tier2="host", key_rotation=args.key_rotation)
            c.k16.copy_(d["k16"])
            c.v16.copy_(d["v16"])
        else:
            k16 = d["k16"] if r == 0 else d["k16"].clone()
            v16 = d["v16"] if r == 0 else d["v16"].clone()
            c = kvq.KVCache(w.B, w.Hkv, w.cap, device=dev, k16=k16, v16=v16, key_rotation=args.key_rotation)
        kvq.kvq_quantize_append(c, w.T - 1)  # prefill; the step appends token T-1
        caches.append(c)
    q = d["q"].contiguous()

    # tolerances: ~fallback_frac of the blocks per bound, from the library's own bounds
    c0 = caches[0]
    if args.key_rotation:
        # tolerances of the plain codec on the same data (a fixed tau)
        c0 = kvq.KVCache(w.B, w.Hkv, w.cap, device=dev, k16=caches[0].k16, v16=caches[0].v16)
        kvq.kvq_quantize_append(c0, w.T - 1)
    kvq.kvq_quantize_append(c0, 1)
    kb, vb, _ = kvq.kvq_bounds(c0, q, sm, 0.0, 0.0, want=("kb", "vb"))
    kbn, vbn = kb.flatten().float().cpu().numpy(), vb.flatten().float().cpu().numpy()

    def tau(vals, frac):
        if frac <= 0:
            return float("inf")
        v = np.sort(vals[np.isfinite(vals)])
        k = max(1, int(round(frac * v.size)))
        return float(np.float32((v[v.size - k - 1] + v[v.size - k]) / 2))

    frac = w.fallback_frac if args.fallback_frac is None else args.fallback_frac
    tau_k, tau_v = tau(kbn, frac), tau(vbn, frac)
    if args.taus:
        tau_k, tau_v = (float(x) for x in args.taus.split(","))
    c0.length = w.T - 1
    if args.key_rotation:
        del c0, kb, vb
        torch.cuda.empty_cache()

    out = torch.empty_like(q)
    mask = torch.empty((w.B, w.Hkv, (w.T + 63) // 64), dtype=torch.uint8, device=dev)
    ws = [kvq.make_workspace(c, w.Hq) for c in caches]
    stream = torch.cuda.current_stream()

    def step(i, ev=None, strm=None):
        strm = stream if strm is None else strm
        c = caches[i % R]
        c.length = w.T - 1
        if args.unfused:
            kvq.kvq_quantize_append(c, 1, strm)
        call = kvq.kvq_decode_attn if args.unfused else kvq.kvq_append_decode
        call(c, q, sm, tau_k, tau_v, out=out, mask_out=mask if i == 0 else None, workspace=ws[i % R],
             stream=strm, kernel=kernel, splits=args.splits)

    step(0)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    dec_bytes = decode_bytes(m, w.B, w.Hq)
    step_bytes = dec_bytes + append_bytes(w.B, w.Hkv)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed loop: exactly `steps` steps between synchronisations, launched
    # eagerly or replayed from captured HIP graphs (the fused step of up to 32
    # layers in one graph, cycling the R layer caches, as a decoder's
    # per-token graph holds every layer)
    ms_step, ms_step_ev = timed_steps(args, R, lambda i, strm: step(i, strm=strm), stream)

    # the dominant kernel's launch time.  The fused step on the matrix-core
    # kernel is that one kernel (its last workgroup per group merges the
    # splits), so the events around the timed loop time it: per launch,
    # their span / steps (which counts the gaps between graph-launched
    # kernels too).  Otherwise the step holds more kernels: the same steps
    # again, eagerly, with events before each call, after its split-K kernel
    # (recorded by the library) and after the call.
    one_kernel = not args.unfused and args.kernel != "valu" and w.G <= 16
    if one_kernel:
        split_ms = call_ms = ms_step_ev
        merge_ms = 0.0
        launch_source = (f"HIP events on the stream around a second pass of the timed loop's {args.steps} "
                         f"{'graph-replayed' if args.graph else 'eager'} steps, queued behind a third, untimed pass "
                         "(so the span starts at the first kernel, not at the host's submission, and the GPU stays "
                         "under load); one kernel per step")
    else:
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
        for e3 in evs:
            for e in e3:
                e.record(stream)
        torch.cuda.synchronize()
        for i in range(args.steps):
            c = caches[i % R]
            c.length = w.T - 1
            if args.unfused:
                kvq.kvq_quantize_append(c, 1, stream)
            evs[i][0].record(stream)
            call = kvq.kvq_decode_attn if args.unfused else kvq.kvq_append_decode
            call(c, q, sm, tau_k, tau_v, out=out, workspace=ws[i % R], stream=stream, kernel=kernel,
                 splits=args.splits, split_done=evs[i][1])
            evs[i][2].record(stream)
        torch.cuda.synchronize()
        split_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        merge_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        call_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in evs]))
        launch_source = f"HIP events on the stream around each of {args.steps} eager decode calls"


    # the certificate needs the matrix-core kernel (group sizes up to 16)
    no_cert = args.no_certify or args.kernel == "valu" or w.G > 16
    certified = None if no_cert else bench_certified(args, w, caches, ws, q, sm, tau_k, tau_v, ms_step)
    adaptive = None if (no_cert or args.no_adaptive or (w.T + 63) // 64 > 8192) else \
        bench_adaptive(args, w, caches, q, sm, tau_k, tau_v, ms_step)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    # the fused kernel appends, reads the tiles, statistics and q and writes
    # the output; a split-K kernel followed by a merge kernel leaves the
    # output to the merge
    split_bytes = step_bytes if one_kernel else dec_bytes - w.B * w.Hq * 256
    split_gbs = split_bytes / (split_ms * 1e-3) / 1e9
    nblk = (w.T + 63) // 64
    kname = "decode_valu_kernel" if args.kernel == "valu" or w.G > 16 else (
        "decode_stream_kernel" if nblk <= 2048 and args.kernel != "mfma_table" else "decode_mfma_kernel")
    traffic = traffic_from_counters(kernel=kname, workload=w.name, nbytes=split_bytes)
    line = {
        "metric": "quantized-KV decode attention: effective KV GB/s (% of HBM peak), tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.B / (ms_step * 1e-3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 K / int4 V codes, fp16 q and fallback tiles, fp32 accumulate",
        "data": "synthetic (seeded normal fp16 K/V/q with per-head K outlier channels)",
        "config": {
            "workload": f"{w.name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} D128 T{w.T}, one decode step "
                        "(append 1 token + certified attention) of one layer",
            "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "context": w.T,
            "fallback_blocks_key": round(float((m & 1).mean()), 5),
            "fallback_blocks_value": round(float(((m >> 1) & 1).mean()), 5),
            "tau_k": tau_k if np.isfinite(tau_k) else "inf", "tau_v": tau_v if np.isfinite(tau_v) else "inf",
            "layers_cycled": R,
            "kernel": args.kernel, "splits": args.splits, "hip_graph": bool(args.graph), "steps_per_graph": graph_steps(args) if args.graph else None,
            "fused_append": not args.unfused,
            "tier2": args.tier2,
            "key_codec": "rotate_k (tolerances of the plain codec)" if args.key_rotation else "plain",
            "bytes_per_step": step_bytes,
        },
        "roofline": {
            "kernel": kname + (" (append, bounds, masks, tiles, online softmax, split merge)" if one_kernel
                               else " (split-K: bounds, masks, tiles, online softmax)"),
            "bound": "hbm",
            "achieved": round(split_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(split_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": split_bytes,
            "mean_launch_ms": round(split_ms, 5),
            "launch_time_source": launch_source,
            "merge_kernel_ms": round(merge_ms, 5),
            "decode_call_ms": round(call_ms, 5),
            "decode_call_gbs": round(dec_bytes / (call_ms * 1e-3) / 1e9, 2),
        },
    }
    if certified is not None:
        line["certified_step"] = certified
    if adaptive is not None:
        line["adaptive_step"] = adaptive
    if args.tier2 == "host":
        # bytes each step reads from host memory: fallback tiles and the
        # appended rows (the rest of the step reads tier 1 in HBM)
        host_bytes = int(((m & 1) != 0).sum() + ((m & 2) != 0).sum()) * 16384 + w.B * w.Hkv * 512
        line["tier2_host"] = {"bytes_per_step": host_bytes,
                              "host_link_gbs": round(host_bytes / (ms_step * 1e-3) / 1e9, 2)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, d, tau_k, tau_v, sm, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
