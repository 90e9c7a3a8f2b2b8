#!/usr/bin/env python3
"""Benchmark of the linear-attention hot path on one MI355X.

Headline (`value`): causal chunked forward, bf16 in / bf16 out, fp32 accumulate,
B=8, H=8, N=65536, d_k=d_v=64, C=64, in tokens/s (B*N per step / step time).
A step is one la_fwd_causal call over the whole batch with the inputs already
resident in HBM.  Alongside it, on the same JSON line:
  roofline      achieved HBM GB/s of the forward (algorithmic bytes: q, k, v read
                once, o written once = 512 B per token-head) against 8 TB/s,
                timed with HIP events on the stream the kernels run on;
  mfma          the chunked method's own flops (4*C*d + 4*d^2 per token-head)
                against dense bf16 MFMA peak (2.5166 PFLOP/s);
  decode        3072 sequential la_decode_step calls at B=256, H=8, d=32, fp32
                (pixel-by-pixel generation of 32x32x3 images), replayed as one
                HIP graph: steps/s and algorithmic bytes (state read and written,
                q, k, v read, o written) against 8 TB/s;
  extra         the length sweep N = 2^9 .. 2^16 (forward and backward time,
                peak device bytes per call), the non-causal workload
                (B=4, H=8, N=4096, d=64), the forward and backward at
                B=8, H=16, N=8192, d=128, C=64, the decay forward and the
                forward with random features (m = 64) at the headline shape;
  cpu_baseline  the fp64 CPU oracle timed on the host cores on a bounded sample
                of the headline workload.
Inputs are seeded synthetic normals.  One GPU only.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6
METRIC = "causal LA fwd tokens/s (N=65536,d=64) + % MFMA peak; decode steps/s, % HBM BW"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The first few dozen calls after the inputs are written run up to 10% slower
    # (clocks and caches settle); the untimed warmup covers them.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extra", action="store_true", help="skip the sweep / non-causal / backward lines")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only", choices=["fwd", "decode", "noncausal", "bwd", "decay", "prf", "decay_bwd", "prf_bwd",
                                       "copy"], default=None,
                    help="run one leg only (for profiler runs); prints its own JSON line")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the plain copy leg")
    return ap.parse_args()


def profiled_traffic(summary: str):
    """HBM bytes per call recorded in profiles/<summary> from rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes, or None when the kernel sources changed since they were taken."""
    import glob
    import hashlib

    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_call", "kernel_source_sha256"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "linear_attention_elu_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256") != h.hexdigest() or "traffic_bytes_per_call" not in fields:
        return None
    return int(float(fields["traffic_bytes_per_call"]))


def time_calls(fn, steps, warmup, stream):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per call


def bench_fwd(steps, warmup, dev, B=8, H=8, N=65536, d=64, C=64, seed=0):
    import torch

    import linear_attention_elu_amd as la
    from linear_attention_elu_amd import inputs

    host = inputs.attention_inputs(B, H, N, d, d, seed=seed)
    q, k, v = (inputs.to_torch(host[n], torch.bfloat16, dev) for n in ("q", "k", "v"))
    del host
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, la.la_fwd_causal_workspace_bytes(B, H, N, d, d, C)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        la.la_fwd_causal(q, k, v, o=o, C=C, ws=ws, want_den=False)

    ms = time_calls(step, steps, warmup, stream)
    token_heads = B * H * N
    bytes_alg = token_heads * 4 * d * 2          # q, k, v read, o written, bf16
    flops_alg = token_heads * (4 * C * d + 4 * d * d)
    return {
        "ms": ms, "tokens_per_s": B * N / (ms * 1e-3), "bytes": bytes_alg, "flops": flops_alg,
        "gbs": bytes_alg / (ms * 1e-3) / 1e9, "tflops": flops_alg / (ms * 1e-3) / 1e12,
    }


def bench_sweep_point(dev, N, steps, warmup, B=8, H=8, d=64, C=64, seed=0):
    """One length of the sweep 2^9 .. 2^16 (velog review 4.3 times the forward and
    the backward and reports peak memory at each length): forward and backward
    time, and the device bytes resident during each call -- inputs, outputs and
    workspace; the allocator's peak over the timed calls is checked to equal
    them (the library allocates nothing)."""
    import torch

    import linear_attention_elu_amd as la
    from linear_attention_elu_amd import inputs

    stream = torch.cuda.current_stream(dev)

    def resident_during(fn, base):
        torch.cuda.synchronize()
        held = torch.cuda.memory_allocated(dev) - base
        torch.cuda.reset_peak_memory_stats(dev)
        ms = time_calls(fn, steps, warmup, stream)
        peak = torch.cuda.max_memory_allocated(dev) - base
        assert peak == held, (peak, held)
        return ms, held

    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)
    host = inputs.attention_inputs(B, H, N, d, d, seed=seed, with_grad=True)
    q, k, v = (inputs.to_torch(host[n], torch.bfloat16, dev) for n in ("q", "k", "v"))
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, la.la_fwd_causal_workspace_bytes(B, H, N, d, d, C)), dtype=torch.uint8, device=dev)
    ms, fwd_bytes = resident_during(lambda: la.la_fwd_causal(q, k, v, o=o, C=C, ws=ws, want_den=False), base)
    del o, ws
    dO = inputs.to_torch(host["dO"], torch.bfloat16, dev)
    del host
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    wsb = torch.empty(max(1, la.la_bwd_causal_workspace_bytes(B, H, N, d, d, C)), dtype=torch.uint8, device=dev)
    bms, bwd_bytes = resident_during(lambda: la.la_bwd_causal(q, k, v, dO, dq=dq, dk=dk, dv=dv, C=C, ws=wsb), base)
    th = B * H * N
    fby, bby = th * 4 * d * 2, th * 7 * d * 2
    flops = th * (4 * C * d + 4 * d * d)
    return {"us": round(ms * 1e3, 2), "tokens_per_s": round(B * N / (ms * 1e-3), 1),
            "hbm_frac": round(fby / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "bwd_us": round(bms * 1e3, 2), "bwd_hbm_frac": round(bby / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fwd_device_bytes": int(fwd_bytes), "bwd_device_bytes": int(bwd_bytes)}


def bench_fwd_decay(steps, warmup, dev, B=8, H=8, N=65536, d=64, C=64, seed=0):
    """The headline shape with a fixed decay per head, 1 - 2^-(3 + h)."""
    import torch

    import linear_attention_elu_amd as la
    from linear_attention_elu_amd import inputs

    host = inputs.attention_inputs(B, H, N, d, d, seed=seed)
    q, k, v = (inputs.to_torch(host[n], torch.bfloat16, dev) for n in ("q", "k", "v"))
    del host
    g = torch.tensor([1.0 - 2.0 ** -(3 + h) for h in range(H)], dtype=torch.float32, device=dev)
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, la.la_fwd_causal_workspace_bytes(B, H, N, d, d, C)), dtype=torch.uint8, device=dev)
    ms = time_calls(lambda: la.la_fwd_causal_decay(q, k, v, g, o=o, C=C, ws=ws, want_den=False), steps, warmup,
                    torch.cuda.current_stream(dev))
    by = B * H * N * 4 * d * 2
    return {"workload": f"causal_decay_fwd_bf16_B{B}_H{H}_N{N}_d{d}_C{C}", "us": round(ms * 1e3, 2),
            "tokens_per_s": round(B * N / (ms * 1e-3), 1), "achieved_GBs": round(by / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def bench_fwd_prf(steps, warmup, dev, B=8, H=8, N=65536, d=64, m=64, C=64, seed=0):
    """The headline shape with Performer's positive random features (m = 64
    directions per head, orthogonal blocks): q, k ~ N(0, d^-1/2), as the map is
    used.  Algorithmic bytes are the call's inputs and output (q, k, v read, o
    written: 512 B per token-head; W is 8 KB per head).  At this shape the
    features are formed in the chunk kernels as q and k are loaded; other shapes
    pass them through the workspace (2 x m x 2 B written and read per
    token-head), which the fraction would not count as useful bytes."""
    import torch

    import linear_attention_elu_amd as la
    from linear_attention_elu_amd import inputs

    host = inputs.attention_inputs(B, H, N, d, d, seed=seed, qk_std=d ** -0.25)
    q, k, v = (inputs.to_torch(host[n], torch.bfloat16, dev) for n in ("q", "k", "v"))
    del host
    W = inputs.to_torch(inputs.random_features(H, m, d, seed=seed + 1), torch.bfloat16, dev)
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, la.la_fwd_causal_fm_workspace_bytes(B, H, N, d, d, C, "prf", m, torch.bfloat16)),
                     dtype=torch.uint8, device=dev)
    ms = time_calls(lambda: la.la_fwd_causal_fm(q, k, v, "prf", W, o=o, C=C, ws=ws, want_den=False), steps, warmup,
                    torch.cuda.current_stream(dev))
    by = B * H * N * 4 * d * 2
    return {"workload": f"causal_prf_fwd_bf16_B{B}_H{H}_N{N}_d{d}_m{m}_C{C}", "us": round(ms * 1e3, 2),
            "tokens_per_s": round(B * N / (ms * 1e-3), 1), "achieved_GBs": round(by / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def bench_decode(dev, T=3072, B=256, H=8, d=32, seed=0, reps=5):
    import torch

    import linear_attention_elu_amd as la
    from linear_attention_elu_amd import inputs

    host = inputs.decode_inputs(T, B, H, d, d, seed=seed)
    q, k, v = (torch.from_numpy(host[n]).to(dev) for n in ("q", "k", "v"))
    del host
    S = torch.zeros(B, H, d, d, device=dev)
    z = torch.zeros(B, H, d, device=dev)
    out = torch.empty(T, B, H, d, device=dev)

    # warm the library and the kernel once outside capture
    la.la_decode_step(S, z, q[0], k[0], v[0], o=out[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for t in range(T):
                la.la_decode_step(S, z, q[t], k[t], v[t], o=out[t])
    torch.cuda.synchronize()
    times = []
    stream = torch.cuda.current_stream(dev)
    for r in range(reps + 1):
        S.zero_()
        z.zero_()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        g.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        if r > 0:  # the first replay is a warm-up
            times.append(start.elapsed_time(stop))
    ms = statistics.median(times)
    steps_per_s = T / (ms * 1e-3)
    per_step_bytes = B * H * (2 * d * d * 4 + 2 * d * 4 + 3 * d * 4 + d * 4)
    gbs = per_step_bytes * steps_per_s / 1e9
    floor_us = graph_node_floor_us(dev, T, reps)
    # a step can take no less than the node floor plus its bytes at the HBM peak
    ceiling = per_step_bytes / (floor_us * 1e-6 + per_step_bytes / (HBM_PEAK_GBS * 1e9)) / 1e9 / HBM_PEAK_GBS
    return {
        "workload": f"decode_fp32_T{T}_B{B}_H{H}_d{d}", "steps": T, "ms_total": round(ms, 4),
        "us_per_step": round(ms * 1e3 / T, 4), "steps_per_s": round(steps_per_s, 1),
        "tokens_per_s": round(steps_per_s * B, 1), "bytes_per_step": per_step_bytes,
        "achieved_GBs": round(gbs, 1), "hbm_peak_GBs": HBM_PEAK_GBS, "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "timing": "one HIP graph of all steps, median of %d replays, launch gaps included" % reps,
        "graph_node_floor_us": round(floor_us, 3), "hbm_frac_ceiling_one_launch_per_step": round(ceiling, 4),
    }


def graph_node_floor_us(dev, T, reps):
    """Time per node of a HIP graph of T one-element fills: what one kernel launch
    per decode step costs before the kernel does any work."""
    import torch

    x = torch.zeros(1, device=dev)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        x.fill_(1.0)
        with torch.cuda.graph(g, stream=side):
            for _ in range(T):
                x.fill_(1.0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    times = []
    for r in range(reps + 1):
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        g.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        if r > 0:
            times.append(start.elapsed_time(stop))
    return statistics.median(times) * 1e3 / T


def bench_noncausal(dev, steps=100, warmup=20, B=4, H=8, N=4096, d=64, seed=0):
    import torch

    import linear_attention_elu_amd as la
    from linear_attention_elu_amd import inputs

    host = inputs.attention_inputs(B, H, N, d, d, seed=seed)
    q, k, v = (inputs.to_torch(host[n], torch.bfloat16, dev) for n in ("q", "k", "v"))
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, la.la_fwd_noncausal_workspace_bytes(B, H, N, d, d)), dtype=torch.uint8, device=dev)
    ms = time_calls(lambda: la.la_fwd_noncausal(q, k, v, o=o, ws=ws), steps, warmup, torch.cuda.current_stream(dev))
    by = B * H * N * 4 * d * 2
    res = {"workload": f"noncausal_fwd_bf16_B{B}_H{H}_N{N}_d{d}", "us": round(ms * 1e3, 3),
           "achieved_GBs": round(by / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # its backward at the same shape: q, k, v, dO read, dq, dk, dv written
    dO = inputs.to_torch(inputs.attention_inputs(B, H, N, d, d, seed=seed, with_grad=True)["dO"], torch.bfloat16, dev)
    wsb = torch.empty(max(1, la.la_bwd_noncausal_workspace_bytes(B, H, N, d, d)), dtype=torch.uint8, device=dev)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    bms = time_calls(lambda: la.la_bwd_noncausal(q, k, v, dO, dq=dq, dk=dk, dv=dv, ws=wsb), steps, warmup,
                     torch.cuda.current_stream(dev))
    bby = B * H * N * 7 * d * 2
    res.update({"bwd_us": round(bms * 1e3, 3), "bwd_GBs": round(bby / (bms * 1e-3) / 1e9, 1),
                "bwd_hbm_frac": round(bby / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    return res


def bench_bwd(dev, steps=20, warmup=20, B=8, H=16, N=8192, d=128, C=64, seed=0):
    import torch

    import linear_attention_elu_amd as la
    from linear_attention_elu_amd import inputs

    host = inputs.attention_inputs(B, H, N, d, d, seed=seed, with_grad=True)
    q, k, v, dO = (inputs.to_torch(host[n], torch.bfloat16, dev) for n in ("q", "k", "v", "dO"))
    del host
    stream = torch.cuda.current_stream(dev)
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    den = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    wsf = torch.empty(max(1, la.la_fwd_causal_workspace_bytes(B, H, N, d, d, C)), dtype=torch.uint8, device=dev)
    fwd_ms = time_calls(lambda: la.la_fwd_causal(q, k, v, o=o, den=den, C=C, ws=wsf), steps, warmup, stream)
    res = {"workload": f"causal_fwd_bwd_bf16_B{B}_H{H}_N{N}_d{d}_C{C}", "fwd_us": round(fwd_ms * 1e3, 2)}
    fwd_bytes = B * H * N * (4 * d * 2 + 4)
    res["fwd_GBs"] = round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1)
    try:
        wsb = torch.empty(max(1, la.la_bwd_causal_workspace_bytes(B, H, N, d, d, C)), dtype=torch.uint8, device=dev)
        dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
        bwd_ms = time_calls(lambda: la.la_bwd_causal(q, k, v, dO, dq=dq, dk=dk, dv=dv, C=C, ws=wsb),
                            steps, warmup, stream)
        bwd_bytes = B * H * N * 7 * d * 2  # q k v dO read; dq dk dv written
        res.update({"bwd_us": round(bwd_ms * 1e3, 2), "bwd_GBs": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9, 1),
                    "bwd_hbm_frac": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    except la.LAError as e:
        res["bwd"] = f"not available: {e}"
    return res


def bench_decay_bwd(dev, steps=20, warmup=20, B=8, H=16, N=8192, d=128, C=64, seed=0):
    """Forward and backward with a fixed decay per head (1 - 2^-(3 + h/2)) at the
    backward workload's shape.  Bytes as in bench_bwd (den is not stored)."""
    import torch

    import linear_attention_elu_amd as la
    from linear_attention_elu_amd import inputs

    host = inputs.attention_inputs(B, H, N, d, d, seed=seed, with_grad=True)
    q, k, v, dO = (inputs.to_torch(host[n], torch.bfloat16, dev) for n in ("q", "k", "v", "dO"))
    del host
    stream = torch.cuda.current_stream(dev)
    g = torch.tensor([1.0 - 2.0 ** -(3 + h / 2) for h in range(H)], dtype=torch.float32, device=dev)
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    wsf = torch.empty(max(1, la.la_fwd_causal_workspace_bytes(B, H, N, d, d, C)), dtype=torch.uint8, device=dev)
    fwd_ms = time_calls(lambda: la.la_fwd_causal_decay(q, k, v, g, o=o, C=C, ws=wsf, want_den=False), steps, warmup,
                        stream)
    wsb = torch.empty(max(1, la.la_bwd_causal_workspace_bytes(B, H, N, d, d, C)), dtype=torch.uint8, device=dev)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    bwd_ms = time_calls(lambda: la.la_bwd_causal_decay(q, k, v, dO, g, dq=dq, dk=dk, dv=dv, C=C, ws=wsb),
                        steps, warmup, stream)
    fwd_bytes, bwd_bytes = B * H * N * 4 * d * 2, B * H * N * 7 * d * 2
    return {"workload": f"causal_decay_fwd_bwd_bf16_B{B}_H{H}_N{N}_d{d}_C{C}", "fwd_us": round(fwd_ms * 1e3, 2),
            "fwd_hbm_frac": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bwd_us": round(bwd_ms * 1e3, 2), "bwd_hbm_frac": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def bench_prf_bwd(dev, steps=5, warmup=3, B=8, H=8, N=65536, d=64, m=64, C=64, seed=0):
    """Backward with Performer's random features (m = 64) at the headline shape.
    Algorithmic bytes are the call's (q, k, v, dO read; dq, dk, dv written: 7 d x 2 B
    per token-head); the features and their gradients pass through the workspace
    in fp32, which the fraction does not count as useful bytes."""
    import torch

    import linear_attention_elu_amd as la
    from linear_attention_elu_amd import inputs

    host = inputs.attention_inputs(B, H, N, d, d, seed=seed, with_grad=True, qk_std=d ** -0.25)
    q, k, v, dO = (inputs.to_torch(host[n], torch.bfloat16, dev) for n in ("q", "k", "v", "dO"))
    del host
    W = inputs.to_torch(inputs.random_features(H, m, d, seed=seed + 1), torch.bfloat16, dev)
    ws = torch.empty(max(1, la.la_bwd_causal_fm_workspace_bytes(B, H, N, d, d, C, "prf", m, torch.bfloat16)),
                     dtype=torch.uint8, device=dev)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    ms = time_calls(lambda: la.la_bwd_causal_fm(q, k, v, dO, "prf", W, dq=dq, dk=dk, dv=dv, C=C, ws=ws), steps, warmup,
                    torch.cuda.current_stream(dev))
    by = B * H * N * 7 * d * 2
    return {"workload": f"causal_prf_bwd_bf16_B{B}_H{H}_N{N}_d{d}_m{m}_C{C}", "us": round(ms * 1e3, 2),
            "hbm_frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "workspace_bytes": ws.numel()}


def bench_copy(dev, mib, steps=10, warmup=2):
    """A plain device copy of known size (the reference for HBM counters)."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms = time_calls(lambda: dst.copy_(src), steps, warmup, torch.cuda.current_stream(dev))
    by = 2 * n * 4
    return {"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "us": round(ms * 1e3, 2),
            "GBs": round(by / (ms * 1e-3) / 1e9, 1)}


def cpu_baseline(B=8, H=8, N=65536, d=64, seed=0, budget_s=15.0):
    """The fp64 oracle on a bounded sample of the headline workload: whole
    sequences (all N tokens) of the first few heads, as many as fit the budget."""
    import numpy as np

    import oracle
    from linear_attention_elu_amd import inputs

    host = inputs.attention_inputs(B, H, N, d, d, seed=seed)
    q = host["q"].reshape(B * H, N, d)
    k = host["k"].reshape(B * H, N, d)
    v = host["v"].reshape(B * H, N, d)
    threads = oracle.num_threads()
    # calibrate on one head, then take as many heads as fit the budget (at least one)
    t0 = time.perf_counter()
    oracle.fwd_causal(q[:1, None].astype(np.float64), k[:1, None].astype(np.float64), v[:1, None].astype(np.float64))
    t1 = time.perf_counter() - t0
    per_round = t1  # a round of `threads` heads takes about one head's time
    rounds = max(1, int(budget_s / max(per_round, 1e-3)))
    heads = int(min(B * H, max(1, rounds * threads)))
    sl = slice(0, heads)
    t0 = time.perf_counter()
    oracle.fwd_causal(q[sl, None].astype(np.float64), k[sl, None].astype(np.float64), v[sl, None].astype(np.float64))
    dt = time.perf_counter() - t0
    tokens_equiv = heads * N / H  # a token carries H heads
    return {"value": round(tokens_equiv / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {B * H} (batch, head) sequences of N={N}, d=64, fp64 recurrent form; "
                      f"{dt:.1f} s wall; tokens counted as heads*N/H"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every (batch, head) is independent: shard B*H across GPUs with no communication).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import linear_attention_elu_amd as la

    la.load()  # fail loudly if the library is not built
    dev = torch.device("cuda:0")

    if args.only:
        log(f"only leg: {args.only}")
        if args.only == "fwd":
            r = bench_fwd(args.steps, args.warmup, dev)
        elif args.only == "decode":
            r = bench_decode(dev, reps=max(1, args.steps // 10))
        elif args.only == "noncausal":
            r = bench_noncausal(dev, args.steps, args.warmup)
        elif args.only == "bwd":
            r = bench_bwd(dev, args.steps, args.warmup)
        elif args.only == "decay":
            r = bench_fwd_decay(args.steps, args.warmup, dev)
        elif args.only == "prf":
            r = bench_fwd_prf(args.steps, args.warmup, dev)
        elif args.only == "decay_bwd":
            r = bench_decay_bwd(dev, args.steps, args.warmup)
        elif args.only == "prf_bwd":
            r = bench_prf_bwd(dev, args.steps, args.warmup)
        else:
            r = bench_copy(dev, args.copy_mib, args.steps, args.warmup)
        print(json.dumps({"only": args.only, **r}))
        return

    log("headline: causal fwd B=8 H=8 N=65536 d=64 C=64 bf16")
    f = bench_fwd(args.steps, args.warmup, dev)
    res = {
        "metric": METRIC,
        "value": round(f["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal_fwd_bf16_B8_H8_N65536_d64_C64", "B": 8, "H": 8, "N": 65536,
                   "d_k": 64, "d_v": 64, "C": 64, "out": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(f["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(f["gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic("causal_fwd_bf16_B8_H8_N65536_d64_C64.md"),
                     "traffic_unit": "HBM bytes per la_fwd_causal call (rocprofv3 counters, calibrated)",
                     "kernel": "la_fwd_causal (segment aggregate + segment scan + chunk loop)",
                     "bytes_per_launch": f["bytes"]},
        "mfma": {"achieved": round(f["tflops"], 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(f["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4),
                 "ceiling_at_hbm_peak": round((f["flops"] / f["bytes"]) * HBM_PEAK_GBS / 1e3 / BF16_MFMA_PEAK_TFLOPS, 4),
                 "flops_per_launch": f["flops"]},
    }
    log(f"fwd {f['ms'] * 1e3:.1f} us/step, {f['gbs']:.0f} GB/s")
    # what a plain device copy reaches on this part, next to the spec peak (context only)
    cp = bench_copy(dev, 1024, steps=10, warmup=3)
    res["hbm_context"] = {"device_copy_GBs": cp["GBs"], "spec_peak_GBs": HBM_PEAK_GBS,
                          "copy": "1 GiB read + 1 GiB written per copy, torch copy_ on the device"}
    if not args.no_decode:
        log("decode: 3072 steps, graph replay")
        res["decode"] = bench_decode(dev)
        res["decode"]["traffic"] = profiled_traffic("decode_fp32_B256_H8_d32.md")
        log(f"decode {res['decode']['us_per_step']} us/step")
    if not args.no_extra:
        log("extra: length sweep, non-causal, fwd+bwd")
        sweep = {}
        for e in range(9, 17):
            sweep[str(2 ** e)] = bench_sweep_point(dev, 2 ** e, max(5, args.steps), 20)
        res["extra"] = {"causal_sweep_B8_H8_d64_C64": sweep, "noncausal": bench_noncausal(dev),
                        "fwd_bwd": bench_bwd(dev), "causal_decay": bench_fwd_decay(args.steps, args.warmup, dev),
                        "causal_prf": bench_fwd_prf(args.steps, args.warmup, dev),
                        "decay_fwd_bwd": bench_decay_bwd(dev), "causal_prf_bwd": bench_prf_bwd(dev)}
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on host cores")
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
