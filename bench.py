"""Benchmark of the gated bidirectional linear-attention mixer on one MI355X.

One step = one whole pass of the hot path over one batch: the state half
(state kernel + cross-chunk reduction, reading k and v) and the output half
(output kernel, reading q and g, writing out), launched through the C ABI on
torch's current stream with inputs already resident in HBM.  Passes cycle
through three copies of the inputs, so no pass finds its inputs left in the
256 MB last-level cache by the pass before (the forward, block-causal and
backward benches).

Prints ONE JSON line.  `value` is tokens/s per layer (B*N tokens per step).
`value` and `ms_per_step` come from K uninstrumented passes of
gla_forward_ws (wall clock, synchronised on both sides).  `roofline`
reports the output kernel (the largest byte stream: q, g read and out
written, 6*D bytes per (token, head)) from HIP events recorded around
gla_output_ws, on the stream it runs on, in max(50, K) further passes;
`state_roofline` does the same for the state half (k, v read, 4*D bytes per
(token, head)); `traffic` is the output kernel's HBM bytes per launch from
the committed rocprofv3 byte counters (profiles/), or null when the kernel
source differs from the one those counters were taken on.
`all_configs` holds, for each of the five layer shapes, the median of
max(50, K) event-timed passes, warm and after a 512 MiB read that evicts
the last-level cache before each pass (the honest figure on the small
shapes, whose tensors would otherwise be read from that cache).
`streaming_ceiling` is what plain 16-byte non-temporal streaming reaches on
the same GPU, in the state half's mix (two reads) and the output half's
(two reads, one write), and each shape's `frac_of_streaming_ceiling` the
pass time those rates imply over its measured median.
`cpu_baseline` times the fp64 oracle on a sample of the workload's heads
(about ten seconds of CPU work) and scales to the whole workload.

`--block-frames F` times the block-causal form instead, `--softmax` the
gated softmax anchor attention (an MFMA-bound roofline in TFLOP/s) and
`--backward` the mixer's backward pass and `--proj` the projection prologue
fused with the mixer (an MFMA-bound roofline in TFLOP/s).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gated linear-attn tokens/s per layer (5B 720p shape); achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = "5b_720p_193f"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(w, q, k, v, g, min_seconds=10.0):
    """Times the fp64 oracle on the first `hs` heads of batch element 0 (one
    head per oracle thread), repeated until about `min_seconds` of CPU work,
    and scales the per-head time to the whole workload (heads are
    independent and cost the same)."""
    import oracle
    grid = oracle.Grid(w.T, w.Hh, w.W, w.theta)
    threads = oracle.num_threads()
    hs = max(1, min(w.H, threads))
    qs, ks, vs, gs = (t[:1, :, :hs].contiguous() for t in (q, k, v, g))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(qs, ks, vs, gs, grid)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    per_head = dt / (reps * hs)
    whole = per_head * w.B * w.H
    return {
        "value": (w.B * w.N) / whole,
        "unit": "tokens/s",
        "cores": threads,
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{hs} of {w.B * w.H} heads (batch 0, all N={w.N} tokens, one head per "
                  f"OpenMP thread), {reps} passes in {dt:.1f} s; {per_head:.3f} s per head, "
                  f"scaled to {w.B * w.H} heads",
    }


COUNTERS = os.path.join(ROOT, "profiles", "counters_5b_720p_193f.md")
KERNEL_SOURCES = [os.path.join(ROOT, "gated_linear_attention_forward_amd", "csrc", f)
                  for f in ("gla_kernels.hip", "gla_device.h", "gla_api.cpp", "gla_internal.h")]
BWD_COUNTERS = os.path.join(ROOT, "profiles", "backward_counters_5b_720p_193f.md")
BWD_SOURCES = [os.path.join(ROOT, "gated_linear_attention_forward_amd", "csrc", f)
               for f in ("gla_backward.hip", "gla_kernels.hip", "gla_device.h", "gla_api.cpp",
                         "gla_internal.h")]


def kernel_source_digest(sources=KERNEL_SOURCES):
    """sha256 over the sources that decide the kernels and their launch shapes."""
    h = hashlib.sha256()
    for path in sources:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(workload_name, path=COUNTERS, field="output_kernel_traffic_bytes",
                    sources=KERNEL_SOURCES):
    """HBM bytes (FETCH_SIZE + WRITE_SIZE, scaled by a calibration copy) from
    a committed counter summary, if it was taken on this workload (5B
    720p/193f) and on the current kernel sources."""
    if workload_name != "5b_720p_193f" or not os.path.exists(path):
        return None, "no counters for this workload"
    fields = {}
    with open(path) as f:
        for line in f:
            key, sep, val = line.partition(":")
            if sep and key.strip() in ("kernel_source_sha256", field):
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != kernel_source_digest(sources):
        return None, "kernel source changed since the counters were taken"
    if field not in fields:
        return None, f"no {field} in the counter summary"
    return float(fields[field]), os.path.relpath(path, ROOT)


def copy_calibration(dev, nbytes=1 << 30):
    """One plain device-to-device copy of known size, so hardware byte counters
    (FETCH_SIZE, WRITE_SIZE) read in the same run can be scaled to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: calibration copy of {nbytes} bytes done")
    del src, dst


def block_bench(args, w, gla, dev, tensors, out, rope, stream):
    """Block-causal pass: K passes of gla_forward_blocks_ws on the workload in
    blocks of args.block_frames latent frames, with the carried state read
    and updated in place (as a generator producing block after block would).
    Prints one JSON line; the roofline is the whole pass (HIP events around
    each pass on its stream) against 10*D bytes per (token, head) plus the
    state read and written."""
    import torch
    qd, kd, vd, gd = tensors
    L = args.block_frames * w.Hh * w.W
    S = torch.zeros((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    z = torch.zeros((w.B, w.H, w.D), dtype=torch.float32, device=dev)
    ws = gla.alloc_workspace_blocks(w.B, w.N, w.H, w.D, L, dev)

    sets = input_sets((qd, kd, vd, gd))

    def step(i=0):
        qs, ks, vs, gs = sets[i % len(sets)]
        gla.gla_forward_blocks_ws(qs, ks, vs, gs, rope, L, ws, S, z, S, z, out, stream)

    log(f"bench: block-causal, {args.block_frames} frames ({L} tokens) per block; "
        f"warmup {args.warmup}")
    warm_up(step, args.warmup)
    log(f"bench: timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    log(f"bench: {args.steps} instrumented steps")
    for i, e in enumerate(evs):
        e[0].record(stream)
        step(i)
        e[1].record(stream)
    torch.cuda.synchronize()
    ev_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    units = w.B * w.N * w.H
    nbytes = 10 * w.D * units + 2 * w.B * w.H * (w.D * w.D + w.D) * 4
    achieved = nbytes / (ev_ms * 1e-3) / 1e9
    result = {
        "metric": "block-causal gated linear-attn tokens/s per layer (carried state); "
                  "achieved HBM GB/s vs peak",
        "value": w.B * w.N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "D": w.D,
                   "grid": [w.T, w.Hh, w.W], "block_frames": args.block_frames,
                   "block_tokens": L, "blocks": -(-w.N // L), "parallelism": "single-gpu"},
        "roofline": {"kernel": "whole pass (state, scan, output kernels)", "bound": "hbm",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
                     "algorithmic_bytes": nbytes, "avg_ms": ev_ms},
    }
    print(json.dumps(result), flush=True)


PEAK_BF16_TFLOPS = 2500.0
EVICT_BYTES = 512 << 20   # twice the MI355X's 256 MB last-level cache (MALL)
ROTATE = 3                # input sets the HBM-bound benches cycle through


def warm_up(step, warmup, min_seconds=0.3):
    """`warmup` untimed steps, then more until about `min_seconds` have
    passed: the first passes over freshly allocated inputs, and an idle
    GPU's first milliseconds, run slower than the steady state."""
    import torch
    i = 0
    t_end = time.perf_counter() + min_seconds
    while i < warmup or time.perf_counter() < t_end:
        step(i)
        i += 1
        if i % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def input_sets(tensors, n=ROTATE):
    """n copies of the device inputs (the first is the given tensors): pass i
    reads set i % n, so no pass finds its inputs left in the last-level cache
    by the pass before, as it would when one set is read over and over."""
    return [tuple(tensors)] + [tuple(t.clone() for t in tensors) for _ in range(n - 1)]


def softmax_cpu_baseline(w, q, k, v, g, min_seconds=10.0):
    """Times the fp64 oracle's softmax rows on query tokens of head (0, 0),
    in batches of rows until about `min_seconds` of CPU work, and scales the
    per-row time to every (token, head) of the workload."""
    import numpy as np

    import oracle
    grid = oracle.Grid(w.T, w.Hh, w.W, w.theta)
    threads = oracle.num_threads()
    qs, ks, vs, gs = (t[:1, :, :1].contiguous() for t in (q, k, v, g))
    batch = 4 * threads
    rows_done = 0
    t0 = time.perf_counter()
    while True:
        rows = (np.arange(batch) * 7919 + rows_done) % w.N
        oracle.softmax_rows(qs, ks, vs, gs, grid, 0, 0, rows)
        rows_done += batch
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    per_row = dt / rows_done
    whole = per_row * w.B * w.H * w.N
    return {
        "value": (w.B * w.N) / whole,
        "unit": "tokens/s",
        "cores": threads,
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{rows_done} query rows of head (0, 0) against all N={w.N} keys in "
                  f"{dt:.1f} s; {per_row * 1e3:.2f} ms per row, scaled to "
                  f"{w.B * w.H * w.N} (token, head) rows",
    }


def softmax_bench(args, w, gla, dev, tensors, rope, stream):
    """Gated softmax anchor attention: K passes of gla_softmax_forward_ws (a
    rotation prep kernel, then the flash kernel).  The roofline is MFMA-bound:
    4*N*N*D flops per head (the score product and the value product, 2*N*N*D
    each) against the bf16 dense peak, over the whole call's event time (the
    prep kernel's share included)."""
    import torch
    qd, kd, vd, gd = tensors
    out = torch.empty_like(qd)
    ws = gla.alloc_workspace_softmax(w.B, w.N, w.H, w.D, dev)

    def step():
        gla.gla_softmax_forward_ws(qd, kd, vd, gd, rope, ws, out, stream)

    log(f"bench: softmax anchor attention; warmup {args.warmup}")
    warm_up(lambda i: step(), args.warmup)
    log(f"bench: timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    log(f"bench: {args.steps} instrumented steps")
    for e in evs:
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    ev_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    flops = 4.0 * w.B * w.H * w.N * w.N * w.D
    achieved = flops / (ev_ms * 1e-3) / 1e12
    result = {
        "metric": "gated softmax anchor attention tokens/s per layer; achieved bf16 MFMA "
                  "TFLOP/s vs peak",
        "value": w.B * w.N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "D": w.D,
                   "grid": [w.T, w.Hh, w.W], "parallelism": "single-gpu"},
        "roofline": {"kernel": "softmax prep + flash kernels", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "algorithmic_flops": flops, "avg_ms": ev_ms},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle (cpu_baseline)")
        q, k, v, g = (t.cpu() for t in tensors)
        result["cpu_baseline"] = softmax_cpu_baseline(w, q, k, v, g)
    print(json.dumps(result), flush=True)


def backward_cpu_baseline(w, q, k, v, g, dout, min_seconds=10.0):
    """Times the fp64 oracle's backward on the first `hs` heads of batch
    element 0 (one head per oracle thread) until about `min_seconds` of CPU
    work, and scales the per-head time to the whole workload."""
    import oracle
    grid = oracle.Grid(w.T, w.Hh, w.W, w.theta)
    threads = oracle.num_threads()
    hs = max(1, min(w.H, threads))
    qs, ks, vs, gs, ds = (t[:1, :, :hs].contiguous() for t in (q, k, v, g, dout))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.backward(qs, ks, vs, gs, ds, grid)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    per_head = dt / (reps * hs)
    return {
        "value": (w.B * w.N) / (per_head * w.B * w.H),
        "unit": "tokens/s",
        "cores": threads,
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{hs} of {w.B * w.H} heads (batch 0, all N={w.N} tokens), {reps} passes in "
                  f"{dt:.1f} s; {per_head:.3f} s per head, scaled to {w.B * w.H} heads",
    }


def backward_bench(args, w, gla, dev, tensors, rope, stream):
    """Backward pass: K passes of gla_backward_ws (state, query, gradient
    state and key kernels).  The roofline is the whole pass against the
    algorithmic minimum of 18*D bytes per (token, head): q, k, v, g and dout
    read, dq, dk, dv and dg written, once each.  "saved_state" times the same
    pass given the forward's fp32 state (gla_backward_saved_ws), against the
    same minimum."""
    import torch

    from workloads import random_grad
    qd, kd, vd, gd = tensors
    dout = random_grad(w.B, w.N, w.H, w.D, seed=w.seed + 1000).to(dev)
    grads = [torch.empty_like(qd) for _ in range(4)]
    ws = gla.alloc_workspace_backward(w.B, w.N, w.H, w.D, dev)

    sets = input_sets((qd, kd, vd, gd, dout))

    def step(i=0):
        qs, ks, vs, gs, ds = sets[i % len(sets)]
        gla.gla_backward_ws(qs, ks, vs, gs, ds, rope, ws, *grads, stream=stream)

    log(f"bench: backward; warmup {args.warmup}")
    warm_up(step, args.warmup)
    log(f"bench: timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    log(f"bench: {args.steps} instrumented steps")
    for i, e in enumerate(evs):
        e[0].record(stream)
        step(i)
        e[1].record(stream)
    torch.cuda.synchronize()
    ev_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    units = w.B * w.N * w.H
    nbytes = 18 * w.D * units
    achieved = nbytes / (ev_ms * 1e-3) / 1e9
    traffic, traffic_src = counter_traffic(w.name, BWD_COUNTERS, "backward_pass_traffic_bytes",
                                           BWD_SOURCES)
    result = {
        "metric": "gated linear-attn backward tokens/s per layer; achieved HBM GB/s vs peak",
        "value": w.B * w.N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "D": w.D,
                   "grid": [w.T, w.Hh, w.W], "parallelism": "single-gpu"},
        "roofline": {"kernel": "whole backward (state, reduce, query, reduce, key kernels)",
                     "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "traffic_source": traffic_src,
                     "traffic_over_algorithmic": traffic / nbytes if traffic else None,
                     "algorithmic_bytes": nbytes, "avg_ms": ev_ms},
    }
    # The same pass given the forward's saved state (gla_backward_saved_ws):
    # the forward's S and z replace the first state pass over k and v.
    S = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    z = torch.empty((w.B, w.H, w.D), dtype=torch.float32, device=dev)
    gla.gla_forward_blocks(qd, kd, vd, gd, rope, w.N, None, None, S, z, stream=stream)

    def step_saved(i=0):
        qs, ks, vs, gs, ds = sets[i % len(sets)]
        gla.gla_backward_saved_ws(qs, ks, vs, gs, ds, S, z, rope, ws, *grads, stream=stream)

    log(f"bench: backward with the saved state; {args.warmup} + {args.steps} steps")
    warm_up(step_saved, args.warmup)
    for i, e in enumerate(evs):
        e[0].record(stream)
        step_saved(i)
        e[1].record(stream)
    torch.cuda.synchronize()
    sv_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    sv_achieved = nbytes / (sv_ms * 1e-3) / 1e9
    sv_traffic, _ = counter_traffic(w.name, BWD_COUNTERS, "saved_state_pass_traffic_bytes",
                                    BWD_SOURCES)
    result["saved_state"] = {
        "entry": "gla_backward_saved_ws", "value": w.B * w.N / (sv_ms * 1e-3), "unit": "tokens/s",
        "avg_ms": sv_ms, "achieved": sv_achieved, "peak": PEAK_HBM_GBPS, "unit_roofline": "GB/s",
        "frac": sv_achieved / PEAK_HBM_GBPS, "traffic": sv_traffic,
        "traffic_over_algorithmic": sv_traffic / nbytes if sv_traffic else None,
        "algorithmic_bytes": nbytes}
    # What the pass would take if each kernel streamed its algorithmic bytes
    # at the plain-streaming rate of its own mix (query 10 D, key 8 D, state
    # 4 D per (token, head); the small partial and reduce traffic left out).
    log("bench: streaming ceiling of the backward mixes")
    ceil = backward_stream_ceiling(gla, dev, stream)
    del sets, grads, ws
    q_ms = 10 * w.D * units / (ceil["read_3_write_2"]["GB/s"] * 1e9) * 1e3
    k_ms = 8 * w.D * units / (ceil["read_2_write_2"]["GB/s"] * 1e9) * 1e3
    s_ms = 4 * w.D * units / (ceil["read_2_streams"]["GB/s"] * 1e9) * 1e3
    ceil["pass_ms_at_these_rates"] = q_ms + k_ms + s_ms
    ceil["saved_state_pass_ms_at_these_rates"] = q_ms + k_ms
    result["streaming_ceiling"] = ceil
    result["frac_of_streaming_ceiling"] = (q_ms + k_ms + s_ms) / ev_ms
    result["saved_state"]["frac_of_streaming_ceiling"] = (q_ms + k_ms) / sv_ms
    if not args.no_cpu_baseline:
        log("bench: timing the oracle (cpu_baseline)")
        q, k, v, g = (t.cpu() for t in tensors)
        result["cpu_baseline"] = backward_cpu_baseline(w, q, k, v, g, dout.cpu())
    print(json.dumps(result), flush=True)


def proj_cpu_baseline(w, x, wt, min_seconds=10.0):
    """Times the oracle's projections + mixer on single heads of batch
    element 0 (the projections parallel over tokens) until about
    `min_seconds` of CPU work, and scales the per-head time to every head."""
    import oracle
    grid = oracle.Grid(w.T, w.Hh, w.W, w.theta)
    xs = x[:1].contiguous()
    heads = 0
    t0 = time.perf_counter()
    while True:
        t = oracle.projected_heads(xs, wt, w.H, w.D, [heads % w.H])
        oracle.forward(t["q"], t["k"], t["v"], t["g"], grid)
        heads += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    per_head = dt / heads
    return {
        "value": (w.B * w.N) / (per_head * w.B * w.H),
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{heads} heads of batch 0 (all N={w.N} tokens, C={w.C}) in {dt:.1f} s; "
                  f"{per_head:.2f} s per head, scaled to {w.B * w.H} heads",
    }


def proj_bench(args, w, gla, dev):
    """Projection prologue fused with the mixer: K passes of
    gla_forward_proj_ws.  MFMA-bound: 2*C*4*H*D flops per token for the
    four maps plus 4*D*D per (token, head) for the state and output
    contractions, against the dense bf16 peak, over the call's event time."""
    import torch

    from workloads import make_projection
    log(f"bench: projection workload {w.name} B={w.B} N={w.N} C={w.C} H={w.H} D={w.D}")
    x, wt = make_projection(w)
    xd, wd = x.to(dev), wt.to(dev)
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D, w.theta)
    stream = torch.cuda.current_stream(dev)
    out = torch.empty((w.B, w.N, w.H, w.D), dtype=torch.bfloat16, device=dev)
    ws = gla.alloc_workspace_proj(w.B, w.N, w.C, w.H, w.D, dev)

    def step():
        gla.gla_forward_proj_ws(xd, wd, w.H, w.D, rope, ws, out, stream)

    log(f"bench: warmup {args.warmup}")
    warm_up(lambda i: step(), args.warmup)
    log(f"bench: timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    log(f"bench: {args.steps} instrumented steps")
    for e in evs:
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    ev_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    tokens = w.B * w.N
    flops = 2.0 * tokens * w.C * 4 * w.H * w.D + 4.0 * tokens * w.H * w.D * w.D
    achieved = flops / (ev_ms * 1e-3) / 1e12
    result = {
        "metric": "projected gated linear-attn layer tokens/s (x -> q,k,v,g -> mixer); "
                  "achieved bf16 MFMA TFLOP/s vs peak",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "C": w.C, "H": w.H, "D": w.D,
                   "grid": [w.T, w.Hh, w.W], "parallelism": "single-gpu"},
        "roofline": {"kernel": "whole layer (kv and qg projection kernels, reduce, output)",
                     "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "algorithmic_flops": flops, "avg_ms": ev_ms},
    }
    rope.close()
    if not args.no_cpu_baseline:
        log("bench: timing the oracle (cpu_baseline)")
        result["cpu_baseline"] = proj_cpu_baseline(w, x, wt)
    print(json.dumps(result), flush=True)


STREAM_PROBE_BYTES = 768 << 20  # per buffer; three sets of three exceed the 256 MB MALL


def stream_ceiling(gla, dev, stream, reps=20):
    """The GPU's plain-streaming bandwidth on the mixer's load path
    (gla_stream_probe: contiguous 16 KB pieces, one per short-lived block,
    16-byte non-temporal loads and stores): two read streams (the state
    half's mix) and two reads plus one write (the output half's mix), over
    three rotating sets of 768 MiB buffers, median of `reps` timed launches
    each."""
    import torch
    sets = [tuple(torch.empty(STREAM_PROBE_BYTES, dtype=torch.uint8, device=dev) for _ in range(3))
            for _ in range(ROTATE)]
    for st in sets:
        for t in st:
            t.fill_(1)
    res = {}
    for mode, name, streams in ((0, "read_2_streams", 2), (1, "read_2_write_1", 3)):
        for i in range(3):
            gla.gla_stream_probe(*sets[i % ROTATE], mode, stream)
        ts = []
        for i in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            gla.gla_stream_probe(*sets[i % ROTATE], mode, stream)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = statistics.median(ts)
        res[name] = {"GB/s": streams * STREAM_PROBE_BYTES / (ms * 1e-3) / 1e9, "ms": ms}
    del sets
    torch.cuda.synchronize()
    res["buffers"] = (f"3 rotating sets of 3 x {STREAM_PROBE_BYTES >> 20} MiB, contiguous 16 KB "
                      f"pieces per block")
    return res


def backward_stream_ceiling(gla, dev, stream, reps=20):
    """Plain-streaming rates of the backward kernels' mixes on the same load
    path (gla_stream_probe_mix, and gla_stream_probe for two reads): three
    reads and two writes (the query kernel: q, g, dout in, dq, dg out), two
    reads and two writes (the key kernel: k, v in, dk, dv out), and two reads
    (the state kernel), over three rotating sets of 768 MiB buffers, median of
    `reps` timed launches each."""
    import torch
    sets = [[torch.empty(STREAM_PROBE_BYTES, dtype=torch.uint8, device=dev) for _ in range(5)]
            for _ in range(ROTATE)]
    for st in sets:
        for t in st:
            t.fill_(1)
    mixes = (("read_3_write_2", 3, 2), ("read_2_write_2", 2, 2), ("read_2_streams", 2, 0))

    def run(i, ns, nd):
        st = sets[i % ROTATE]
        if nd == 0:
            gla.gla_stream_probe(st[0], st[1], st[2], 0, stream)
        else:
            gla.gla_stream_probe_mix(st[:ns], st[3:3 + nd], stream)

    res = {}
    for name, ns, nd in mixes:
        for i in range(3):
            run(i, ns, nd)
        ts = []
        for i in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(i, ns, nd)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = statistics.median(ts)
        res[name] = {"GB/s": (ns + nd) * STREAM_PROBE_BYTES / (ms * 1e-3) / 1e9, "ms": ms}
    del sets
    torch.cuda.synchronize()
    res["buffers"] = (f"3 rotating sets of 5 x {STREAM_PROBE_BYTES >> 20} MiB, contiguous 16 KB "
                      f"pieces per block")
    return res


def device_inputs(w, dev):
    """Inputs of a timing-only shape, drawn on the GPU (N(0, 1), q and k
    scaled by the workload's qk_scale, rounded to bf16): the same
    distribution as the seeded CPU inputs, without minutes of host work on
    the long shapes."""
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    out = []
    for i in range(4):
        x = torch.randn((w.B, w.N, w.H, w.D), generator=gen, dtype=torch.float32, device=dev)
        if i < 2 and w.qk_scale != 1.0:
            x.mul_(w.qk_scale)
        out.append(x.to(torch.bfloat16))
        del x
    return tuple(out)


def time_forward(gla, w, sets, rope, ws, out, stream, n, evict=None):
    """Median and mean of n passes of gla_forward_ws (HIP events on the launch
    stream around each call), cycling through the input sets; with `evict`,
    a 512 MiB read runs before each pass outside its events."""
    import torch
    ts = []
    for i in range(n):
        qs, ks, vs, gs = sets[i % len(sets)]
        if evict is not None:
            evict.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gla.gla_forward_ws(qs, ks, vs, gs, rope, out, ws, stream)
        e1.record(stream)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ts]
    return statistics.median(ms), sum(ms) / len(ms)


def config_figures(w, ms):
    units = w.B * w.N * w.H
    nbytes = 10 * w.D * units
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "tokens_per_s": w.B * w.N / (ms * 1e-3), "GB/s": gbps,
            "frac_of_8TBps": gbps / PEAK_HBM_GBPS, "algorithmic_bytes": nbytes}


def forward_bench(args, w, gla, dev, stream, host_inputs, dev_inputs):
    """The bidirectional mixer.  First, on every one of the five layer
    shapes, the median of >= 50 event-timed passes of gla_forward_ws (warm,
    and after a 512 MiB cache eviction).  Then the headline on the workload:
    W warmup passes and K wall-clock passes (one call per pass, inputs
    resident in HBM, three rotating sets), and per-kernel event times of the
    two halves for the roofline.  Last, the streaming ceiling and the oracle
    baseline."""
    import torch
    from workloads import WORKLOADS

    npass = max(50, args.steps)
    configs = list(WORKLOADS) if any(x.name == w.name for x in WORKLOADS) else [w]
    # the headline workload last, so the headline's warmup follows its own
    # passes (not the 10 GB of the 60 s layer's inputs)
    configs = [x for x in configs if x.name != w.name] + [w]
    if args.no_sweep:
        configs = [w]
    scratch = torch.zeros(EVICT_BYTES // 4, dtype=torch.float32, device=dev)
    # about half a second of streaming first, untimed: an idle GPU runs its
    # first milliseconds of work at lower clocks
    spin_end = time.perf_counter() + 0.5
    while time.perf_counter() < spin_end:
        for _ in range(100):
            scratch.sum()
        torch.cuda.synchronize()
    all_cfg = []
    head = None
    for wl in configs:
        if wl.name == w.name:
            qd, kd, vd, gd = dev_inputs
        else:
            qd, kd, vd, gd = device_inputs(wl, dev)
        sets = input_sets((qd, kd, vd, gd))
        del qd, kd, vd, gd
        rope = gla.gla_rope_create(wl.T, wl.Hh, wl.W, wl.D, wl.theta)
        ws = gla.alloc_workspace(wl.B, wl.N, wl.H, wl.D, dev)
        out = torch.empty_like(sets[0][0])
        # untimed passes first, at least 20 and 0.2 s: the first passes over
        # freshly allocated inputs run slower (address translation warms up)
        i = 0
        t_end = time.perf_counter() + 0.2
        while i < 20 or time.perf_counter() < t_end:
            qs, ks, vs, gs = sets[i % len(sets)]
            gla.gla_forward_ws(qs, ks, vs, gs, rope, out, ws, stream)
            i += 1
            if i % 20 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        log(f"bench: {wl.name}: {npass} event-timed passes, warm and after cache eviction")
        warm_med, warm_mean = time_forward(gla, wl, sets, rope, ws, out, stream, npass)
        cold_med, _ = time_forward(gla, wl, sets, rope, ws, out, stream, npass, evict=scratch)
        fig = config_figures(wl, warm_med)
        fig.update({"workload": wl.name, "B": wl.B, "N": wl.N, "H": wl.H, "D": wl.D,
                    "passes": npass, "mean_ms": warm_mean, "cold_cache_median_ms": cold_med,
                    "cold_cache_frac_of_8TBps": config_figures(wl, cold_med)["frac_of_8TBps"]})
        all_cfg.append(fig)
        if wl.name == w.name:
            head = (sets, rope, ws, out)  # timed below, after the sweep
        else:
            rope.close()
        del sets, ws, out
        torch.cuda.synchronize()
    del scratch

    # the headline: W warmup passes, then exactly K passes, nothing else
    # enqueued, on the GPU the sweep above has brought up to speed
    sets, rope, ws, out = head
    log(f"bench: {w.name}: {args.warmup} warmup steps, then timing {args.steps} steps")
    for i in range(args.warmup):
        qs, ks, vs, gs = sets[i % len(sets)]
        gla.gla_forward_ws(qs, ks, vs, gs, rope, out, ws, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        qs, ks, vs, gs = sets[i % len(sets)]
        gla.gla_forward_ws(qs, ks, vs, gs, rope, out, ws, stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # per-kernel durations of the two halves: state (state + reduce kernels)
    # and output (the output kernel alone), HIP events on the stream they run on
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(npass)]
    for i, e in enumerate(evs):
        qs, ks, vs, gs = sets[i % len(sets)]
        e[0].record(stream)
        gla.gla_state_ws(ks, vs, rope, ws, stream)
        e[1].record(stream)
        gla.gla_output_ws(qs, gs, rope, out, ws, stream)
        e[2].record(stream)
    torch.cuda.synchronize()
    state_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / npass
    out_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / npass
    rope.close()
    del head, sets, ws, out
    torch.cuda.synchronize()
    ceiling = None
    if not args.no_sweep:
        log("bench: streaming ceiling")
        ceiling = stream_ceiling(gla, dev, stream)
        rd, rw = ceiling["read_2_streams"]["GB/s"], ceiling["read_2_write_1"]["GB/s"]
        for fig, wl in zip(all_cfg, configs):
            units = wl.B * wl.N * wl.H
            t_ceil = 4 * wl.D * units / (rd * 1e9) + 6 * wl.D * units / (rw * 1e9)
            fig["frac_of_streaming_ceiling"] = t_ceil * 1e3 / fig["ms"]
    # reported in the canonical order of the five layer shapes
    rank = {x.name: i for i, x in enumerate(WORKLOADS)}
    all_cfg.sort(key=lambda f: rank.get(f["workload"], len(rank)))

    units = w.B * w.N * w.H
    out_bytes = 6 * w.D * units
    state_bytes = 4 * w.D * units
    achieved = out_bytes / (out_ms * 1e-3) / 1e9
    traffic, traffic_src = counter_traffic(w.name)
    head_fig = next(f for f in all_cfg if f["workload"] == w.name)
    result = {
        "metric": METRIC,
        "value": w.B * w.N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "D": w.D,
                   "grid": [w.T, w.Hh, w.W], "parallelism": "single-gpu"},
        "hbm_gbps_effective": 10 * w.D * units / (ms_step * 1e-3) / 1e9,
        "frac_of_8TBps": 10 * w.D * units / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "pass_median_ms": head_fig["ms"],
        "pass_median_frac_of_8TBps": head_fig["frac_of_8TBps"],
        "phases_ms": {"state": state_ms, "output": out_ms},
        "roofline": {
            "kernel": "output_persist_kernel",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "traffic_source": traffic_src,
            "traffic_over_algorithmic": traffic / out_bytes if traffic else None,
            "algorithmic_bytes": out_bytes,
            "avg_ms": out_ms,
        },
        "state_roofline": {
            "kernels": "state_tile_kernel + reduce_kernel",
            "bound": "hbm",
            "achieved": state_bytes / (state_ms * 1e-3) / 1e9,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": state_bytes / (state_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "algorithmic_bytes": state_bytes,
            "avg_ms": state_ms,
        },
        "streaming_ceiling": ceiling,
        "all_configs": all_cfg,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle (cpu_baseline)")
        q, k, v, g = host_inputs
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, g)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="time only the workload (no five-shape sweep, no streaming ceiling): "
                         "for profiler runs whose kernel statistics must cover it alone")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy first (for hardware byte counters)")
    ap.add_argument("--block-frames", type=int, default=0,
                    help="time the block-causal pass (gla_forward_blocks) in blocks of this "
                         "many latent frames, carrying the state in place, instead of the "
                         "bidirectional mixer")
    ap.add_argument("--softmax", action="store_true",
                    help="time the gated softmax anchor attention (gla_softmax_forward) "
                         "instead; the workload defaults to anchor_5b_720p_193f")
    ap.add_argument("--backward", action="store_true",
                    help="time the mixer's backward pass (gla_backward) instead")
    ap.add_argument("--proj", action="store_true",
                    help="time the projection prologue fused with the mixer (gla_forward_proj); "
                         "the workload defaults to proj_5b_720p_193f")
    args = ap.parse_args()
    if args.proj and args.workload == DEFAULT_WORKLOAD:
        args.workload = "proj_5b_720p_193f"
    if args.softmax and args.workload == DEFAULT_WORKLOAD:
        args.workload = "anchor_5b_720p_193f"

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the mixer's state is exchanged within one "
              f"device; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_linear_attention_forward_amd as gla
    from workloads import BY_NAME, make_inputs

    w = BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.proj:
        proj_bench(args, w, gla, dev)
        return
    log(f"bench: workload {w.name} B={w.B} N={w.N} H={w.H} D={w.D}; generating inputs")
    q, k, v, g = make_inputs(w)
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D, w.theta)
    stream = torch.cuda.current_stream(dev)
    if args.calibrate_copy:
        copy_calibration(dev)
    if args.softmax:
        softmax_bench(args, w, gla, dev, (qd, kd, vd, gd), rope, stream)
        return
    if args.backward:
        backward_bench(args, w, gla, dev, (qd, kd, vd, gd), rope, stream)
        return
    if args.block_frames > 0:
        out = torch.empty_like(qd)
        block_bench(args, w, gla, dev, (qd, kd, vd, gd), out, rope, stream)
        return
    rope.close()
    forward_bench(args, w, gla, dev, stream, (q, k, v, g), (qd, kd, vd, gd))


if __name__ == "__main__":
    main()
