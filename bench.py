#!/usr/bin/env python3
"""Benchmark of the fused MoE router on one MI355X.

Headline (the latency point of the router's own metric): router_fwd at
M=1 token, H=7168, E=256, k=8, softmax, no bias, renorm.  One step = one
token through 40 MoE layers = 40 router calls, each with its own gate matrix
and activation.  Gate matrices rotate through a 160-matrix pool (587 MB, more
than twice the 256 MB Infinity Cache) so that W_gate comes from HBM; the 40
calls of a step are captured in a HIP graph and replayed.  `value` is
microseconds per router call (lower is better).

Also reported (same JSON line):
  roofline      the decode kernel: algorithmic bytes per launch over its mean
                duration from per-launch HIP events on its stream, vs 8 TB/s;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload;
  extras        cache-hot cycle, verify widths M=2/8 at H=4096, the biased M=2
                table on/off delta, the standalone top-k at M=4096, and the
                8192-token prefill (tokens/s and fraction of bf16 MFMA peak).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
LAYERS = 40
POOL = 160


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def event_times_ms(torch, fn, n, stream):
    """Per-launch durations (ms) from an event pair recorded around each launch on `stream`."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        starts[i].record(stream)
        fn(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the router shards tokens across GPUs with no exchange, so each GPU "
              "runs this same single-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    from gate_projection_top_amd import router as R
    from gate_projection_top_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R.load()
    R.init(0)
    stream = torch.cuda.current_stream(dev)

    # ------------------------------------------------------------------ headline
    H, E, k = 7168, 256, 8
    log(f"generating pools: W {POOL}x{E}x{H} bf16, X {LAYERS}x1x{H}")
    wpool = W.torch_gaussian_bf16((POOL, E, H), 1.0 / H ** 0.5, seed=1, device=dev)
    xpool = W.torch_rms_normalised_bf16((LAYERS, 1, H), seed=2, device=dev)
    inds = torch.empty((LAYERS, 1, k), dtype=torch.int32, device=dev)
    wts = torch.empty((LAYERS, 1, k), dtype=torch.float32, device=dev)

    def call(layer, widx):
        R.router_fwd(xpool[layer], wpool[widx], None, k, W.SOFTMAX, True,
                     out_inds=inds[layer], out_weights=wts[layer])

    groups = POOL // LAYERS
    for g in range(groups):              # eager warm-up (also initialises everything)
        for l in range(LAYERS):
            call(l, g * LAYERS + l)
    torch.cuda.synchronize()

    graphs = []
    for g in range(groups):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for l in range(LAYERS):
                call(l, g * LAYERS + l)
        graphs.append(gr)
    torch.cuda.synchronize()

    for s in range(args.warmup):
        graphs[s % groups].replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps x {LAYERS} calls (cold W pool, graph replay)")
    t0 = time.perf_counter()
    for s in range(args.steps):
        graphs[s % groups].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    us_per_call = ms_per_step * 1e3 / LAYERS

    # per-launch kernel durations with HIP events (eager, same stream, cold pool)
    n_ev = args.steps * LAYERS
    ev = event_times_ms(torch, lambda i: call(i % LAYERS, i % POOL), n_ev, stream)
    kern_us = 1e3 * sum(ev) / len(ev)
    bytes_per_launch = E * H * 2 + H * 2 + k * 8  # W + x + (inds, weights)
    achieved_gbs = bytes_per_launch / (kern_us * 1e-6) / 1e9

    extras = {"decode_M1_H7168_event_us_per_launch": round(kern_us, 3)}

    # cache-hot cycle: the same 40 gate matrices every step (MALL-resident)
    for _ in range(args.warmup):
        graphs[0].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graphs[0].replay()
    torch.cuda.synchronize()
    extras["decode_M1_H7168_hot_us_per_call"] = round((time.perf_counter() - t0) * 1e6 / (args.steps * LAYERS), 3)
    del graphs

    if not args.no_extras:
        extras.update(run_extras(torch, R, W, dev, stream, args))

    # ------------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(W, args.cpu_seconds)

    out = {
        "metric": "router µs/call at M=1,H=7168,E=256,k=8; tokens/s at M=8192; % HBM/MFMA peak",
        "value": round(us_per_call, 3),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode router M=1 H=7168 E=256 k=8 softmax renorm, no bias; "
                        "one step = 40 layers x 1 call, distinct W_gate per call from a "
                        "160-matrix (587 MB) pool, HIP-graph replay",
            "M": 1, "H": H, "E": E, "k": k, "calls_per_step": LAYERS,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_router_kernel",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "bytes_per_launch": bytes_per_launch,
            "launch_us": round(kern_us, 3),
        },
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(out), flush=True)


def run_extras(torch, R, W, dev, stream, args):
    ex = {}
    reps = max(args.steps, 10)

    def graph_us(fn, n_calls):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / (reps * n_calls)

    # verify widths at H=4096 (40-layer hot cycle)
    H, E = 4096, 256
    wl = W.torch_gaussian_bf16((LAYERS, E, H), 1.0 / H ** 0.5, seed=3, device=dev)
    for M in (1, 2, 8):
        x = W.torch_rms_normalised_bf16((LAYERS, M, H), seed=4 + M, device=dev)
        oi = torch.empty((LAYERS, M, 8), dtype=torch.int32, device=dev)
        ow = torch.empty((LAYERS, M, 8), dtype=torch.float32, device=dev)

        def step(x=x, oi=oi, ow=ow):
            for l in range(LAYERS):
                R.router_fwd(x[l], wl[l], None, 8, W.SOFTMAX, True, out_inds=oi[l], out_weights=ow[l])
        ex[f"decode_M{M}_H4096_hot_us_per_call"] = round(graph_us(step, LAYERS), 3)
    log("verify widths done")

    # biased M=2 with and without the unique-route table (k=6)
    bias = W.torch_uniform_f32(E, -0.05, 0.05, seed=9, device=dev)
    x2 = W.torch_gaussian_bf16((LAYERS, 2, H), 1.0, seed=10, device=dev)
    oi = torch.empty((LAYERS, 2, 6), dtype=torch.int32, device=dev)
    ow = torch.empty((LAYERS, 2, 6), dtype=torch.float32, device=dev)
    tabs = [{n: torch.empty(12 if n != "unique_count" else 1, dtype=torch.int32, device=dev)
             for n in ("unique_ids", "token_mask", "slot_to_unique", "unique_count")}
            for _ in range(LAYERS)]

    def step_off():
        for l in range(LAYERS):
            R.router_fwd(x2[l], wl[l], bias, 6, W.SQRT_SOFTPLUS, True, out_inds=oi[l], out_weights=ow[l])

    def step_on():
        for l in range(LAYERS):
            R.router_fwd_m2_table(x2[l], wl[l], bias, 6, W.SQRT_SOFTPLUS, True,
                                  out=dict(inds=oi[l], weights=ow[l], **tabs[l]))
    off = graph_us(step_off, LAYERS)
    on = graph_us(step_on, LAYERS)
    ex["biased_M2_k6_table_off_us_per_call"] = round(off, 3)
    ex["biased_M2_k6_table_on_us_per_call"] = round(on, 3)
    ex["table_overhead_us_per_call"] = round(on - off, 3)
    ex["table_overhead_context_b70_us_per_layer"] = 3.132
    del wl
    log("table on/off done")

    # standalone top-k at M=4096
    lg = torch.randn((4, 4096, 256), device=dev, dtype=torch.float32) * 2 ** 0.5
    ti = torch.empty((4096, 8), dtype=torch.int32, device=dev)
    tw = torch.empty((4096, 8), dtype=torch.float32, device=dev)
    evt = event_times_ms(torch, lambda i: R.router_topk_from_logits(lg[i % 4], None, 8, out_inds=ti, out_weights=tw),
                         reps, stream)
    t_us = 1e3 * sum(evt) / len(evt)
    ex["topk_M4096_us_per_call"] = round(t_us, 3)
    ex["topk_M4096_GBs"] = round((4096 * 256 * 4 + 4096 * 64) / (t_us * 1e-6) / 1e9, 1)
    del lg
    log("top-k done")

    # prefill M=8192, H=7168 (4 rotating X buffers: 470 MB, cold)
    M, H = 8192, 7168
    xs = W.torch_gaussian_bf16((4, M, H), 1.0, seed=11, device=dev)
    wp = W.torch_gaussian_bf16((E, H), 1.0 / H ** 0.5, seed=12, device=dev)
    bp = W.torch_uniform_f32(E, -0.02, 0.02, seed=13, device=dev)
    pi = torch.empty((M, 8), dtype=torch.int32, device=dev)
    pw = torch.empty((M, 8), dtype=torch.float32, device=dev)
    for i in range(args.warmup):
        R.router_fwd(xs[i % 4], wp, bp, 8, W.SOFTMAX, True, out_inds=pi, out_weights=pw)
    evp = event_times_ms(torch, lambda i: R.router_fwd(xs[i % 4], wp, bp, 8, W.SOFTMAX, True,
                                                       out_inds=pi, out_weights=pw), reps, stream)
    p_us = 1e3 * sum(evp) / len(evp)
    flops = 2.0 * M * E * H
    ex["prefill_M8192_H7168_us_per_call"] = round(p_us, 2)
    ex["prefill_M8192_tokens_per_s"] = round(M / (p_us * 1e-6), 0)
    ex["prefill_mfma_tflops"] = round(flops / (p_us * 1e-6) / 1e12, 1)
    ex["prefill_mfma_frac"] = round(flops / (p_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    ex["prefill_hbm_frac"] = round((M * H * 2 + E * H * 2 + M * 64) / (p_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    log("prefill done")
    return ex


def cpu_baseline(W, seconds):
    """The oracle (as written, single thread) on M=1 H=7168 router calls for ~`seconds`."""
    import numpy as np
    import oracle

    orc = oracle.get()
    case = W.metric_case(0)
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.router(case.x, case.w, case.bias, case.k, case.scoring, case.renorm)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    log(f"cpu baseline: {n} oracle calls in {el:.1f}s")
    return {"value": round(el * 1e6 / n, 1), "unit": "µs/call", "cores": 1, "kind": "oracle",
            "sample": f"{n} single-token router calls (H=7168, E=256, k=8, softmax, renorm) "
                      f"through the C oracle, one thread"}


if __name__ == "__main__":
    main()
