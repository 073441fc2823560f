#!/usr/bin/env python3
"""Benchmark of the fused MoE router on one MI355X.

Headline (the latency point of the router's own metric): router_fwd at
M=1 token, H=7168, E=256, k=8, softmax, no bias, renorm.  One step = one
token through 40 MoE layers = 40 router calls, each with its own gate matrix
and activation.  Gate matrices rotate through a 160-matrix pool (587 MB, more
than twice the 256 MB Infinity Cache) so that W_gate comes from HBM.  The 40
calls of a step are captured in a HIP graph and replayed; `value` is
microseconds per router call (lower is better), from the wall clock around the
timed replays.

Also reported (same JSON line):
  roofline      the decode kernel: algorithmic bytes per launch over its mean
                duration (a HIP event pair on the launching stream around the
                timed replays, divided by the launch count), vs 8 TB/s; traffic
                from the committed rocprofv3 counter summary when the kernel
                sources still match it, else null;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload, one
                thread (extras.cpu_baseline_all_threads: the same calls on up to
                16 threads at once, as throughput);
  extras        the same calls launched eagerly (through the Python binding,
                and straight through the C ABI), the cache-hot cycle, verify
                widths M=1/2/8 at H=4096 (cache-hot, and cold from a 537 MB
                pool), the fused-vs-unfused A/B at those widths (a library GEMM
                writing logits + router_topk_from_logits), the biased M=2 table
                on/off delta and M=16/64, the launch-floor probes (other
                grid sizes and hand-off protocols too), the
                streaming-read ceiling of HBM (plain and non-temporal
                loads) and the prefill main loop's
                load streams taken apart (libfloorprobes.so), the MXFP4
                and MXFP8 gates at M=1 and M=8
                (H=7168, 585 / 606 MB pools) and at the 8192-token prefill, the
                routed gather + shared-expert add at M=2 (explicit rows, all
                remote, table rows) and at M=4096, the expert GEMM1 on the
                table at M=2 (F=4096, D=7168, 15 GB of expert weights), the
                standalone top-k at M=4096, the 8192-token prefill
                (tokens/s, fraction of bf16 MFMA and HBM peak, and a roofline
                block of its own; with X cold and cache-hot), and router_fwd
                across batch sizes from 16
                to 4096 tokens.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--section S]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
LAYERS = 40
POOL = 160
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_expert_M1_H7168_traffic.txt")
MX_TRAFFIC_SUMMARY = {f: os.path.join(ROOT, "profiles", f"decode_expert_{f}_M1_H7168_traffic.txt")
                      for f in ("mxfp4", "mxfp8")}
GATHER_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gather_shared_add_M2_k6_D7168_traffic.txt")
GEMM1_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "expert_gemm1_M2_k6_F4096_D7168_traffic.txt")
KERNEL_SOURCES = ["route_common.hpp", "softmax_exp.hpp", "coherent.hpp", "decode_expert_kernel.hip", "launch.hpp", "router_api.cpp"]
PREFILL_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "prefill_router_M8192_H7168_traffic.txt")
PREFILL_SOURCES = ["route_common.hpp", "softmax_exp.hpp", "coherent.hpp", "prefill_kernel.hip", "launch.hpp", "router_api.cpp"]
GATHER_SOURCES = ["gather_kernel.hip", "route_common.hpp", "softmax_exp.hpp", "launch.hpp", "router_api.cpp"]
GEMM1_SOURCES = ["gemm1_kernel.hip", "route_common.hpp", "softmax_exp.hpp", "coherent.hpp", "launch.hpp", "router_api.cpp"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--section", choices=["all", "decode", "widths", "mxfp4", "mxfp8", "gather", "gemm1", "prefill",
                                          "topk", "floor", "sizes"],
                    default="all",
                    help="restrict to one workload (for counter-collection runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--mxfp4-widths", default="1,8",
                    help="token counts of the MXFP4 section (comma-separated, each <= 64)")
    ap.add_argument("--mxfp8-widths", default="1,8",
                    help="token counts of the MXFP8 section (comma-separated, each <= 64)")
    ap.add_argument("--gather-disjoint-only", action="store_true",
                    help="gather section: only the M=2 explicit-row case (counter-collection runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def kernel_source_digest(names=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "gate_projection_top_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(path=TRAFFIC_SUMMARY, sources=KERNEL_SOURCES):
    """Bytes per launch from a committed counter summary, if the kernel sources still match it."""
    try:
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_sources_sha256_16") != kernel_source_digest(sources):
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class GraphTimer:
    """A HIP graph of calls (replayed for the wall-clock `value`)."""

    def __init__(self, torch, calls):
        for c in calls:  # eager warm-up (allocates nothing inside capture)
            c()
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for c in calls:
                c()

    def replay(self):
        self.graph.replay()


def timed_replays(torch, graphs, steps, warmup):
    """Time `steps` replays (round-robin over graphs) after warm-up.

    Returns (wall seconds, event milliseconds): the wall clock around the
    replay loop, and a HIP event pair recorded on the replaying stream at its
    two ends (GPU time of the back-to-back launches, host launch latency
    excluded).
    """
    for s in range(warmup):
        graphs[s % len(graphs)].replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for s in range(steps):
        graphs[s % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, start.elapsed_time(end)


def graph_call_us(torch, calls, steps, warmup):
    """Mean GPU microseconds per call: `calls` captured once, replayed `steps` times."""
    g = GraphTimer(torch, calls)
    _, ms = timed_replays(torch, [g], steps, warmup)
    return ms * 1e3 / (steps * len(calls))


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

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration_mib} MiB device-to-device copy")
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": "router µs/call at M=1,H=7168,E=256,k=8; tokens/s at M=8192; % HBM/MFMA peak",
        "value": None,
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode router M=1 H=7168 E=256 k=8 softmax renorm, no bias; "
                        "one step = 40 layers x 1 call, distinct W_gate per call from a "
                        "160-matrix (587 MB) pool, HIP-graph replay",
            "M": 1, "H": 7168, "E": 256, "k": 8, "calls_per_step": LAYERS,
        },
        "roofline": None,
        "cpu_baseline": None,
        "extras": {},
    }

    if args.section in ("all", "decode"):
        decode_headline(torch, R, W, dev, args, out)
    if args.section in ("all", "widths"):
        out["extras"].update(decode_extras(torch, R, W, dev, args))
    if args.section in ("all", "floor"):
        out["extras"].update(floor_extras(torch, W, dev, args))
    for fmt in ("mxfp4", "mxfp8"):
        if args.section in ("all", fmt):
            out["extras"].update(block_scaled_extras(torch, R, W, dev, args, fmt))
    if args.section in ("all", "gather"):
        out["extras"].update(gather_extras(torch, R, W, dev, args))
    if args.section in ("all", "gemm1"):
        out["extras"].update(gemm1_extras(torch, R, W, dev, args))
    if args.section in ("all", "topk"):
        out["extras"].update(topk_extras(torch, R, W, dev, args))
    if args.section in ("all", "prefill"):
        out["extras"].update(prefill_extras(torch, R, W, dev, args))
    if args.section in ("all", "sizes"):
        out["extras"].update(size_extras(torch, R, W, dev, args))
    if args.section == "all" and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_seconds)
        out["extras"]["cpu_baseline_all_threads"] = cpu_baseline_threads(W, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def decode_headline(torch, R, W, dev, args, out):
    H, E, k = 7168, 256, 8
    log(f"generating pools: W {POOL}x{E}x{H} bf16, X {LAYERS}x1x{H}")
    wpool = W.torch_gaussian_bf16((POOL, E, H), 1.0 / H ** 0.5, seed=1, device=dev)
    xpool = W.torch_rms_normalised_bf16((LAYERS, 1, H), seed=2, device=dev)
    inds = torch.empty((LAYERS, 1, k), dtype=torch.int32, device=dev)
    wts = torch.empty((LAYERS, 1, k), dtype=torch.float32, device=dev)

    def call(layer, widx):
        return lambda: R.router_fwd(xpool[layer], wpool[widx], None, k, W.SOFTMAX, True,
                                    out_inds=inds[layer], out_weights=wts[layer])

    groups = POOL // LAYERS
    step_calls = [[call(l, g * LAYERS + l) for l in range(LAYERS)] for g in range(groups)]
    clean = [GraphTimer(torch, c) for c in step_calls]

    log(f"timing {args.steps} steps x {LAYERS} calls (cold W pool, graph replay)")
    wall, ev_ms = timed_replays(torch, clean, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    out["value"] = round(ms_per_step * 1e3 / LAYERS, 3)
    out["ms_per_step"] = round(ms_per_step, 4)

    n_launch = args.steps * LAYERS
    kern_us = ev_ms * 1e3 / n_launch
    bytes_per_launch = E * H * 2 + H * 2 + k * 8  # W + x + (inds, weights)
    achieved = bytes_per_launch / (kern_us * 1e-6) / 1e9
    traffic = committed_traffic()
    out["roofline"] = {
        "bound": "hbm",
        "kernel": "decode_expert_kernel",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "bytes_per_launch": bytes_per_launch,
        "launch_us": round(kern_us, 3),
        "launches_timed": n_launch,
        "launch_timing": "HIP event pair on the launching stream around the timed replays "
                         "(back-to-back launches) / launch count",
    }
    # the same calls launched eagerly (host launch path included), cold pool
    eager_calls = [c for grp in step_calls for c in grp]
    for c in eager_calls[:LAYERS]:
        c()
    torch.cuda.synchronize()
    n_eager = args.steps * LAYERS
    t0 = time.perf_counter()
    for i in range(n_eager):
        eager_calls[i % len(eager_calls)]()
    torch.cuda.synchronize()
    out["extras"]["decode_M1_H7168_eager_us_per_call"] = round((time.perf_counter() - t0) * 1e6 / n_eager, 3)
    # the same eager calls straight through the C ABI with their arguments
    # marshalled beforehand: the library's own host path per call
    lib = R.load()
    stream = torch.cuda.current_stream().cuda_stream
    raw = [(xpool[i % LAYERS].data_ptr(), wpool[i % POOL].data_ptr(), inds[i % LAYERS].data_ptr(),
            wts[i % LAYERS].data_ptr()) for i in range(POOL)]
    for xp, wp, ip, op in raw[:LAYERS]:
        lib.router_fwd(xp, wp, None, 1, H, E, k, W.SOFTMAX, 1, ip, op, None, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_eager):
        xp, wp, ip, op = raw[i % POOL]
        if lib.router_fwd(xp, wp, None, 1, H, E, k, W.SOFTMAX, 1, ip, op, None, stream) != 0:
            raise RuntimeError("router_fwd failed")
    torch.cuda.synchronize()
    out["extras"]["decode_M1_H7168_eager_c_abi_us_per_call"] = round((time.perf_counter() - t0) * 1e6 / n_eager, 3)
    # cache-hot cycle: the same 40 gate matrices every step (Infinity-Cache resident)
    hot, _ = timed_replays(torch, clean[:1], args.steps, args.warmup)
    out["extras"]["decode_M1_H7168_hot_us_per_call"] = round(hot * 1e6 / (args.steps * LAYERS), 3)
    out["extras"]["decode_kernel_sources_sha256_16"] = kernel_source_digest()
    del clean, wpool


def decode_extras(torch, R, W, dev, args):
    ex = {}
    H, E = 4096, 256
    wl = W.torch_gaussian_bf16((LAYERS, E, H), 1.0 / H ** 0.5, seed=3, device=dev)
    for M in (1, 2, 8):
        x = W.torch_rms_normalised_bf16((LAYERS, M, H), seed=4 + M, device=dev)
        oi = torch.empty((LAYERS, M, 8), dtype=torch.int32, device=dev)
        ow = torch.empty((LAYERS, M, 8), dtype=torch.float32, device=dev)
        calls = [(lambda l=l, x=x, oi=oi, ow=ow: R.router_fwd(x[l], wl[l], None, 8, W.SOFTMAX, True,
                                                               out_inds=oi[l], out_weights=ow[l]))
                 for l in range(LAYERS)]
        ex[f"decode_M{M}_H4096_hot_us_per_call"] = round(graph_call_us(torch, calls, args.steps, args.warmup), 3)
    log("verify widths (hot) done")
    ex.update(decode_widths_cold_and_unfused(torch, R, W, dev, args))

    # biased M=2 with and without the unique-route table (k=6)
    bias = W.torch_uniform_f32(E, -0.05, 0.05, seed=9, device=dev)
    x2 = W.torch_gaussian_bf16((LAYERS, 2, H), 1.0, seed=10, device=dev)
    oi = torch.empty((LAYERS, 2, 6), dtype=torch.int32, device=dev)
    ow = torch.empty((LAYERS, 2, 6), dtype=torch.float32, device=dev)
    tabs = [{n: torch.empty(12 if n != "unique_count" else 1, dtype=torch.int32, device=dev)
             for n in ("unique_ids", "token_mask", "slot_to_unique", "unique_count")}
            for _ in range(LAYERS)]
    off = [(lambda l=l: R.router_fwd(x2[l], wl[l], bias, 6, W.SQRT_SOFTPLUS, True,
                                     out_inds=oi[l], out_weights=ow[l])) for l in range(LAYERS)]
    on = [(lambda l=l: R.router_fwd_m2_table(x2[l], wl[l], bias, 6, W.SQRT_SOFTPLUS, True,
                                             out=dict(inds=oi[l], weights=ow[l], **tabs[l])))
          for l in range(LAYERS)]
    t_off = graph_call_us(torch, off, args.steps, args.warmup)
    t_on = graph_call_us(torch, on, args.steps, args.warmup)
    ex["biased_M2_k6_table_off_us_per_call"] = round(t_off, 3)
    ex["biased_M2_k6_table_on_us_per_call"] = round(t_on, 3)
    ex["table_overhead_us_per_call"] = round(t_on - t_off, 3)
    ex["table_overhead_context_b70_us_per_layer"] = 3.132
    # the table at the widest verify width (M=8, k=8: 64 slots), decode router
    x8 = W.torch_rms_normalised_bf16((LAYERS, 8, H), seed=12, device=dev)
    oi8 = torch.empty((LAYERS, 8, 8), dtype=torch.int32, device=dev)
    ow8 = torch.empty((LAYERS, 8, 8), dtype=torch.float32, device=dev)
    tabs8 = [{n: torch.empty(64 if n != "unique_count" else 1, dtype=torch.int32, device=dev)
              for n in ("unique_ids", "token_mask", "slot_to_unique", "unique_count")}
             for _ in range(LAYERS)]
    off8 = [(lambda l=l: R.router_fwd(x8[l], wl[l], None, 8, W.SOFTMAX, True,
                                      out_inds=oi8[l], out_weights=ow8[l])) for l in range(LAYERS)]
    on8 = [(lambda l=l: R.router_fwd_route_table(x8[l], wl[l], None, 8, W.SOFTMAX, True,
                                                 out=dict(inds=oi8[l], weights=ow8[l], **tabs8[l])))
           for l in range(LAYERS)]
    t_off8 = graph_call_us(torch, off8, args.steps, args.warmup)
    t_on8 = graph_call_us(torch, on8, args.steps, args.warmup)
    ex["table_M8_k8_off_us_per_call"] = round(t_off8, 3)
    ex["table_M8_k8_on_us_per_call"] = round(t_on8, 3)
    ex["table_M8_k8_overhead_us_per_call"] = round(t_on8 - t_off8, 3)
    for M in (16, 64):
        xm = W.torch_gaussian_bf16((LAYERS, M, H), 1.0, seed=20 + M, device=dev)
        oim = torch.empty((LAYERS, M, 6), dtype=torch.int32, device=dev)
        owm = torch.empty((LAYERS, M, 6), dtype=torch.float32, device=dev)
        calls = [(lambda l=l, xm=xm, oim=oim, owm=owm: R.router_fwd(
            xm[l], wl[l], bias, 6, W.SQRT_SOFTPLUS, True, out_inds=oim[l], out_weights=owm[l]))
            for l in range(LAYERS)]
        ex[f"biased_M{M}_k6_us_per_call"] = round(graph_call_us(torch, calls, args.steps, args.warmup), 3)
    log("biased router done")
    return ex


def decode_widths_cold_and_unfused(torch, R, W, dev, args):
    """Verify widths M in {1, 2, 8} at H=4096 with the gate matrices cold: 40
    calls per step from a 256-matrix pool (537 MB, twice the Infinity Cache),
    fused (router_fwd) and unfused (the projection as a library fp32 GEMM
    writing fp32 logits to HBM, then router_topk_from_logits on them: the two
    back-to-back launches of the pages' isolated A/B gate).  The unfused
    path's GEMM reads fp32 copies of the gate (twice the bytes of bf16: the
    library has no bf16 x bf16 -> fp32 GEMM through torch here), stated with
    the numbers."""
    ex = {}
    H, E, k, pool = 4096, 256, 8, 256
    groups = pool // LAYERS
    wpool = W.torch_gaussian_bf16((pool, E, H), 1.0 / H ** 0.5, seed=70, device=dev)
    for M in (1, 2, 8):
        x = W.torch_rms_normalised_bf16((LAYERS, M, H), seed=71 + M, device=dev)
        oi = torch.empty((LAYERS, M, k), dtype=torch.int32, device=dev)
        ow = torch.empty((LAYERS, M, k), dtype=torch.float32, device=dev)
        graphs = [GraphTimer(torch, [(lambda l=l, g=g: R.router_fwd(x[l], wpool[g * LAYERS + l], None, k, W.SOFTMAX,
                                                                   True, out_inds=oi[l], out_weights=ow[l]))
                                     for l in range(LAYERS)]) for g in range(groups)]
        wall, ev_ms = timed_replays(torch, graphs, args.steps, args.warmup)
        ex[f"decode_M{M}_H4096_cold_us_per_call"] = round(wall * 1e6 / (args.steps * LAYERS), 3)
        del graphs
    log("verify widths (cold) done")
    # unfused A/B on a smaller cold pool of fp32 gates (40 x 4 MiB per step, 6 steps' worth)
    upool = 240
    wf = wpool[:upool].float().transpose(1, 2).contiguous()  # [pool, H, E] fp32: logits = x @ wf
    del wpool
    ugroups = upool // LAYERS
    for M in (1, 2, 8):
        x = W.torch_rms_normalised_bf16((LAYERS, M, H), seed=71 + M, device=dev).float()
        lg = torch.empty((LAYERS, M, E), dtype=torch.float32, device=dev)
        oi = torch.empty((LAYERS, M, k), dtype=torch.int32, device=dev)
        ow = torch.empty((LAYERS, M, k), dtype=torch.float32, device=dev)

        def unfused(l, widx, x=x, lg=lg, oi=oi, ow=ow):
            def run():
                torch.mm(x[l], wf[widx], out=lg[l])
                R.router_topk_from_logits(lg[l], None, k, W.SOFTMAX, True, out_inds=oi[l], out_weights=ow[l])
            return run

        try:
            graphs = [GraphTimer(torch, [unfused(l, g * LAYERS + l) for l in range(LAYERS)]) for g in range(ugroups)]
        except RuntimeError as exc:  # library GEMM not capturable
            log(f"unfused A/B skipped: {exc}")
            break
        wall, _ = timed_replays(torch, graphs, args.steps, args.warmup)
        ex[f"decode_M{M}_H4096_unfused_gemm_plus_topk_cold_us_per_call"] = round(wall * 1e6 / (args.steps * LAYERS), 3)
        del graphs
    ex["decode_unfused_note"] = ("unfused = torch.mm fp32 GEMM (fp32 copy of the gate, 2x its bf16 bytes) "
                                 "writing logits + router_topk_from_logits, two launches per call")
    del wf
    log("fused vs unfused A/B done")
    return ex


def block_scaled_extras(torch, R, W, dev, args, fmt):
    """The router on a block-scaled gate (fmt "mxfp4" or "mxfp8") at the decode
    widths of --<fmt>-widths, H=7168: 40 calls per step, each with its own gate
    from a pool larger than twice the Infinity Cache (MXFP4: 600 matrices,
    585 MB; MXFP8: 320 matrices, 606 MB), cold; and the 8192-token prefill."""
    ex = {}
    H, E, k = 7168, 256, 8
    if fmt == "mxfp4":
        pool, gate, fwd, widths = 600, W.torch_mxfp4_gate, R.router_fwd_mxfp4, args.mxfp4_widths
        code_bytes, seeds = E * H // 2, (30, 31, 35, 36, 37)
    else:
        pool, gate, fwd, widths = 320, W.torch_mxfp8_gate, R.router_fwd_mxfp8, args.mxfp8_widths
        code_bytes, seeds = E * H, (40, 41, 45, 46, 47)
    codes, scales = gate(pool, E, H, seed=seeds[0], device=dev)
    groups = pool // LAYERS
    for M in [int(m) for m in widths.split(",")]:
        x = W.torch_rms_normalised_bf16((LAYERS, M, H), seed=seeds[1] + M, device=dev)
        oi = torch.empty((LAYERS, M, k), dtype=torch.int32, device=dev)
        ow = torch.empty((LAYERS, M, k), dtype=torch.float32, device=dev)

        def call(l, widx, x=x, oi=oi, ow=ow):
            return lambda: fwd(x[l], codes[widx], scales[widx], None, k, W.SOFTMAX,
                               True, out_inds=oi[l], out_weights=ow[l])

        graphs = [GraphTimer(torch, [call(l, g * LAYERS + l) for l in range(LAYERS)])
                  for g in range(groups)]
        wall, ev_ms = timed_replays(torch, graphs, args.steps, args.warmup)
        launch_us = ev_ms * 1e3 / (args.steps * LAYERS)
        ex[f"{fmt}_decode_M{M}_H7168_us_per_call"] = round(wall * 1e6 / (args.steps * LAYERS), 3)
        ex[f"{fmt}_decode_M{M}_H7168_launch_us"] = round(launch_us, 3)
        if M == 1:
            algo = code_bytes + E * H // 32 + M * H * 2 + M * k * 8  # codes + scales + x + outputs
            ex[f"{fmt}_decode_M1_bytes_per_launch"] = algo
            ex[f"{fmt}_decode_M1_hbm_frac"] = round(algo / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            ex[f"{fmt}_decode_M1_traffic"] = committed_traffic(MX_TRAFFIC_SUMMARY[fmt])
        del graphs
    del codes, scales
    # prefill: M=8192 tokens over four cold 117 MB activations, one gate
    M = 8192
    xs = W.torch_gaussian_bf16((4, M, H), 1.0, seed=seeds[2], device=dev)
    pc, psc = gate(1, E, H, seed=seeds[3], device=dev)
    bp = W.torch_uniform_f32(E, -0.02, 0.02, seed=seeds[4], device=dev)
    pi = torch.empty((M, k), dtype=torch.int32, device=dev)
    pw = torch.empty((M, k), dtype=torch.float32, device=dev)
    calls = [(lambda i=i: fwd(xs[i], pc[0], psc[0], bp, k, W.SOFTMAX, True,
                              out_inds=pi, out_weights=pw)) for i in range(4)]
    p_us = graph_call_us(torch, calls, max(args.steps // 2, 2), 2)
    tflops = 2.0 * M * E * H / (p_us * 1e-6) / 1e12
    ex[f"{fmt}_prefill_M8192_H7168_event_us_per_call"] = round(p_us, 2)
    ex[f"{fmt}_prefill_M8192_tokens_per_s"] = round(M / (p_us * 1e-6), 0)
    ex[f"{fmt}_prefill_mfma_frac"] = round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)
    del xs
    log(f"{fmt} done")
    return ex


def gather_extras(torch, R, W, dev, args):
    """Routed gather + shared-expert add at the MTP1 pair (M=2, k=6, D=7168): 40
    calls per step, each layer's 12 expert output rows from a 1600-layer pool
    (275 MB, cold); the table variant on a table the router produced; all-remote
    routes; and M=4096, k=8 (bandwidth)."""
    ex = {}
    M, k, D, pool = 2, 6, 7168, 1600
    ys = W.torch_gaussian_bf16((pool, M * k, D), 1.0, seed=40, device=dev)
    shared = W.torch_gaussian_bf16((LAYERS, M, D), 1.0, seed=41, device=dev)
    u = W.torch_uniform_f32(LAYERS * M * k, 0.05, 1.0, seed=42, device=dev).view(LAYERS, M, k)
    wts = (u / u.sum(dim=2, keepdim=True)).contiguous()
    out = torch.empty((LAYERS, M, D), dtype=torch.bfloat16, device=dev)
    disjoint = torch.arange(M * k, dtype=torch.int32, device=dev).view(M, k)   # 12 distinct rows
    remote = torch.full((M, k), -1, dtype=torch.int32, device=dev)
    groups = pool // LAYERS

    def timed(rows_of, label):
        graphs = [GraphTimer(torch, [(lambda l=l, g=g: R.router_gather_shared_add(
            ys[g * LAYERS + l], rows_of, wts[l], shared[l], out=out[l])) for l in range(LAYERS)])
            for g in range(groups)]
        wall, ev_ms = timed_replays(torch, graphs, args.steps, args.warmup)
        n = args.steps * LAYERS
        ex[f"gather_M2_k6_D7168_{label}_us_per_call"] = round(wall * 1e6 / n, 3)
        ex[f"gather_M2_k6_D7168_{label}_launch_us"] = round(ev_ms * 1e3 / n, 3)
        return ev_ms * 1e3 / n

    launch_us = timed(disjoint, "disjoint")
    algo = M * k * D * 2 + 2 * M * D * 2 + M * k * 8  # rows read + shared + out + map/weights
    ex["gather_M2_k6_D7168_bytes_per_launch"] = algo
    ex["gather_M2_k6_D7168_hbm_frac"] = round(algo / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    ex["gather_M2_k6_D7168_traffic"] = committed_traffic(GATHER_TRAFFIC_SUMMARY, GATHER_SOURCES)
    if args.gather_disjoint_only:
        return ex
    timed(remote, "all_remote")

    # the table variant, on the table the decode router emits for one biased MTP1 pair
    case = W.verify_table_case(2, seed=4, k=k, biased=True)
    xb = torch.from_numpy(case.x.view("int16")).view(torch.bfloat16).to(dev)
    wg = torch.from_numpy(case.w.view("int16")).view(torch.bfloat16).to(dev)
    bb = torch.from_numpy(case.bias).to(dev)
    tab = R.router_fwd_route_table(xb, wg, bb, k, case.scoring, case.renorm)
    ex["gather_table_unique_experts"] = int(tab["unique_count"].item())
    graphs = [GraphTimer(torch, [(lambda l=l, g=g: R.router_gather_shared_add_table(
        ys[g * LAYERS + l], tab, tab["weights"], shared[l], out=out[l])) for l in range(LAYERS)])
        for g in range(groups)]
    wall, ev_ms = timed_replays(torch, graphs, args.steps, args.warmup)
    ex["gather_M2_k6_D7168_table_us_per_call"] = round(wall * 1e6 / (args.steps * LAYERS), 3)
    del graphs, ys

    # bandwidth: M=4096 tokens, k=8 distinct rows each (470 MB of expert rows)
    Mb, kb = 4096, 8
    yb = W.torch_gaussian_bf16((Mb * kb, D), 1.0, seed=43, device=dev)
    sb = W.torch_gaussian_bf16((Mb, D), 1.0, seed=44, device=dev)
    rb = torch.arange(Mb * kb, dtype=torch.int32, device=dev).view(Mb, kb)
    ub = W.torch_uniform_f32(Mb * kb, 0.05, 1.0, seed=45, device=dev).view(Mb, kb)
    wb = (ub / ub.sum(dim=1, keepdim=True)).contiguous()
    ob = torch.empty((Mb, D), dtype=torch.bfloat16, device=dev)
    # eight back-to-back calls per graph, like the other sections (one call
    # per replay would add each replay's launch gap to the call)
    b_us = graph_call_us(torch, [lambda: R.router_gather_shared_add(yb, rb, wb, sb, out=ob)] * 8,
                         max(args.steps // 2, 2), 2)
    bbytes = Mb * kb * D * 2 + 2 * Mb * D * 2 + Mb * kb * 8
    ex["gather_M4096_k8_D7168_event_us_per_call"] = round(b_us, 2)
    ex["gather_M4096_k8_D7168_hbm_frac"] = round(bbytes / (b_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    del yb
    log("gather done")
    return ex


def gemm1_extras(torch, R, W, dev, args):
    """Expert GEMM1 on the unique-route table at the MTP1 pair: M=2, k=6, E=256
    experts of F=4096 (gate and up, 2 x 2048) by D=7168 in bf16 (15 GB of expert
    weights); 40 calls per step, each on the table one router call produced for
    its own pair of tokens, so every call reads its unique experts' weights cold."""
    ex = {}
    M, k, E, F, D = 2, 6, 256, 4096, 7168
    log(f"generating expert weights: {E}x{F}x{D} bf16")
    w1 = torch.empty((E, F, D), dtype=torch.bfloat16, device=dev)
    for e0 in range(0, E, 16):
        w1[e0:e0 + 16] = W.torch_gaussian_bf16((16, F, D), 0.02, seed=60 + e0, device=dev)
    gate = W.torch_gaussian_bf16((E, D), 1.0 / D ** 0.5, seed=61, device=dev)
    bias = W.torch_uniform_f32(E, -0.05, 0.05, seed=62, device=dev)
    xs = W.torch_rms_normalised_bf16((LAYERS, M, D), seed=63, device=dev)
    tables = [R.router_fwd_route_table(xs[l], gate, bias, k, W.SQRT_SOFTPLUS, True) for l in range(LAYERS)]
    torch.cuda.synchronize()
    uniq = [int(t["unique_count"].item()) for t in tables]
    outs = torch.empty((LAYERS, M * k, F), dtype=torch.bfloat16, device=dev)
    g = GraphTimer(torch, [(lambda l=l: R.router_expert_gemm1_table(xs[l], w1, tables[l], k, out=outs[l]))
                           for l in range(LAYERS)])
    wall, ev_ms = timed_replays(torch, [g], max(args.steps // 2, 2), 2)
    n = max(args.steps // 2, 2) * LAYERS
    launch_us = ev_ms * 1e3 / n
    mean_u = sum(uniq) / len(uniq)
    algo = mean_u * F * D * 2 + M * D * 2 + M * k * F * 2  # unique experts' weights + x + the M*k rows written
    ex["gemm1_M2_k6_F4096_D7168_us_per_call"] = round(wall * 1e6 / n, 2)
    ex["gemm1_M2_k6_F4096_D7168_launch_us"] = round(launch_us, 2)
    ex["gemm1_mean_unique_experts"] = round(mean_u, 2)
    ex["gemm1_bytes_per_launch"] = round(algo)
    ex["gemm1_hbm_frac"] = round(algo / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    ex["gemm1_traffic"] = committed_traffic(GEMM1_TRAFFIC_SUMMARY, GEMM1_SOURCES)
    del g, w1
    log("gemm1 done")
    return ex


def topk_extras(torch, R, W, dev, args):
    ex = {}
    lg = torch.randn((4, 4096, 256), device=dev, dtype=torch.float32) * 2 ** 0.5
    ti = torch.empty((4, 4096, 8), dtype=torch.int32, device=dev)
    tw = torch.empty((4, 4096, 8), dtype=torch.float32, device=dev)
    calls = [(lambda i=i: R.router_topk_from_logits(lg[i], None, 8, out_inds=ti[i], out_weights=tw[i]))
             for i in range(4)]
    t_us = graph_call_us(torch, calls, max(args.steps // 2, 2), 2)
    ex["topk_M4096_event_us_per_call"] = round(t_us, 3)
    ex["topk_M4096_GBs"] = round((4096 * 256 * 4 + 4096 * 64) / (t_us * 1e-6) / 1e9, 1)
    log("top-k done")
    return ex


def prefill_extras(torch, R, W, dev, args):
    ex = {}
    M, H, E = 8192, 7168, 256
    xs = W.torch_gaussian_bf16((4, M, H), 1.0, seed=11, device=dev)   # 470 MB: cold X
    wp = W.torch_gaussian_bf16((E, H), 1.0 / H ** 0.5, seed=12, device=dev)
    bp = W.torch_uniform_f32(E, -0.02, 0.02, seed=13, device=dev)
    pi = torch.empty((M, 8), dtype=torch.int32, device=dev)
    pw = torch.empty((M, 8), dtype=torch.float32, device=dev)
    calls = [(lambda i=i: R.router_fwd(xs[i], wp, bp, 8, W.SOFTMAX, True, out_inds=pi, out_weights=pw))
             for i in range(4)]
    p_us = graph_call_us(torch, calls, max(args.steps // 2, 2), 2)
    flops = 2.0 * M * E * H
    tflops = flops / (p_us * 1e-6) / 1e12
    ex["prefill_M8192_H7168_event_us_per_call"] = round(p_us, 2)
    ex["prefill_M8192_tokens_per_s"] = round(M / (p_us * 1e-6), 0)
    ex["prefill_mfma_tflops"] = round(tflops, 1)
    ex["prefill_mfma_frac"] = round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)
    algo_bytes = M * H * 2 + E * H * 2 + E * 4 + M * 64
    ex["prefill_hbm_frac"] = round(algo_bytes / (p_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    ex["prefill_roofline"] = {
        "bound": "mfma",
        "kernel": "prefill_router_kernel",
        "achieved": round(tflops, 1),
        "peak": MFMA_BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "traffic": committed_traffic(PREFILL_TRAFFIC_SUMMARY, PREFILL_SOURCES),
        "flops_per_launch": flops,
        "algorithmic_bytes_per_launch": algo_bytes,
        "launch_us": round(p_us, 2),
        "launch_timing": "HIP event pair on the launching stream around the timed graph replays / launch count",
    }
    # the same call with X cache-hot: one 117 MB activation (inside the 256 MB
    # Infinity Cache) every call
    hot_us = graph_call_us(torch, calls[:1] * 4, max(args.steps // 2, 2), 2)
    ex["prefill_M8192_H7168_hot_x_event_us_per_call"] = round(hot_us, 2)
    ex["prefill_hot_x_mfma_frac"] = round(flops / (hot_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    # context: the vendor GEMM (hipBLASLt through torch) on the same projection, logits only
    xf = xs[0]
    wpt = wp.t().contiguous()  # [H, E]: no transposed view reaches the library GEMM
    try:
        mm_us = graph_call_us(torch, [lambda: torch.mm(xf, wpt)] * 4, max(args.steps // 2, 2), 2)
        ex["context_torch_mm_bf16_logits_only_us"] = round(mm_us, 2)
    except RuntimeError as exc:  # library GEMM not capturable
        log(f"torch.mm context skipped: {exc}")
    log("prefill done")
    return ex


def size_extras(torch, R, W, dev, args):
    """router_fwd across batch sizes (H=7168, E=256, k=8, softmax with a
    U(-0.02,0.02) bias, one activation per size, four calls per graph): which
    kernel takes each size and what it costs."""
    ex = {}
    H, E, k = 7168, 256, 8
    w = W.torch_gaussian_bf16((E, H), 1.0 / H ** 0.5, seed=21, device=dev)
    b = W.torch_uniform_f32(E, -0.02, 0.02, seed=22, device=dev)
    for M in (16, 64, 128, 256, 257, 512, 1024, 2048, 4096):
        x = W.torch_gaussian_bf16((M, H), 1.0, seed=23, device=dev)
        oi = torch.empty((M, k), dtype=torch.int32, device=dev)
        ow = torch.empty((M, k), dtype=torch.float32, device=dev)
        us = graph_call_us(torch, [lambda: R.router_fwd(x, w, b, k, W.SOFTMAX, True, out_inds=oi, out_weights=ow)] * 4,
                           max(args.steps // 2, 2), 2)
        ex[f"sizes_M{M}_H7168_us_per_call"] = round(us, 2)
        del x
    log("sizes done")
    return ex


def floor_extras(torch, W, dev, args):
    """Launch-floor probes on the single-token decode router's grid (256
    workgroups, one per expert at E=256): each adds one ingredient of the
    router's launch to the one before (libfloorprobes.so, measurement only).
    Timed like the headline: 40 launches per step in a HIP graph, each on its
    own gate-sized matrix from a 160-matrix (587 MB) pool."""
    import ctypes
    ex = {}
    lib = ctypes.CDLL(os.path.join(ROOT, "gate_projection_top_amd", "libfloorprobes.so"))
    P, ci = ctypes.c_void_p, ctypes.c_int
    lib.floor_empty.argtypes = [ci, ci, P]
    lib.floor_read.argtypes = [P, ci, ci, P, P]
    lib.floor_ticket.argtypes = [P, ci, ci, P, P, P, P, ci, P]
    lib.floor_latency.argtypes = [P, P, ci, P, P]
    E, H = 256, 7168
    n16 = H * 2 // 16
    pool = torch.randn((POOL, E, H), device=dev, dtype=torch.bfloat16)
    out = torch.zeros(2 * E + 1, dtype=torch.float32, device=dev)  # floor_read: one float per workgroup
    ctr = torch.zeros(16 * 17, dtype=torch.int32, device=dev)
    slots = torch.zeros(E * 2, dtype=torch.int32, device=dev)
    epoch = torch.zeros(1, dtype=torch.int32, device=dev)

    def stream():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"floor probe failed: {rc}")

    probes = {
        "empty": lambda m: check(lib.floor_empty(E, 256, stream())),
        "empty_1x64": lambda m: check(lib.floor_empty(1, 64, stream())),
        "empty_256x64": lambda m: check(lib.floor_empty(E, 64, stream())),
        "empty_256x320": lambda m: check(lib.floor_empty(E, 320, stream())),
        "empty_512x256": lambda m: check(lib.floor_empty(2 * E, 256, stream())),
        "read": lambda m: check(lib.floor_read(ctypes.c_void_p(pool[m].data_ptr()), n16, E,
                                               ctypes.c_void_p(out.data_ptr()), stream())),
        "ticket": lambda m: check(lib.floor_ticket(ctypes.c_void_p(pool[m].data_ptr()), n16, E,
                                                   ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ctr.data_ptr()),
                                                   ctypes.c_void_p(slots.data_ptr()),
                                                   ctypes.c_void_p(epoch.data_ptr()), 0, stream())),
        "handoff": lambda m: check(lib.floor_ticket(ctypes.c_void_p(pool[m].data_ptr()), n16, E,
                                                    ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ctr.data_ptr()),
                                                    ctypes.c_void_p(slots.data_ptr()),
                                                    ctypes.c_void_p(epoch.data_ptr()), 1, stream())),
        # the same bytes on other grids: 512 x 7 KiB and 128 x 28 KiB
        "read_512x7k": lambda m: check(lib.floor_read(ctypes.c_void_p(pool[m].data_ptr()), n16 // 2, 2 * E,
                                                      ctypes.c_void_p(out.data_ptr()), stream())),
        "read_128x28k": lambda m: check(lib.floor_read(ctypes.c_void_p(pool[m].data_ptr()), 2 * n16, E // 2,
                                                       ctypes.c_void_p(out.data_ptr()), stream())),
        "handoff_128x28k": lambda m: check(lib.floor_ticket(ctypes.c_void_p(pool[m].data_ptr()), 2 * n16, E // 2,
                                                            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ctr.data_ptr()),
                                                            ctypes.c_void_p(slots.data_ptr()),
                                                            ctypes.c_void_p(epoch.data_ptr()), 1, stream())),
        "handoff_after_publish": lambda m: check(lib.floor_ticket(ctypes.c_void_p(pool[m].data_ptr()), n16, E,
                                                                  ctypes.c_void_p(out.data_ptr()),
                                                                  ctypes.c_void_p(ctr.data_ptr()),
                                                                  ctypes.c_void_p(slots.data_ptr()),
                                                                  ctypes.c_void_p(epoch.data_ptr()), 3, stream())),
        "handoff_fixed": lambda m: check(lib.floor_ticket(ctypes.c_void_p(pool[m].data_ptr()), n16, E,
                                                          ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ctr.data_ptr()),
                                                          ctypes.c_void_p(slots.data_ptr()),
                                                          ctypes.c_void_p(epoch.data_ptr()), 2, stream())),
    }
    groups = POOL // LAYERS
    for name, fn in probes.items():
        graphs = [GraphTimer(torch, [(lambda l=l, g=g: fn(g * LAYERS + l)) for l in range(LAYERS)])
                  for g in range(groups)]
        _, ev_ms = timed_replays(torch, graphs, args.steps, args.warmup)
        ex[f"floor_{name}_us_per_launch"] = round(ev_ms * 1e3 / (args.steps * LAYERS), 3)
        del graphs
    # dependent round trips, in-kernel clock (100 MHz): atomic, coherent load, cold load
    lat = torch.zeros(4, dtype=torch.float32, device=dev)
    scratch = torch.zeros(1024, dtype=torch.int32, device=dev)
    acc = [0.0, 0.0, 0.0]
    runs = 8
    for r in range(runs):
        check(lib.floor_latency(ctypes.c_void_p(scratch.data_ptr()), ctypes.c_void_p(pool[97 + r].data_ptr()), 64,
                                ctypes.c_void_p(lat.data_ptr()), stream()))
        torch.cuda.synchronize()
        v = lat.tolist()
        for i in range(3):
            acc[i] += v[i] / runs
    ex["floor_atomic_rtt_us"] = round(acc[0] / 100.0, 3)
    ex["floor_coherent_load_rtt_us"] = round(acc[1] / 100.0, 3)
    ex["floor_cold_load_rtt_us"] = round(acc[2] / 100.0, 3)
    del pool
    # the practical HBM read ceiling: a 2 GiB buffer (8x the Infinity Cache)
    # read once per launch with 16-byte loads, at several grid sizes
    # (plain loads, then non-temporal ones)
    lib.floor_stream_read.argtypes = [P, ctypes.c_int64, ci, P]
    lib.floor_stream_read_nt.argtypes = [P, ctypes.c_int64, ci, P]
    nbytes = 2 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
    sums = torch.zeros(16384, dtype=torch.float32, device=dev)
    best = 0.0
    for label, fn in (("", lib.floor_stream_read), ("nt_", lib.floor_stream_read_nt)):
        best_mode = 0.0
        for grid in (1024, 2048, 4096, 8192, 16384):
            run = lambda: check(fn(ctypes.c_void_p(buf.data_ptr()), nbytes, grid,
                                   ctypes.c_void_p(sums.data_ptr()), stream()))
            run()
            torch.cuda.synchronize()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            start.record()
            for _ in range(reps):
                run()
            end.record()
            torch.cuda.synchronize()
            tbs = nbytes * reps / (start.elapsed_time(end) * 1e-3) / 1e12
            ex[f"hbm_stream_read_{label}{grid}wg_TBs"] = round(tbs, 3)
            best_mode = max(best_mode, tbs)
        ex[f"hbm_stream_read_{label}best_mode_TBs"] = round(best_mode, 3)
        best = max(best, best_mode)
    ex["hbm_stream_read_best_TBs"] = round(best, 3)
    ex["hbm_stream_read_best_frac_of_8TBs"] = round(best / (HBM_PEAK_GBS / 1000.0), 4)
    del buf, sums
    # the 8192-token prefill's main loop taken apart (prefill_stream_probe.hip):
    # its X and W load streams alone and together, W always hitting, and the
    # loop with its fragment reads and MFMAs; four activations cycled (cold X)
    lib.pf_stream_probe.argtypes = [P, P, ci, ci, ci, P, P]
    Mx, Hx = 8192, 7168
    xs = W.torch_gaussian_bf16((4, Mx, Hx), 1.0, seed=21, device=dev)
    wq = W.torch_gaussian_bf16((256, Hx), 1.0 / Hx ** 0.5, seed=22, device=dev)
    po = torch.zeros(Mx // 128 * 4, dtype=torch.float32, device=dev)
    for mode, name in ((0, "x_and_w"), (1, "x_only"), (2, "w_only"), (3, "x_and_w_hits"), (4, "main_loop")):
        def launch(i, mode=mode):
            check(lib.pf_stream_probe(ctypes.c_void_p(xs[i % 4].data_ptr()), ctypes.c_void_p(wq.data_ptr()),
                                      Mx, Hx, mode, ctypes.c_void_p(po.data_ptr()), stream()))
        for i in range(4):
            launch(i)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        start.record()
        for i in range(reps):
            launch(i)
        end.record()
        torch.cuda.synchronize()
        ex[f"prefill_streams_{name}_us"] = round(start.elapsed_time(end) * 1e3 / reps, 2)
    del xs, wq, po
    log("floor probes done")
    return ex


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, seconds):
    """The oracle (as written, single thread) on M=1 H=7168 router calls for ~`seconds`."""
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
            "cpu": cpu_model(),
            "sample": f"{n} single-token router calls (H=7168, E=256, k=8, softmax, renorm) "
                      f"through the C oracle, one thread"}


def cpu_baseline_threads(W, seconds):
    """The same oracle calls on every host core this process may use (at most
    16 threads): independent calls in parallel threads (the C oracle runs
    without the interpreter lock), reported as µs per call of throughput."""
    import threading
    import oracle

    orc = oracle.get()
    case = W.metric_case(0)
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(16, avail))
    counts = [0] * threads
    t0 = time.perf_counter()
    deadline = t0 + seconds

    def work(i):
        while time.perf_counter() < deadline:
            orc.router(case.x, case.w, case.bias, case.k, case.scoring, case.renorm)
            counts[i] += 1

    pool = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    el = time.perf_counter() - t0
    n = sum(counts)
    log(f"cpu baseline ({threads} threads): {n} oracle calls in {el:.1f}s")
    return {"value": round(el * 1e6 / max(n, 1), 2), "unit": "µs/call", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{n} single-token router calls (H=7168, E=256, k=8, softmax, renorm), "
                      f"independent calls on {threads} threads"}


if __name__ == "__main__":
    main()
