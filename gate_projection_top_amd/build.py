"""Build librouter.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m gate_projection_top_amd.build

Flags: -O3 without fast-math and without FP contraction, IEEE denormals,
and packed-FP32 instructions disabled in device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "librouter.so")

SOURCES = ["router_api.cpp", "topk_kernel.hip", "decode_kernel.hip", "decode_expert_kernel.hip",
           "prefill_kernel.hip", "gather_kernel.hip", "gemm1_kernel.hip"]
HEADERS = ["route_common.hpp", "softmax_exp.hpp", "launch.hpp", "coherent.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


PROBE_SOURCES = ["floor_probes.hip", "prefill_stream_probe.hip"]
PROBE_LIB_PATH = os.path.join(PKG, "libfloorprobes.so")


def build_probes(out: str = PROBE_LIB_PATH, verbose: bool = False) -> str:
    """Compile the measurement probes the benchmark times (launch floor, HBM read
    ceiling, the prefill main loop's streams); not part of the router."""
    return build(out, verbose, sources=PROBE_SOURCES)


def build(out: str = LIB_PATH, verbose: bool = False, sources=None) -> str:
    """Compile every source into one shared library (always rebuilds)."""
    srcs = [os.path.join(CSRC, s) for s in (sources or SOURCES)]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; that note is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and "(ignoring feature)" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probes(verbose=True))
