"""bench.py's host-side contract, checked without a GPU: the one-GPU guard,
the rule that a committed counter summary counts only while the kernel
sources still match its digest, and the oracle's CPU timings."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for an unsupported run


def _summary(tmp_path, digest, bytes_):
    p = tmp_path / "summary.txt"
    p.write_text(f"# header\nhbm_bytes_per_launch: {bytes_}\nkernel_sources_sha256_16: {digest}\n")
    return str(p)


def test_traffic_counts_only_for_matching_sources(tmp_path):
    current = bench.kernel_source_digest(bench.KERNEL_SOURCES)
    assert bench.committed_traffic(_summary(tmp_path, current, 1234567), bench.KERNEL_SOURCES) == 1234567.0
    assert bench.committed_traffic(_summary(tmp_path, "0" * 16, 1234567), bench.KERNEL_SOURCES) is None
    assert bench.committed_traffic(str(tmp_path / "missing.txt"), bench.KERNEL_SOURCES) is None


def test_digest_covers_every_listed_source():
    # a digest over the listed files only: reordering or dropping one changes it
    names = bench.KERNEL_SOURCES
    d = bench.kernel_source_digest(names)
    assert len(d) == 16
    assert bench.kernel_source_digest(names[:-1]) != d
    for group in (bench.KERNEL_SOURCES, bench.GATHER_SOURCES, bench.GEMM1_SOURCES):
        for name in group:
            assert os.path.exists(os.path.join(ROOT, "gate_projection_top_amd", "csrc", name)), name


@pytest.mark.parametrize("fn", ["cpu_baseline", "cpu_baseline_threads"])
def test_oracle_timing_fields(fn):
    from gate_projection_top_amd import workloads as W
    out = getattr(bench, fn)(W, 0.3)
    assert out["kind"] == "oracle" and out["unit"] == "µs/call"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "router calls" in out["sample"]
