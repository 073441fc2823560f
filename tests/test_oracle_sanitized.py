"""The oracle's C under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

oracle.c is rebuilt with ``-fsanitize=address,undefined`` (every report fatal)
and the pins, the golden fixture and the sharded helper are run again against
that build in a child Python with the ASan runtime preloaded.  Any
out-of-bounds access, use after free or undefined operation in the oracle on
those inputs ends the child with a report.  Two mistakes planted in copies of
oracle.c (a read one element past a row, a shift past the width of int) show
that each sanitizer is really armed in this set-up.
"""
import os
import subprocess
import sys

import pytest

import oracle

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
SUITES = ["test_oracle_pins.py", "test_golden.py", "test_oracle_par.py"]


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's ASan runtime is not installed")
    return path


def _env(lib):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = _asan_runtime() + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["ORACLE_LIB"] = lib
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    return env


def _build(tmp_path, name, source=None):
    out = str(tmp_path / name)
    oracle.build(out, sources=[source] if source else None, extra_flags=SAN_FLAGS)
    return out


def _run_pins(lib, only=None):
    args = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-x", "--capture=sys"]
    args += [os.path.join(TESTS, s) for s in SUITES]
    if only:
        args += ["-k", only]
    return subprocess.run(args, cwd=ROOT, env=_env(lib), capture_output=True, text=True, timeout=600)


def _planted(tmp_path, name, old, new):
    with open(oracle.SOURCES[0]) as f:
        src = f.read()
    assert src.count(old) == 1, old
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    return _build(tmp_path, "lib" + name + ".so", str(path))


def test_pins_clean_under_sanitizers(tmp_path):
    lib = _build(tmp_path, "liboracle_san.so")
    r = _run_pins(lib)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert " passed" in r.stdout, report


def test_sanitizers_catch_planted_mistakes(tmp_path):
    oob = _planted(tmp_path, "oob", "for (int64_t i = 0; i < H; ++i) {", "for (int64_t i = 0; i <= H; ++i) {")
    r = _run_pins(oob, only="logits_small_integers")
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
    shift = _planted(tmp_path, "shift", "token_mask[pos] |= 1 << token;", "token_mask[pos] |= 1 << (token + 31);")
    r = _run_pins(shift, only="table_hand_cases")
    assert r.returncode != 0 and "runtime error" in r.stderr, r.stderr[-2000:]
