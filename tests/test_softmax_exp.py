"""The routing kernels' double-precision exp (csrc/softmax_exp.hpp) on the CPU.

The softmax scores exp(l - max l) of the router (dense_router_decode notes,
"DenseRouterDecodeKernel": softmax scoring in a wider type) are computed on
the device by a table-driven exp; these tests pin it to exact decimal
arithmetic: the table of 2^(j/64) pairs and the Cody-Waite constants in the
header, and the function itself (its host build, with the header's table)
within one unit in the last place of exp(x) over the shifts a softmax row
produces (x <= 0), its range edges and reduction boundaries.
"""
import ctypes
import math
import os
import re
import struct
import subprocess
import tempfile
from decimal import Decimal, getcontext

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "gate_projection_top_amd", "csrc", "softmax_exp.hpp")
getcontext().prec = 60
LN2 = Decimal(2).ln()


def _hexfloats(text):
    return [float.fromhex(t) for t in re.findall(r"-?0x[0-9a-fA-F.]+p[-+]?\d+", text)]


def _header():
    src = open(HDR).read()
    consts = {}
    for name in ("kExpInvL", "kExpLhi", "kExpLlo"):
        m = re.search(r"constexpr double %s = (-?0x[0-9a-fA-F.]+p[-+]?\d+);" % name, src)
        consts[name] = float.fromhex(m.group(1))
    body = src[src.index("kExp2Table[64][2] = {"):]
    body = body[:body.index("};")]
    vals = _hexfloats(body)
    assert len(vals) == 128
    return consts, np.array(vals, dtype=np.float64).reshape(64, 2)


def test_table_pairs_are_the_nearest_doubles():
    _, tab = _header()
    for j in range(64):
        exact = (LN2 * j / 64).exp()
        hi, lo = tab[j]
        assert hi == float(exact), j                       # nearest double to 2^(j/64)
        assert lo == float(exact - Decimal(hi)), j         # nearest double to the rest
        assert abs(Decimal(hi) + Decimal(lo) - exact) <= exact * Decimal(2) ** -105


def test_reduction_constants():
    c, _ = _header()
    L = LN2 / 64
    assert c["kExpInvL"] == float(64 / LN2)
    bits = struct.unpack("<Q", struct.pack("<d", c["kExpLhi"]))[0]
    assert bits & ((1 << 17) - 1) == 0                      # k * LHI exact for |k| < 2^17
    assert abs(Decimal(c["kExpLhi"]) - L) < L * Decimal(2) ** -35
    assert c["kExpLlo"] == float(L - Decimal(c["kExpLhi"]))
    # the pair is exact to half an ulp of LLO (2^-99): with |k| < 2^17 the
    # reduced argument is off by at most 2^-82, far below its last place
    assert abs(Decimal(c["kExpLhi"]) + Decimal(c["kExpLlo"]) - L) <= Decimal(math.ulp(c["kExpLlo"])) / 2


SHIM = r"""
#include "softmax_exp.hpp"
extern "C" double exp_host(double x, const double* tab)
{
    int k = 0;
    const double r = gpt::exp_reduce(x, k);
    const int j = k & 63;
    return gpt::exp_finish(r, k, tab[2 * j], tab[2 * j + 1]);
}
"""


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    d = tmp_path_factory.mktemp("expshim")
    src = d / "shim.hip"
    src.write_text(SHIM)
    so = d / "shim.so"
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-I", os.path.dirname(HDR), str(src), "-o", str(so)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-2000:])
    lib = ctypes.CDLL(str(so))
    lib.exp_host.restype = ctypes.c_double
    lib.exp_host.argtypes = [ctypes.c_double, ctypes.POINTER(ctypes.c_double)]
    _, tab = _header()
    tab = np.ascontiguousarray(tab.reshape(-1))
    ptr = tab.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    return lambda x: lib.exp_host(float(x), ptr), tab


def _ulps(got, x):
    exact = Decimal(x).exp()
    ref = float(exact)
    if ref == 0.0:
        return 0.0 if got == 0.0 else math.inf
    # distance in units of the last place of the correctly rounded value
    # (the spacing of denormals below 2^-1022)
    return abs(Decimal(got) - exact) / Decimal(math.ulp(ref))


def _cases():
    rng = np.random.default_rng(20261202)
    xs = [0.0, -0.0, -1e-300, -5e-324, -1e-17, -1e-9, -0.5, -1.0, -2.0, -10.0, -700.0,
          -708.39, -708.4, -709.0, -744.0, -745.0, -745.1, -745.2, -746.0, -799.0, -800.0, -801.0, -1e5,
          -3.4e38, 0.5, 1.0, 10.0, 88.7]
    xs += list(-rng.exponential(2.0, 3000))                    # typical softmax shifts
    xs += list(rng.uniform(-800.0, 0.0, 1000))
    # near the reduction's rounding points: x = (k + 1/2) ln2/64 and k ln2/64
    L = math.log(2) / 64
    for kk in rng.integers(-73000, 0, 400):
        for off in (-0.5, 0.5, 0.0):
            b = (float(kk) + off) * L
            xs += [b, math.nextafter(b, -math.inf), math.nextafter(b, math.inf)]
    # shifts between fp32 logits, as the kernels form them
    l = rng.standard_normal(2000).astype(np.float32) * np.float32(3)
    xs += [float(np.float64(a) - np.float64(l.max())) for a in l]
    return xs


def test_within_one_ulp(shim):
    f, _ = shim
    worst = 0.0
    for x in _cases():
        got = f(x)
        if x < -800.0:
            assert got == 0.0, x
            continue
        e = _ulps(got, x)
        worst = max(worst, float(e))
        assert e <= 1, (x, got, float(Decimal(x).exp()), float(e))
    assert worst > 0.0  # the comparison saw rounding at all


def test_exact_points(shim):
    f, _ = shim
    assert f(0.0) == 1.0
    assert f(-0.0) == 1.0
    for j in range(64):
        # x = -j ln2/64 exactly as the kernels would see it lands on table entries
        x = -j * math.log(2) / 64
        assert _ulps(f(x), x) <= 1
    assert f(-1000.0) == 0.0 and f(-800.0) == 0.0
