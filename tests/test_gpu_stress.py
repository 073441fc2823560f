"""Bounded stress run of the decode router: 2000 seeded random calls (no GPU fault sought).

Every call draws its shape at random within the documented limits (M up to
the decode maximum of 256, any E up to 256 including sizes that are not a
multiple of the expert block, k up to min(E, 16), H any multiple of 8 up to
7168, both scorings, bias on or off, renormalisation on or off), so the one-expert
kernel (up to 4 tokens), the split kernel (5 to 256 tokens) and the
allocation-free entry point all run many times in one process with their
workspaces reused across shapes.  Outputs live inside larger buffers whose
words before and after the output carry a canary pattern: a write outside
the output, or a change to the inputs, fails the call.  Every call is checked
against the oracle (logits within the bound, selection by the band rule);
calls made without a logits output must give the same bytes as the same call
made with one.  The sticky status must stay clear throughout.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.compare import check_router
from gate_projection_top_amd import router as R
from gate_projection_top_amd import workloads as W
from gpu_util import DEV, bf16_dev, f32_dev, host, say

pytestmark = pytest.mark.gpu

CALLS_PER_CHUNK = 500
CHUNKS = 4
PAD = 64                      # canary words on each side of every output
CANARY = 0x5AC3A55A
M_CHOICES = [1, 1, 1, 2, 2, 3, 4, 4, 5, 6, 7, 8, 8, 9, 12, 16, 17, 31, 32, 33, 48, 63, 64, 80, 128, 200]
H_CHOICES = [8, 16, 64, 136, 256, 520, 1024, 2048, 4096, 7168]
H_WEIGHTS = [1, 1, 2, 2, 3, 2, 3, 2, 2, 2]
E_CHOICES = [1, 2, 7, 16, 33, 64, 100, 128, 255, 256, 256, 256]


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _padded(n: int, dtype):
    buf = torch.full((n + 2 * PAD,), CANARY, dtype=torch.int32, device=DEV)
    return buf, buf[PAD:PAD + n].view(dtype)


def _canaries_intact(buf, n) -> bool:
    b = host(buf)
    return bool(np.all(b[:PAD] == CANARY) and np.all(b[PAD + n:] == CANARY))


def _draw(rng, index):
    M = int(rng.choice(M_CHOICES))
    H = int(rng.choice(H_CHOICES, p=np.array(H_WEIGHTS) / sum(H_WEIGHTS)))
    E = int(rng.choice(E_CHOICES))
    k = int(rng.integers(1, min(E, 16) + 1))
    scoring = int(rng.integers(0, 2))
    with_bias = bool(rng.integers(0, 2))
    renorm = bool(rng.integers(0, 2))
    return W.shape_case(M, H, E, k, scoring, with_bias, renorm, seed=10000 + index)


def _call(case, noalloc, want_logits):
    M, H = case.x.shape
    E, k = case.w.shape[0], case.k
    x, w, b = bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias)
    ib, inds = _padded(M * k, torch.int32)
    wb, wts = _padded(M * k, torch.float32)
    lb, lg = _padded(M * E, torch.float32) if want_logits else (None, None)
    fn = R.router_fwd_noalloc if noalloc else R.router_fwd
    fn(x, w, b, k, case.scoring, case.renorm, out_inds=inds.view(M, k), out_weights=wts.view(M, k),
       logits_out=None if lg is None else lg.view(M, E))
    torch.cuda.synchronize()
    assert _canaries_intact(ib, M * k), f"{case.name}: write outside the index output"
    assert _canaries_intact(wb, M * k), f"{case.name}: write outside the weight output"
    if lb is not None:
        assert _canaries_intact(lb, M * E), f"{case.name}: write outside the logits output"
    assert np.array_equal(host(x.view(torch.int16)), case.x.view(np.int16)), f"{case.name}: x changed"
    assert np.array_equal(host(w.view(torch.int16)), case.w.view(np.int16)), f"{case.name}: w changed"
    return (host(inds).reshape(M, k), host(wts).reshape(M, k),
            None if lg is None else host(lg).reshape(M, E))


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_random_decode_calls(orc, chunk):
    R.init()
    R.status(clear=True)
    rng = np.random.default_rng(7000 + chunk)
    kernels = {"expert": 0, "split": 0, "noalloc": 0}
    for i in range(CALLS_PER_CHUNK):
        index = chunk * CALLS_PER_CHUNK + i
        case = _draw(rng, index)
        M = case.x.shape[0]
        noalloc = M <= R.NOALLOC_MAX_M and rng.integers(0, 3) == 0
        with_logits = rng.integers(0, 4) != 0
        if i % 100 == 0:
            say(f"stress chunk {chunk} call {i}: {case.name} noalloc={noalloc} logits={with_logits}")
        gi, gw, gl = _call(case, noalloc, True)
        check_router(orc, case, gi, gw, gl)
        if not with_logits:
            gi2, gw2, _ = _call(case, noalloc, False)
            assert gi2.tobytes() == gi.tobytes() and gw2.tobytes() == gw.tobytes(), case.name
        kernels["noalloc" if noalloc else ("expert" if M <= 4 else "split")] += 1
    say(f"stress chunk {chunk}: {kernels}")
    assert min(kernels.values()) > 0, kernels
    assert R.status(clear=True) == 0
