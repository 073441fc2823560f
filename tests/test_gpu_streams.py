"""Fused calls on several streams at once, each stream on its own workspace.

Calls are enqueued on three side streams in an interleaved order with no
synchronisation between them, so their launches can overlap on the device;
every call must still match the oracle.  A stream beyond the device's
workspace count is refused with ROUTER_ERR_BUSY (nothing launched, outputs
untouched) until a stream gives its workspace back.
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

MAKERS = [lambda s: W.metric_case(700 + s),
          lambda s: W.biased_case(2, seed=710 + s),
          lambda s: W.decode_case(8, seed=720 + s),
          lambda s: W.biased_case(64, seed=730 + s),
          lambda s: W.shape_case(300, 1024, 256, 8, W.SOFTMAX, True, True, seed=740 + s)]


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def test_overlapping_streams_each_exact(orc):
    R.init()
    R.status(clear=True)
    streams = [torch.cuda.Stream() for _ in range(3)]
    try:
        for rnd in range(4):
            say(f"streams round {rnd}")
            cases = [make(rnd * 10 + i) for i, make in enumerate(MAKERS)] * 2
            dev_in = [(bf16_dev(c.x), bf16_dev(c.w), f32_dev(c.bias)) for c in cases]
            outs = [(torch.empty((c.x.shape[0], c.k), dtype=torch.int32, device=DEV),
                     torch.empty((c.x.shape[0], c.k), dtype=torch.float32, device=DEV),
                     torch.empty((c.x.shape[0], c.w.shape[0]), dtype=torch.float32, device=DEV)) for c in cases]
            for s in streams:
                s.wait_stream(torch.cuda.current_stream())
            # round-robin over the streams, no waits between them
            for i, (c, (x, w, b), (oi, ow, ol)) in enumerate(zip(cases, dev_in, outs)):
                with torch.cuda.stream(streams[i % len(streams)]):
                    R.router_fwd(x, w, b, c.k, c.scoring, c.renorm, out_inds=oi, out_weights=ow, logits_out=ol)
            torch.cuda.synchronize()
            for c, (oi, ow, ol) in zip(cases, outs):
                check_router(orc, c, host(oi), host(ow), host(ol))
        assert R.status(clear=True) == 0
    finally:
        torch.cuda.synchronize()
        for s in streams:
            R.release_stream(s)


def test_stream_beyond_the_workspaces_is_refused_until_one_is_released(orc):
    R.init()
    case = W.metric_case(750)
    x, w = bf16_dev(case.x), bf16_dev(case.w)
    held = []
    refused = None
    try:
        for _ in range(R.MAX_STREAMS + 1):
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            oi = torch.full((1, case.k), -5, dtype=torch.int32, device=DEV)
            ow = torch.full((1, case.k), -5.0, dtype=torch.float32, device=DEV)
            try:
                with torch.cuda.stream(s):
                    R.router_fwd(x, w, None, case.k, case.scoring, case.renorm, out_inds=oi, out_weights=ow)
            except R.RouterError as exc:
                assert exc.code == R.ERR_BUSY, exc
                torch.cuda.synchronize()
                assert np.all(host(oi) == -5) and np.all(host(ow) == -5.0)  # nothing launched
                refused = s
                break
            held.append(s)
        assert refused is not None, "a stream beyond the workspace count was not refused"
        assert 1 <= len(held) <= R.MAX_STREAMS
        # give one back: the refused stream now gets a workspace and an exact result
        torch.cuda.synchronize()
        R.release_stream(held.pop())
        oi = torch.empty((1, case.k), dtype=torch.int32, device=DEV)
        ow = torch.empty((1, case.k), dtype=torch.float32, device=DEV)
        ol = torch.empty((1, case.w.shape[0]), dtype=torch.float32, device=DEV)
        with torch.cuda.stream(refused):
            R.router_fwd(x, w, None, case.k, case.scoring, case.renorm, out_inds=oi, out_weights=ow, logits_out=ol)
        torch.cuda.synchronize()
        check_router(orc, case, host(oi), host(ow), host(ol))
        held.append(refused)
    finally:
        torch.cuda.synchronize()
        for s in held:
            R.release_stream(s)


def test_first_call_under_capture_is_refused_not_allocated():
    """A fresh process whose first fused call is made under stream capture
    gets ROUTER_ERR_NOT_INITIALIZED (no allocation inside the capture), and
    after router_init the same capture succeeds and replays exactly."""
    import os
    import subprocess
    import sys
    code = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from gate_projection_top_amd import router as R
x = torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda:0")
w = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda:0")
oi = torch.empty((1, 2), dtype=torch.int32, device="cuda:0")
ow = torch.empty((1, 2), dtype=torch.float32, device="cuda:0")
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
code = None
try:
    with torch.cuda.graph(g):
        R.router_fwd(x, w, None, 2, out_inds=oi, out_weights=ow)
except R.RouterError as exc:
    code = exc.code
print("first", code, flush=True)
R.init()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):
    R.router_fwd(x, w, None, 2, out_inds=oi, out_weights=ow)
g.replay()
torch.cuda.synchronize()
print("after", oi.cpu().tolist(), flush=True)
"""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code, root], capture_output=True, text=True, timeout=240)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-2000:]
    assert f"first {R.ERR_NOT_INITIALIZED}" in r.stdout, r.stdout
    assert "after [[0, 1]]" in r.stdout, r.stdout
