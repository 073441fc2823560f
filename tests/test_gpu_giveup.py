"""The decode finisher's bounded wait, forced from the host.

With the wait limit at 0 a finisher gives a row up unless its logits are
already in place at the first look: the row must then come out as index -1
with a NaN weight in each of its k places and the sticky status must say so;
a row not given up must be the oracle's.  Whatever happened, the next calls
(limit restored) must match the oracle exactly, on the same shapes and on
others, eagerly and under graph replay: values published after a finisher
stopped waiting carry an older launch's tag and never pass for a later
launch's.  Every kernel still exits normally (the limit only shortens waits).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.compare import check_router, check_table
from gate_projection_top_amd import router as R
from gate_projection_top_amd import workloads as W
from gpu_util import bf16_dev, f32_dev, host, say

pytestmark = pytest.mark.gpu

DEFAULT_LIMIT_US = 100000
SHAPES = [("expert kernel M=1 H=7168", lambda s: W.metric_case(500 + s)),
          ("expert kernel M=2 biased", lambda s: W.biased_case(2, seed=510 + s)),
          ("split kernel M=8", lambda s: W.decode_case(8, seed=520 + s)),
          ("split kernel M=64 biased", lambda s: W.biased_case(64, seed=530 + s))]


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(autouse=True)
def restore_limit():
    yield
    R.set_decode_wait_limit_us(DEFAULT_LIMIT_US)


def _call(case):
    gi, gw, gl = R.router_fwd(bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k, case.scoring,
                              case.renorm, return_logits=True)
    torch.cuda.synchronize()
    return host(gi), host(gw), host(gl)


def _rows_exact_or_given_up(orc, case, gi, gw, gl):
    """Rows given up are -1 / NaN throughout; every other row meets rule (b)."""
    given_up = np.all(gi == -1, axis=1)
    for t in np.flatnonzero(given_up):
        assert np.all(np.isnan(gw[t])), (case.name, t, gw[t])
    rows = np.flatnonzero(~given_up)
    assert np.all(gi[rows] >= 0), case.name
    if rows.size:
        check_router(orc, case, gi[rows], gw[rows], gl[rows], rows=rows)
    return int(given_up.sum())


@pytest.mark.parametrize("name,make", SHAPES, ids=[s[0] for s in SHAPES])
def test_forced_give_up_then_exact(orc, name, make):
    R.init()
    R.status(clear=True)
    say(f"give-up at limit 0: {name}")
    R.set_decode_wait_limit_us(0)
    total_given_up = 0
    for s in range(3):
        case = make(s)
        gi, gw, gl = _call(case)
        total_given_up += _rows_exact_or_given_up(orc, case, gi, gw, gl)
    flags = R.status(clear=True)
    assert (flags & R.STATUS_WAIT_LIMIT) == (R.STATUS_WAIT_LIMIT if total_given_up else 0), (flags, total_given_up)
    R.set_decode_wait_limit_us(DEFAULT_LIMIT_US)
    # the next calls: same shape (same and new inputs), then every other shape
    for s in (2, 3, 4):
        case = make(s)
        say(f"after give-up: {case.name}")
        gi, gw, gl = _call(case)
        check_router(orc, case, gi, gw, gl)
    for other_name, other in SHAPES:
        case = other(7)
        say(f"after give-up, other shape: {case.name}")
        gi, gw, gl = _call(case)
        check_router(orc, case, gi, gw, gl)
    assert R.status(clear=True) == 0


def test_forced_give_up_then_exact_graph_replays(orc):
    """The give-up, then graph replays of a table call with inputs rewritten between
    replays: every replay exact on every field."""
    R.init()
    R.status(clear=True)
    cases = [W.biased_case(2, seed=600 + s) for s in range(8)]
    x = torch.empty((2, cases[0].x.shape[1]), dtype=torch.bfloat16, device="cuda:0")
    w = torch.empty((cases[0].w.shape[0], cases[0].w.shape[1]), dtype=torch.bfloat16, device="cuda:0")
    b = torch.empty(cases[0].w.shape[0], dtype=torch.float32, device="cuda:0")
    out = {n: torch.empty(12 if n != "unique_count" else 1, dtype=torch.int32, device="cuda:0")
           for n in ("unique_ids", "token_mask", "slot_to_unique", "unique_count")}
    out["inds"] = torch.empty((2, 6), dtype=torch.int32, device="cuda:0")
    out["weights"] = torch.empty((2, 6), dtype=torch.float32, device="cuda:0")
    out["logits"] = torch.empty((2, 256), dtype=torch.float32, device="cuda:0")

    def load(case):
        x.copy_(torch.from_numpy(case.x.view(np.int16)).view(torch.bfloat16))
        w.copy_(torch.from_numpy(case.w.view(np.int16)).view(torch.bfloat16))
        b.copy_(torch.from_numpy(case.bias))

    def call():
        R.router_fwd_m2_table(x, w, b, 6, W.SQRT_SOFTPLUS, True, out=out)

    load(cases[0])
    R.set_decode_wait_limit_us(0)
    say("table call at limit 0")
    call()
    torch.cuda.synchronize()
    R.set_decode_wait_limit_us(DEFAULT_LIMIT_US)
    R.status(clear=True)
    graph = torch.cuda.CUDAGraph()
    load(cases[1])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for i, case in enumerate(cases[1:]):
        say(f"replay {i} after give-up ({case.name})")
        load(case)
        graph.replay()
        torch.cuda.synchronize()
        got = {n: host(t) for n, t in out.items()}
        check_router(orc, case, got["inds"], got["weights"], got["logits"])
        check_table(orc, got["inds"], {n: got[n] for n in ("unique_ids", "token_mask", "slot_to_unique",
                                                            "unique_count")})
    assert R.status(clear=True) == 0
