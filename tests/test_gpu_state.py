"""Workspace state across calls.

The decode kernel's partial slots (sentinel-filled between calls) and arrival
counters, and the prefill kernel's counters, are restored by every call.  So
any sequence of shapes, and any number of HIP-graph replays, must give the
same bytes as the first call of each shape.
"""
import numpy as np
import pytest
import torch

from gate_projection_top_amd import router as R
from gate_projection_top_amd import workloads as W
from gpu_util import bf16_dev, f32_dev, say

pytestmark = pytest.mark.gpu


def _shapes():
    """(name, callable writing into preallocated outputs, output tensors)."""
    out = []

    def fwd_case(name, case, logits=True):
        x, w, b = bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias)
        M, E = case.x.shape[0], case.w.shape[0]
        oi = torch.empty((M, case.k), dtype=torch.int32, device="cuda:0")
        ow = torch.empty((M, case.k), dtype=torch.float32, device="cuda:0")
        ol = torch.empty((M, E), dtype=torch.float32, device="cuda:0") if logits else None
        fn = lambda: R.router_fwd(x, w, b, case.k, case.scoring, case.renorm, out_inds=oi,
                                  out_weights=ow, logits_out=ol)
        out.append((name, fn, [t for t in (oi, ow, ol) if t is not None]))

    fwd_case("decode M=1 H=7168", W.metric_case(5))
    fwd_case("decode M=8 H=4096", W.decode_case(8, seed=6), logits=False)
    fwd_case("biased M=64", W.biased_case(64, seed=7))
    fwd_case("biased M=16", W.biased_case(16, seed=8), logits=False)
    fwd_case("ragged E=100 k=4 M=3 H=256", W.decode_case(3, H=256, seed=9, E=100, k=4))
    fwd_case("tiny E=16 k=2", W.tiny_case(1))
    fwd_case("decode M=200 H=512", W.prefill_case(M=200, H=512, seed=10))
    fwd_case("prefill M=520 H=512", W.prefill_case(M=520, H=512, seed=12))

    case = W.biased_case(2, seed=11)
    x, w, b = bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias)
    t = {n: torch.empty(2 * case.k if n != "unique_count" else 1, dtype=torch.int32,
                        device="cuda:0")
         for n in ("unique_ids", "token_mask", "slot_to_unique", "unique_count")}
    t["inds"] = torch.empty((2, case.k), dtype=torch.int32, device="cuda:0")
    t["weights"] = torch.empty((2, case.k), dtype=torch.float32, device="cuda:0")
    out.append(("m2 table", lambda: R.router_fwd_m2_table(x, w, b, case.k, case.scoring,
                                                           case.renorm, out=t), list(t.values())))

    case8 = W.verify_table_case(8, seed=13)
    x8, w8 = bf16_dev(case8.x), bf16_dev(case8.w)
    t8 = {n: torch.empty(8 * case8.k if n != "unique_count" else 1, dtype=torch.int32,
                         device="cuda:0")
          for n in ("unique_ids", "token_mask", "slot_to_unique", "unique_count")}
    t8["inds"] = torch.empty((8, case8.k), dtype=torch.int32, device="cuda:0")
    t8["weights"] = torch.empty((8, case8.k), dtype=torch.float32, device="cuda:0")
    out.append(("M=8 table", lambda: R.router_fwd_route_table(x8, w8, None, case8.k, case8.scoring,
                                                              case8.renorm, out=t8),
                list(t8.values())))

    lg = f32_dev(W.adversarial_logits(64, seed=12).logits)
    ti = torch.empty((64, 8), dtype=torch.int32, device="cuda:0")
    tw = torch.empty((64, 8), dtype=torch.float32, device="cuda:0")
    out.append(("topk M=64", lambda: R.router_topk_from_logits(lg, None, 8, out_inds=ti,
                                                               out_weights=tw), [ti, tw]))
    return out


def _snapshot(tensors):
    return [t.clone() for t in tensors]


def _same(a, b):
    return all(torch.equal(x.view(torch.int32), y.view(torch.int32)) for x, y in zip(a, b))


def _poison(tensors):
    for t in tensors:
        t.view(torch.int32).fill_(-7)


def test_shape_sequence_restores_state():
    R.init()
    shapes = _shapes()
    refs = []
    for name, fn, outs in shapes:
        say(f"state ref {name}")
        fn()
        torch.cuda.synchronize()
        refs.append(_snapshot(outs))
    rng = np.random.default_rng(0)
    for it in range(4):
        for i in rng.permutation(len(shapes)):
            name, fn, outs = shapes[i]
            _poison(outs)
            fn()
            torch.cuda.synchronize()
            assert _same(outs, refs[i]), (it, name)


def test_graph_replays_match_eager():
    R.init()
    shapes = _shapes()
    refs = []
    for name, fn, outs in shapes:
        fn()
        torch.cuda.synchronize()
        refs.append(_snapshot(outs))
    graph = torch.cuda.CUDAGraph()
    say("capturing every shape in one graph")
    with torch.cuda.graph(graph):
        for _, fn, _ in shapes:
            fn()
    torch.cuda.synchronize()
    for rep in range(5):
        for _, _, outs in shapes:
            _poison(outs)
        say(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for (name, _, outs), ref in zip(shapes, refs):
            assert _same(outs, ref), (rep, name)
        # eager calls between replays, in another order
        for name, fn, outs in reversed(shapes):
            fn()
        torch.cuda.synchronize()
        for (name, _, outs), ref in zip(shapes, refs):
            assert _same(outs, ref), (rep, "eager", name)
