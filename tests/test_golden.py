"""The tiny-router fixture still matches the generator and the oracle (no GPU)."""
import json
import os

import numpy as np

import oracle
from gate_projection_top_amd import workloads as W

from golden.make_golden import digest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_router.json")


def _cases():
    return [W.tiny_case(0)] + W.tiny_tie_cases(0)


def test_golden_inputs_and_oracle():
    with open(GOLDEN) as f:
        gold = json.load(f)["cases"]
    o = oracle.get()
    cases = _cases()
    assert len(gold) == len(cases)
    for g, c in zip(gold, cases):
        assert g["name"] == c.name
        assert g["inputs_sha256"] == digest(c.x, c.w, c.bias), c.name
        inds, wts, lg, _ = o.router(c.x, c.w, c.bias, c.k, c.scoring, c.renorm)
        assert inds.tolist() == g["inds"], c.name
        assert [[f"{v:08x}" for v in r] for r in wts.view(np.uint32).tolist()] == g["weights_f32_bits"]
        assert [[f"{v:08x}" for v in r] for r in lg.view(np.uint32).tolist()] == g["logits_f32_bits"]


def test_golden_tie_rows_pick_lower_index():
    """In every tie row the selected tied expert is the lowest-indexed of its tie group."""
    o = oracle.get()
    for c in W.tiny_tie_cases(0):
        inds, _, lg, _ = o.router(c.x, c.w, c.bias, c.k, c.scoring, c.renorm)
        row = lg[0]
        for j, e in enumerate(inds[0]):
            tied = np.flatnonzero(row == row[e])
            chosen = [i for i in inds[0] if row[i] == row[e]]
            assert chosen == sorted(tied)[:len(chosen)], (c.name, j, tied, inds)
