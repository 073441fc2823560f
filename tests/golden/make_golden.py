"""Write tests/golden/tiny_router.json from the CPU oracle (and nothing else).

The fixture freezes the oracle's answer on the tiny router workload (M=4,
H=256, E=16, k=2, softmax, no bias, renorm; seed 0) and on its four
single-token exact-tie rows, together with a digest of the generated inputs.
It guards against silent drift of either the input generator or the oracle:
a change to either must regenerate this file in the same commit and say why.

Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from gate_projection_top_amd import workloads as W  # noqa: E402


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def record(case, o):
    inds, wts, lg, ad = o.router(case.x, case.w, case.bias, case.k, case.scoring, case.renorm)
    return {
        "name": case.name,
        "M": case.M, "H": case.H, "E": case.E, "k": case.k,
        "scoring": case.scoring, "renorm": bool(case.renorm),
        "inputs_sha256": digest(case.x, case.w, case.bias),
        "inds": inds.tolist(),
        "weights_f32_bits": [[f"{v:08x}" for v in row] for row in wts.view(np.uint32).tolist()],
        "logits_f32_bits": [[f"{v:08x}" for v in row] for row in lg.view(np.uint32).tolist()],
    }


def main():
    o = oracle.get()
    cases = [W.tiny_case(0)] + W.tiny_tie_cases(0)
    out = {
        "source": "written by tests/golden/make_golden.py from the CPU oracle only",
        "workload": "tiny router M=4 H=256 E=16 k=2 softmax, no bias, renorm; seed 0; "
                    "plus four single-token rows with exact logit ties around the k=2 cut",
        "cases": [record(c, o) for c in cases],
    }
    with open(os.path.join(HERE, "tiny_router.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
