"""The row-sharded oracle helper returns exactly the single-call oracle's bytes."""
import numpy as np

import oracle
import oracle_par
from gate_projection_top_amd import workloads as W


def test_sharded_router_equals_single_call():
    orc = oracle.get()
    case = W.prefill_case(M=37, H=64, seed=5)
    one = orc.router(case.x, case.w, case.bias, case.k, case.scoring, case.renorm)
    for threads in (1, 5, 37, 64):
        many = oracle_par.router(orc, case.x, case.w, case.bias, case.k, case.scoring, case.renorm,
                                 threads=threads)
        for a, b in zip(one, many):
            assert a.shape == b.shape and a.tobytes() == b.tobytes()


def test_sharded_mx_routers_equal_single_call():
    orc = oracle.get()
    for make, fn, par in ((W.mxfp4_case, orc.router_mxfp4, oracle_par.router_mxfp4),
                          (W.mxfp8_case, orc.router_mxfp8, oracle_par.router_mxfp8)):
        case = make(23, H=128, seed=3, with_bias=True)
        one = fn(case.x, case.elems, case.scales, case.bias, case.k, case.scoring, case.renorm)
        many = par(orc, case.x, case.elems, case.scales, case.bias, case.k, case.scoring, case.renorm,
                   threads=4)
        for a, b in zip(one, many):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
