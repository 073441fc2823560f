"""Edge-case shapes and a seeded sweep, fused router and standalone top-k vs the oracle.

Covers what the workload configs do not: H that is not a multiple of the
32-wide (decode) or 64-wide (prefill) k-step, E that is not a multiple of 16
or 4 (down to E = 1), k = 1 and k = 16 (the limit), renorm off, both
scorings with and without bias, ragged last prefill tiles, and M on every
side of the decode/prefill and split-count boundaries (64/65 rows; 64/65 and
128/129 tiles of 128 rows).  Every case is compared under rule (b) (rule (a)
for the top-k); inputs come from seeded generators only.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.compare import check_router, check_topk
from gate_projection_top_amd import router as R
from gate_projection_top_amd import workloads as W
from gpu_util import bf16_dev, f32_dev, host, say

pytestmark = pytest.mark.gpu

SM, SSP = W.SOFTMAX, W.SQRT_SOFTPLUS


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def run_case(orc, case):
    say(f"router {case.name}")
    gi, gw, gl = R.router_fwd(bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k,
                              case.scoring, case.renorm, return_logits=True)
    torch.cuda.synchronize()
    return check_router(orc, case, host(gi), host(gw), host(gl))


# (M, H, E, k, scoring, bias, renorm)
DECODE_EDGES = [
    (1, 8, 256, 8, SM, False, True),        # one 8-wide chunk of H
    (1, 200, 256, 8, SM, True, True),       # H % 32 != 0
    (3, 1000, 100, 4, SSP, True, True),     # E % 16 != 0, H % 32 != 0
    (7, 520, 16, 1, SM, False, True),       # k = 1, one expert block
    (2, 64, 1, 1, SM, False, True),         # E = 1
    (5, 64, 17, 3, SSP, False, False),      # E = 17: two blocks, one mostly padding; raw weights
    (16, 7176, 256, 16, SM, True, True),    # k = 16, H just past 7168
    (64, 4096, 255, 9, SSP, True, True),    # four row blocks, E % 4 != 0
    (80, 1000, 100, 4, SSP, True, True),    # five row blocks: several splits per CU's share
    (256, 520, 256, 8, SM, True, True),     # M at the decode limit: 16 row blocks, one split
    (241, 256, 17, 16, SM, False, True),    # ragged last row block, k = 16 with E = 17
    (9, 4096, 256, 8, SM, False, False),    # softmax without renorm: full-row probabilities
    (4, 4096, 256, 8, SM, True, True),      # the most tokens of the one-expert kernel
    (5, 4096, 256, 8, SM, True, True),      # the fewest tokens of the split kernel
]


@pytest.mark.parametrize("M,H,E,k,scoring,bias,renorm", DECODE_EDGES)
def test_decode_edges(orc, M, H, E, k, scoring, bias, renorm):
    run_case(orc, W.shape_case(M, H, E, k, scoring, bias, renorm, seed=M * 7 + H))


PREFILL_EDGES = [
    (257, 200, 256, 8, SM, True, True),     # first prefill size, H % 64 != 0
    (385, 1000, 100, 4, SSP, True, True),   # ragged fourth tile, E % 16 != 0
    (300, 520, 17, 16, SM, False, True),    # k = 16 with E = 17
    (1000, 64, 256, 1, SSP, False, False),  # k = 1, a single k-step
    (8192, 64, 256, 8, SM, True, True),     # 64 tiles: the last size with 4 splits
    (8193, 64, 256, 8, SM, True, True),     # 65 tiles: 2 splits, one row in the last tile
    (16384, 64, 256, 8, SSP, True, True),   # 128 tiles: the last size with 2 splits
    (16385, 64, 256, 8, SM, False, True),   # 129 tiles: no split
    (700, 4096, 256, 8, SM, False, False),  # softmax without renorm
]


@pytest.mark.parametrize("M,H,E,k,scoring,bias,renorm", PREFILL_EDGES)
def test_prefill_edges(orc, M, H, E, k, scoring, bias, renorm):
    run_case(orc, W.shape_case(M, H, E, k, scoring, bias, renorm, seed=M + H))


def test_random_sweep(orc):
    """40 seeded random shapes across both paths and every option."""
    rng = np.random.default_rng(2024)
    for i in range(40):
        M = int(rng.choice([1, 2, 3, 8, 16, 33, 64, 65, 130, 257, 600]))
        H = int(rng.integers(1, 130)) * 8
        E = int(rng.choice([8, 16, 31, 64, 100, 128, 200, 256]))
        k = int(rng.integers(1, min(E, 16) + 1))
        scoring = int(rng.integers(0, 2))
        bias = bool(rng.integers(0, 2))
        renorm = bool(rng.integers(0, 2))
        run_case(orc, W.shape_case(M, H, E, k, scoring, bias, renorm, seed=1000 + i))


@pytest.mark.parametrize("M,E,k", [(1, 1, 1), (5, 3, 3), (64, 17, 16), (1000, 255, 8), (33, 256, 16)])
@pytest.mark.parametrize("scoring,bias,renorm", [(SM, False, True), (SM, True, False),
                                                 (SSP, True, True)])
def test_topk_edges(orc, M, E, k, scoring, bias, renorm):
    rng = np.random.default_rng(M * 31 + E)
    logits = (rng.standard_normal((M, E)) * 1.5).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32) if bias else None
    say(f"topk M={M} E={E} k={k} scoring={scoring} bias={bias} renorm={renorm}")
    gi, gw = R.router_topk_from_logits(f32_dev(logits), f32_dev(b), k, scoring, renorm)
    torch.cuda.synchronize()
    ri, rw = orc.topk_from_logits(logits, b, k, scoring, renorm)
    check_topk(host(gi), host(gw), ri, rw, what=f"topk M={M} E={E} k={k}")
