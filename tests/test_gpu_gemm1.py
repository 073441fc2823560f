"""router_expert_gemm1_table (expert GEMM1 on the unique-route table) vs the oracle.

Each unique expert's rows must equal the exact dot products within fp32
accumulation plus one BF16 rounding: |out - exact| <= 2^-8 |exact| +
1e-4 * sum|x*w| (the router's logit bound, for the fp32 sum; 2^-8 covers the
BF16 half-ulp).  Rows past the table's compact layout must stay untouched.
Workloads (seeded, synthetic): tables from router_fwd_route_table on the
verify-width decode workload (M in {1,2,4,8}, k in {6,8}) with expert weights
~ N(0, 0.02^2) in bf16, and hand-built tables over 12 experts at F up to
1024, D up to 7168 (ragged F and D included).
"""
import numpy as np
import pytest
import torch

import oracle
from gate_projection_top_amd import router as R
from gate_projection_top_amd import workloads as W
from gpu_util import bf16_dev, f32_dev, host, say

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FA5  # a NaN pattern the kernel never writes


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def bits(t):
    return host(t.view(torch.int16)).view(np.uint16)


def run_and_check(orc, x, w1, table, k, what):
    M, D = x.shape
    E, F, _ = w1.shape
    out = torch.full((M * k, F), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    R.router_expert_gemm1_table(bf16_dev(x), bf16_dev(w1), table, k, out=out)
    torch.cuda.synchronize()
    got_bits = bits(out)
    ids, mask, cnt = (host(table["unique_ids"]), host(table["token_mask"]),
                      int(host(table["unique_count"])[0]))
    exact, ad = orc.expert_gemm1_table(x, w1, ids, mask, cnt)
    n = exact.shape[0]
    got = W.bf16_bits_to_f32(got_bits[:n]).astype(np.float64)
    err = np.abs(got - exact)
    tol = 2.0 ** -8 * np.abs(exact) + 1e-4 * ad
    if not np.all(err <= tol):
        r, f = np.unravel_index(int(np.argmax(err - tol)), err.shape)
        raise AssertionError(f"{what}: row {r} feature {f}: gpu {got[r, f]!r} exact {exact[r, f]!r} "
                             f"tol {tol[r, f]:.3e}")
    assert np.all(got_bits[n:] == SENTINEL), f"{what}: rows past the layout were written"
    return got_bits, n


def table_dict(ids, mask, cnt):
    return dict(unique_ids=i32_dev(ids), token_mask=i32_dev(mask),
                unique_count=i32_dev(np.array([cnt], np.int32)))


@pytest.mark.parametrize("M,k", [(1, 8), (2, 6), (2, 8), (4, 8), (8, 8)])
@pytest.mark.parametrize("seed", [0, 7])
def test_router_tables(orc, M, k, seed):
    case = W.verify_table_case(M, seed=seed, k=k, biased=(M == 2))
    res = R.router_fwd_route_table(bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k,
                                   case.scoring, case.renorm)
    torch.cuda.synchronize()
    rng = np.random.default_rng(100 + seed)
    w1 = W.gaussian_bf16(rng, (256, 64, case.x.shape[1]), 0.02)
    say(f"gemm1 router table M={M} k={k} seed={seed}")
    run_and_check(orc, case.x, w1, res, k, f"router table M={M} k={k}")


@pytest.mark.parametrize("F,D", [(16, 64), (100, 1032), (1024, 7168), (64, 200)])
@pytest.mark.parametrize("kind", ["same", "disjoint", "overlap"])
def test_hand_tables(orc, F, D, kind):
    rng = np.random.default_rng(F + D)
    M, k, E = 2, 6, 12
    if kind == "same":
        row = rng.choice(E, k, replace=False)
        inds = np.stack([row, row])
    elif kind == "disjoint":
        inds = rng.permutation(E)[:2 * k].reshape(2, k)
    else:
        inds = np.stack([rng.choice(E, k, replace=False) for _ in range(M)])
    ids, mask, s2u, cnt = orc.route_table(inds.astype(np.int32))
    x = W.gaussian_bf16(rng, (M, D), 1.0)
    w1 = W.gaussian_bf16(rng, (E, F, D), 1.0 / np.sqrt(D))
    say(f"gemm1 hand {kind} F={F} D={D}")
    run_and_check(orc, x, w1, table_dict(ids, mask, cnt), k, f"{kind} F={F} D={D}")


def test_sixteen_tokens(orc):
    rng = np.random.default_rng(3)
    M, k, E, F, D = 16, 4, 20, 96, 512
    inds = np.stack([rng.choice(E, k, replace=False) for _ in range(M)]).astype(np.int32)
    ids, mask, s2u, cnt = orc.route_table(inds)
    x = W.gaussian_bf16(rng, (M, D), 1.0)
    w1 = W.gaussian_bf16(rng, (E, F, D), 0.05)
    run_and_check(orc, x, w1, table_dict(ids, mask, cnt), k, "16 tokens")


def test_unknown_expert_writes_nothing(orc):
    rng = np.random.default_rng(4)
    M, k, E, F, D = 2, 3, 8, 32, 128
    ids, mask, s2u, cnt = orc.route_table(np.array([[1, 2, 3], [2, 4, 5]], np.int32))
    x = W.gaussian_bf16(rng, (M, D), 1.0)
    w1 = W.gaussian_bf16(rng, (E, F, D), 0.1)
    bad = ids.copy()
    bad[1] = E + 3            # expert 2 (both tokens: rows 1 and 2) is out of range
    out = torch.full((M * k, F), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    R.router_expert_gemm1_table(bf16_dev(x), bf16_dev(w1), table_dict(bad, mask, cnt), k, out=out)
    torch.cuda.synchronize()
    b = bits(out)
    assert np.all(b[1:3] == SENTINEL) and np.all(b[3:] != SENTINEL) and np.all(b[0] != SENTINEL)


def test_repeat_calls_are_deterministic(orc):
    rng = np.random.default_rng(5)
    ids, mask, s2u, cnt = orc.route_table(np.array([[0, 3, 5, 7], [3, 5, 8, 9]], np.int32))
    x = bf16_dev(W.gaussian_bf16(rng, (2, 7168), 1.0))
    w1 = bf16_dev(W.gaussian_bf16(rng, (10, 256, 7168), 0.01))
    tab = table_dict(ids, mask, cnt)
    ref = bits(R.router_expert_gemm1_table(x, w1, tab, 4))
    for _ in range(5):
        assert np.array_equal(bits(R.router_expert_gemm1_table(x, w1, tab, 4)), ref)


def test_chain_router_gemm1_gather(orc):
    """Router table -> GEMM1 rows -> gather from the same compact rows, all on the device:
    the gather reads exactly the rows GEMM1 wrote (checked bit for bit against the
    oracle's gather on the GPU's GEMM1 output)."""
    M, k, F = 2, 6, 256
    case = W.verify_table_case(M, seed=2, k=k, biased=True)
    res = R.router_fwd_route_table(bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k,
                                   case.scoring, case.renorm)
    rng = np.random.default_rng(9)
    w1 = W.gaussian_bf16(rng, (256, F, case.x.shape[1]), 0.02)
    y = R.router_expert_gemm1_table(bf16_dev(case.x), bf16_dev(w1), res, k)
    shared = W.gaussian_bf16(rng, (M, F), 1.0)
    out = R.router_gather_shared_add_table(y, res, res["weights"], bf16_dev(shared))
    torch.cuda.synchronize()
    cnt = int(host(res["unique_count"])[0])
    rows = orc.table_rows(host(res["token_mask"]), host(res["slot_to_unique"]), cnt, M, k)
    want = orc.gather_shared_add(bits(y), rows, host(res["weights"]), shared)
    assert np.array_equal(bits(out), want)
