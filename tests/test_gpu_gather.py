"""router_gather_shared_add / router_gather_shared_add_table vs the oracle.

The rounding chain is fixed (fp32 products and sums in slot order, BF16,
+ shared in fp32, BF16), so the kernel must match the oracle bit for bit.
Workloads (seeded, synthetic): expert output rows and shared outputs
~ N(0,1) in bf16, router-like weights; the B70 note's route classes (same,
disjoint, cross-token overlap, within-token duplicate, all-duplicate,
all-local, all-remote) plus partly remote maps and a tie-heavy integer case;
M = 2 (the MTP1 pair) up to large M; the table variant on tables produced by
router_fwd_route_table on the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from gate_projection_top_amd import router as R
from gate_projection_top_amd import workloads as W
from gpu_util import bf16_dev, f32_dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def run_gather(case):
    out = R.router_gather_shared_add(bf16_dev(case.y), i32_dev(case.slot_rows), f32_dev(case.weights),
                                     bf16_dev(case.shared))
    torch.cuda.synchronize()
    return host(out.view(torch.int16)).view(np.uint16)


def check_exact(got, want, what):
    if not np.array_equal(got, want):
        t, d = np.argwhere(got != want)[0]
        raise AssertionError(f"{what}: [{t},{d}] gpu {got[t, d]:#06x} oracle {want[t, d]:#06x} "
                             f"({int((got != want).sum())} of {got.size} differ)")


def check_case(orc, case):
    say(f"gather {case.name}")
    got = run_gather(case)
    want = orc.gather_shared_add(case.y, case.slot_rows, case.weights, case.shared)
    check_exact(got, want, case.name)


@pytest.mark.parametrize("pattern", W.GATHER_PATTERNS)
@pytest.mark.parametrize("seed", [0, 1])
def test_route_classes_m2(orc, pattern, seed):
    check_case(orc, W.gather_case(2, 6, 7168, pattern, seed=seed))


@pytest.mark.parametrize("M,k,D", [(1, 1, 8), (1, 8, 64), (2, 3, 1032), (3, 16, 2056), (8, 8, 4096),
                                   (16, 4, 7168), (100, 6, 512)])
@pytest.mark.parametrize("pattern", ["typical", "some_remote", "ties"])
def test_shapes(orc, M, k, D, pattern):
    check_case(orc, W.gather_case(M, k, D, pattern, seed=M + k))


@pytest.mark.parametrize("M,k", [(85, 3), (32, 8), (64, 4)])
@pytest.mark.parametrize("pattern", ["typical", "some_remote"])
def test_streaming_load_threshold(orc, M, k, pattern):
    # 255 rows per call take plain row loads, 256 the non-temporal ones:
    # both sides of the switch against the oracle
    check_case(orc, W.gather_case(M, k, 1032, pattern, seed=M * k))


def test_large_m(orc):
    check_case(orc, W.gather_case(2048, 8, 4096, "some_remote", seed=5, R=3000))


def test_rows_outside_the_buffer_add_nothing(orc):
    case = W.gather_case(4, 6, 256, "typical", seed=6, R=10)
    case.slot_rows[0, 1] = 10      # one past the last row
    case.slot_rows[1, 2] = -7
    case.slot_rows[3, :] = 1 << 30
    got = run_gather(case)
    clean = case.slot_rows.copy()
    clean[(clean < -1) | (clean >= 10)] = -1
    check_exact(got, orc.gather_shared_add(case.y, clean, case.weights, case.shared), "bad rows")


def test_in_place_on_shared(orc):
    case = W.gather_case(2, 6, 7168, "overlap", seed=7)
    shared = bf16_dev(case.shared)
    out = R.router_gather_shared_add(bf16_dev(case.y), i32_dev(case.slot_rows), f32_dev(case.weights),
                                     shared, out=shared)
    torch.cuda.synchronize()
    assert out.data_ptr() == shared.data_ptr()
    check_exact(host(out.view(torch.int16)).view(np.uint16),
                orc.gather_shared_add(case.y, case.slot_rows, case.weights, case.shared), "in place")


def test_changing_inputs_under_graph_replay(orc):
    """The note's changing-input graph cases: one captured launch, new rows,
    weights, expert outputs and shared outputs written in place before every
    replay, each replay checked against the oracle."""
    M, k, D, Rr = 2, 6, 2048, 12
    first = W.gather_case(M, k, D, "typical", seed=100, R=Rr)
    y, rows, w, sh = (bf16_dev(first.y), i32_dev(first.slot_rows), f32_dev(first.weights),
                      bf16_dev(first.shared))
    out = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    R.router_gather_shared_add(y, rows, w, sh, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        R.router_gather_shared_add(y, rows, w, sh, out=out)
    for i, pattern in enumerate(W.GATHER_PATTERNS * 3):
        case = W.gather_case(M, k, D, pattern, seed=200 + i, R=Rr)
        y.copy_(bf16_dev(case.y))
        rows.copy_(i32_dev(case.slot_rows))
        w.copy_(f32_dev(case.weights))
        sh.copy_(bf16_dev(case.shared))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_exact(host(out.view(torch.int16)).view(np.uint16),
                    orc.gather_shared_add(case.y, case.slot_rows, case.weights, case.shared),
                    f"replay {i} ({pattern})")


def _table_inputs(M, k, seed):
    """A route table and weights from router_fwd_route_table on a decode case."""
    case = W.verify_table_case(M, seed=seed, k=k, biased=(M == 2))
    res = R.router_fwd_route_table(bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k,
                                   case.scoring, case.renorm)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("M,k", [(1, 8), (2, 6), (2, 8), (4, 8), (8, 8), (16, 4)])
@pytest.mark.parametrize("seed", [0, 3])
def test_table_variant(orc, M, k, seed):
    res = _table_inputs(M, k, seed)
    D = 4096
    rng = np.random.default_rng(seed + 10 * M)
    y = W.gaussian_bf16(rng, (M * k, D), 1.0)
    shared = W.gaussian_bf16(rng, (M, D), 1.0)
    say(f"gather table M={M} k={k} seed={seed}")
    out = R.router_gather_shared_add_table(bf16_dev(y), res, res["weights"], bf16_dev(shared))
    torch.cuda.synchronize()
    got = host(out.view(torch.int16)).view(np.uint16)
    mask, s2u, cnt = host(res["token_mask"]), host(res["slot_to_unique"]), int(host(res["unique_count"])[0])
    rows = orc.table_rows(mask, s2u, cnt, M, k)
    want = orc.gather_shared_add(y, rows, host(res["weights"]), shared)
    check_exact(got, want, f"table M={M} k={k}")
    # the same rows through the explicit map give the same bits
    out2 = R.router_gather_shared_add(bf16_dev(y), i32_dev(rows), res["weights"], bf16_dev(shared))
    torch.cuda.synchronize()
    check_exact(host(out2.view(torch.int16)).view(np.uint16), got, "table vs explicit rows")


def test_table_variant_rows_stay_in_the_layout(orc):
    """Identical tokens (every expert shared) and disjoint tokens give the two
    extreme compact layouts (k rows and M*k rows)."""
    for seed in (4, 7):  # seed % 10 < 5 forces experts both tokens pick
        case = W.verify_table_case(2, seed=seed, k=6, biased=True)
        res = R.router_fwd_route_table(bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k,
                                       case.scoring, case.renorm)
        torch.cuda.synchronize()
        cnt = int(host(res["unique_count"])[0])
        assert 6 <= cnt <= 12
        y = W.gaussian_bf16(np.random.default_rng(cnt), (12, 512), 1.0)
        shared = W.gaussian_bf16(np.random.default_rng(cnt + 1), (2, 512), 1.0)
        out = R.router_gather_shared_add_table(bf16_dev(y), res, res["weights"], bf16_dev(shared))
        torch.cuda.synchronize()
        rows = orc.table_rows(host(res["token_mask"]), host(res["slot_to_unique"]), cnt, 2, 6)
        assert rows.max() == sum(bin(int(m)).count("1") for m in host(res["token_mask"])[:cnt]) - 1
        check_exact(host(out.view(torch.int16)).view(np.uint16),
                    orc.gather_shared_add(y, rows, host(res["weights"]), shared), "table layout")


def test_empty_batch():
    y = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    out = R.router_gather_shared_add(y, torch.empty((0, 6), dtype=torch.int32, device="cuda"),
                                     torch.empty((0, 6), dtype=torch.float32, device="cuda"),
                                     torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert out.shape == (0, 64)
