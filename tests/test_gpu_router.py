"""router_fwd / router_fwd_m2_table / router_fwd_route_table vs the oracle (rules b and c) and
self-consistency.

Workloads (seeded, synthetic): the tiny E=16 router with exact-tie rows, the
verify-width decode router (M in {1,2,8}, H=4096, unit-RMS activations), the
single-token H=7168 decode, the DeepSeek-V4-style biased sqrt-softplus router
(M in {1,2,16,64}, k=6, table at M=2) and prefill shapes up to M=8192,
H=7168 (every row at full size).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.compare import check_router, check_table
from gate_projection_top_amd import router as R
from gate_projection_top_amd import workloads as W
from gpu_util import bf16_dev, f32_dev, host, say
import oracle_par

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def run_fwd(case):
    gi, gw, gl = R.router_fwd(bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k,
                              case.scoring, case.renorm, return_logits=True)
    torch.cuda.synchronize()
    return host(gi), host(gw), host(gl)


def test_tiny_router_and_ties(orc):
    for case in [W.tiny_case(0)] + W.tiny_tie_cases(0):
        say(f"router {case.name}")
        gi, gw, gl = run_fwd(case)
        check_router(orc, case, gi, gw, gl)
        ri, rw, rl, _ = orc.router(case.x, case.w, case.bias, case.k, case.scoring, case.renorm)
        # tie rows: duplicated gate rows give bitwise-equal logits on the GPU too,
        # and the lower index must win
        assert np.array_equal(gi, ri), (case.name, gi, ri)


@pytest.mark.parametrize("M", [1, 2, 8])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_verify_widths(orc, M, seed):
    case = W.decode_case(M, H=4096, seed=seed)
    say(f"router {case.name}")
    gi, gw, gl = run_fwd(case)
    rep = check_router(orc, case, gi, gw, gl)
    assert rep.max_weight_rel_err <= 1e-5


@pytest.mark.parametrize("seed", [0, 1])
def test_decode_metric_shape(orc, seed):
    case = W.metric_case(seed)
    say(f"router {case.name}")
    gi, gw, gl = run_fwd(case)
    check_router(orc, case, gi, gw, gl)


@pytest.mark.parametrize("M", [1, 2, 16, 64])
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_biased_router(orc, M, seed):
    case = W.biased_case(M, seed=seed)
    say(f"router {case.name}")
    gi, gw, gl = run_fwd(case)
    check_router(orc, case, gi, gw, gl)


@pytest.mark.parametrize("seed", list(range(10)))
def test_m2_table(orc, seed):
    case = W.biased_case(2, seed=seed)
    say(f"router m2 table {case.name}")
    res = R.router_fwd_m2_table(bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k,
                                case.scoring, case.renorm, return_logits=True)
    torch.cuda.synchronize()
    gi, gw, gl = host(res["inds"]), host(res["weights"]), host(res["logits"])
    check_router(orc, case, gi, gw, gl)
    check_table(orc, gi, {k: host(res[k]) for k in
                          ("unique_ids", "token_mask", "slot_to_unique", "unique_count")})
    # the table changes nothing else: same bytes as the table-free call
    pi, pw, _ = run_fwd(case)
    assert np.array_equal(pi, gi) and np.array_equal(pw.view(np.uint32), gw.view(np.uint32))
    if seed % 10 < 3:
        assert int(host(res["unique_count"])[0]) < 2 * case.k  # shared experts were forced


def test_m2_table_extremes(orc):
    """Identical tokens (k unique) and the softmax/no-bias variant."""
    case = W.decode_case(2, H=4096, seed=4)
    case.x[1] = case.x[0]
    res = R.router_fwd_m2_table(bf16_dev(case.x), bf16_dev(case.w), None, 8, W.SOFTMAX, True)
    torch.cuda.synchronize()
    gi = host(res["inds"])
    assert np.array_equal(gi[0], gi[1])
    assert int(host(res["unique_count"])[0]) == 8
    assert np.all(host(res["token_mask"])[:8] == 3) and np.all(host(res["unique_ids"])[8:] == -1)
    check_table(orc, gi, {k: host(res[k]) for k in
                          ("unique_ids", "token_mask", "slot_to_unique", "unique_count")})


TABLE_WIDTHS = [(1, 8, False), (3, 8, False), (4, 8, False), (8, 8, False), (16, 4, False),
                (3, 6, True), (8, 6, True), (10, 6, True)]


@pytest.mark.parametrize("M,k,biased", TABLE_WIDTHS, ids=lambda v: str(v))
@pytest.mark.parametrize("seed", [0, 1, 3, 5, 8])
def test_route_table_verify_widths(orc, M, k, biased, seed):
    """The table at every verify width (M*k <= 64 slots) is the oracle's table of the
    returned indices, and inds/weights are the bytes router_fwd gives."""
    case = W.verify_table_case(M, seed=seed, k=k, biased=biased)
    say(f"route table {case.name}")
    res = R.router_fwd_route_table(bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k,
                                   case.scoring, case.renorm, return_logits=True)
    torch.cuda.synchronize()
    gi, gw, gl = host(res["inds"]), host(res["weights"]), host(res["logits"])
    check_router(orc, case, gi, gw, gl)
    check_table(orc, gi, {k: host(res[k]) for k in
                          ("unique_ids", "token_mask", "slot_to_unique", "unique_count")})
    pi, pw, _ = run_fwd(case)
    assert np.array_equal(pi, gi) and np.array_equal(pw.view(np.uint32), gw.view(np.uint32))
    if seed % 10 < 5 and M > 1:
        assert int(host(res["unique_count"])[0]) < M * case.k  # shared experts were forced


def test_route_table_m2_matches_general(orc):
    case = W.biased_case(2, seed=2)
    args = (bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias), case.k, case.scoring, case.renorm)
    a, b = R.router_fwd_m2_table(*args), R.router_fwd_route_table(*args)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name].view(torch.int32), b[name].view(torch.int32)), name


@pytest.mark.parametrize("M", [257, 300, 333, 1000, 2100, 4000])
@pytest.mark.parametrize("scoring,with_bias", [(W.SOFTMAX, True), (W.SOFTMAX, False),
                                               (W.SQRT_SOFTPLUS, True)])
def test_prefill_ragged(orc, M, scoring, with_bias):
    """257-2048 tokens take 16 K splits per tile, up to 4096 eight, then four."""
    case = W.prefill_case(M=M, H=1024, seed=M)
    case.scoring = scoring
    if not with_bias:
        case.bias = None
    say(f"router prefill M={M} scoring={scoring} bias={with_bias}")
    gi, gw, gl = run_fwd(case)
    check_router(orc, case, gi, gw, gl)


@pytest.mark.parametrize("M", [65, 100, 128, 129, 200, 256])
@pytest.mark.parametrize("scoring,with_bias", [(W.SOFTMAX, True), (W.SQRT_SOFTPLUS, True),
                                               (W.SOFTMAX, False)])
def test_decode_many_row_blocks(orc, M, scoring, with_bias):
    """65..256 tokens take the split decode kernel with 5..16 row blocks (and
    one split per workgroup once the row blocks alone fill the CUs)."""
    case = W.prefill_case(M=M, H=1024, seed=500 + M)
    case.scoring = scoring
    if not with_bias:
        case.bias = None
    say(f"router decode M={M} scoring={scoring} bias={with_bias}")
    gi, gw, gl = run_fwd(case)
    check_router(orc, case, gi, gw, gl)


@pytest.mark.parametrize("scale", [4, 8])
def test_prefill_peaked_softmax_with_bias(orc, scale):
    # the prefill case's gate scaled by 4 or 8 (exact in bf16): logits of that
    # standard deviation, peaked softmax keys with the bias spreading the
    # tail, so the lockstep groups' threshold searches run past six tries
    base = W.prefill_case(M=1024, H=1024, seed=90 + scale)
    w = W.f32_to_bf16_bits(W.bf16_bits_to_f32(base.w) * np.float32(scale))
    case = W.RouterCase(base.x, w, base.bias, base.k, base.scoring, base.renorm,
                        name=f"prefill peaked x{scale}")
    say(f"router {case.name}")
    gi, gw, gl = run_fwd(case)
    check_router(orc, case, gi, gw, gl)


@pytest.mark.parametrize("M,H", [(10000, 256), (20000, 128)])
def test_prefill_two_and_one_splits(orc, M, H):
    """10000 rows = 79 tiles (two K splits); 20000 rows = 157 tiles (no split)."""
    case = W.prefill_case(M=M, H=H, seed=M)
    say(f"router prefill M={M} H={H}")
    gi, gw, gl = run_fwd(case)
    check_router(orc, case, gi, gw, gl)


@pytest.mark.parametrize("M", [520, 4000, 8192, 10000])
def test_prefill_handover_path_matches(orc, M):
    """Zero exchange wait: splits hand their rows over (16, 8, 4 and 2 K splits);
    results unchanged."""
    case = W.prefill_case(M=M, H={8192: 7168, 10000: 256}.get(M, 1024), seed=77)
    x, w, b = bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias)
    say(f"prefill hand-over M={M}")
    ref = R.router_fwd(x, w, b, case.k, case.scoring, case.renorm, return_logits=True)
    try:
        R.set_exchange_timeout_us(0)
        got = R.router_fwd(x, w, b, case.k, case.scoring, case.renorm, return_logits=True)
        torch.cuda.synchronize()
    finally:
        R.set_exchange_timeout_us(200)
    for a, g in zip(ref, got):
        assert torch.equal(a.view(torch.int32), g.view(torch.int32))
    if M != 8192:
        check_router(orc, case, host(got[0]), host(got[1]), host(got[2]))


@pytest.mark.slow
@pytest.mark.parametrize("H", [7168, 1024])
def test_prefill_full_size_every_row(orc, H):
    """M=8192 tokens, every row against the oracle (rows sharded over host threads).
    H=7168 is the prefill workload itself (112 k-steps over four K splits of the
    64 tiles); H=1024 puts the multi-stage LDS rings through a full-M launch with
    a different split length."""
    case = W.prefill_case(H=H)
    say(f"router {case.name} (every row)")
    gi, gw, gl = run_fwd(case)
    ref = oracle_par.router(orc, case.x, case.w, case.bias, case.k, case.scoring, case.renorm)
    rep = check_router(orc, case, gi, gw, gl, ref=ref)
    assert rep.rows == 8192
    assert rep.max_weight_rel_err <= 1e-5


def test_fused_equals_unfused(orc):
    """Gate G-A analogue: router_fwd == router_topk_from_logits(router_fwd's own logits)."""
    cases = [W.decode_case(8, seed=11), W.biased_case(64, seed=12), W.metric_case(3),
             W.prefill_case(M=520, H=512, seed=13), W.prefill_case(M=200, H=512, seed=14)]
    for case in cases:
        say(f"fused vs unfused {case.name}")
        gi, gw, gl = run_fwd(case)
        ui, uw = R.router_topk_from_logits(f32_dev(gl), f32_dev(case.bias), case.k, case.scoring,
                                           case.renorm)
        torch.cuda.synchronize()
        assert np.array_equal(host(ui), gi), case.name
        assert np.array_equal(host(uw).view(np.uint32), gw.view(np.uint32)), case.name


def test_logits_output_does_not_perturb():
    for case in (W.decode_case(2, seed=21), W.biased_case(16, seed=22), W.prefill_case(M=96, H=512),
                 W.prefill_case(M=384, H=512)):
        x, w, b = bf16_dev(case.x), bf16_dev(case.w), f32_dev(case.bias)
        say(f"logits on/off {case.name}")
        i1, w1 = R.router_fwd(x, w, b, case.k, case.scoring, case.renorm)
        i2, w2, _ = R.router_fwd(x, w, b, case.k, case.scoring, case.renorm, return_logits=True)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2) and torch.equal(w1.view(torch.int32), w2.view(torch.int32))


def test_repeat_calls_are_deterministic():
    case = W.decode_case(8, H=7168, seed=31)
    x, w = bf16_dev(case.x), bf16_dev(case.w)
    ref = R.router_fwd(x, w, None, 8, W.SOFTMAX, True, return_logits=True)
    for _ in range(20):
        got = R.router_fwd(x, w, None, 8, W.SOFTMAX, True, return_logits=True)
        for a, b in zip(ref, got):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_empty_batch():
    x = torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((256, 4096), dtype=torch.bfloat16, device="cuda:0")
    gi, gw = R.router_fwd(x, w, None, 8)
    assert gi.shape == (0, 8)
