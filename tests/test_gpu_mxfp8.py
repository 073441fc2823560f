"""router_fwd_mxfp8 (the fused router on a block-scaled FP8 gate) vs the oracle.

Parity rule (b) as for the bf16 gate: the oracle dequantises every MXFP8
weight exactly (E4M3 code times its block's E8M0 scale) and forms the fp64
dot product, the kernels convert the codes to bf16 on chip and accumulate in
fp32.  Workloads (seeded, synthetic): unit-RMS activations, W ~ N(0, 1/H)
quantised to MXFP8; decode widths M in {1, 2, 4, 8, 16, 64}; H = 4096, 7168
and ragged H (a last 128-block with one, two or three 32-blocks); E = 256,
100 and 16; every finite E4M3 code (subnormals, both zeros, +-448) at
ordinary and extreme scales; prefill sizes M in {257, 300, 333, 1000} (four
K splits), 10000 (two) and 20000 (one), and M = 8192, H = 7168 on every
row.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.compare import check_router
from gate_projection_top_amd import router as R
from gate_projection_top_amd import workloads as W
from gpu_util import bf16_dev, f32_dev, host, say
import oracle_par

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def run_mx(case):
    gi, gw, gl = R.router_fwd_mxfp8(bf16_dev(case.x), u8_dev(case.elems), u8_dev(case.scales),
                                    f32_dev(case.bias), case.k, case.scoring, case.renorm,
                                    return_logits=True)
    torch.cuda.synchronize()
    return host(gi), host(gw), host(gl)


def check_mx(orc, case):
    say(f"mxfp8 {case.name}")
    gi, gw, gl = run_mx(case)
    ref = orc.router_mxfp8(case.x, case.elems, case.scales, case.bias, case.k, case.scoring,
                           case.renorm)
    return check_router(orc, case, gi, gw, gl, ref=ref)


def every_code_case(M, H, seed, E=64, k=8, scale=None):
    """Rows whose codes run through all 254 finite E4M3 codes (shifted per row),
    scales from the ordinary quantiser or one fixed value."""
    case = W.mxfp8_case(M, H=H, seed=seed, E=E, k=k)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    el = np.empty((E, H), dtype=np.uint8)
    for e in range(E):
        el[e] = np.resize(np.roll(finite, 7 * e), H)
    case.elems = el
    if scale is not None:
        case.scales = np.full_like(case.scales, scale)
    return case


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 64])
@pytest.mark.parametrize("seed", [0, 1])
def test_decode_widths(orc, M, seed):
    rep = check_mx(orc, W.mxfp8_case(M, H=4096, seed=seed))
    assert rep.max_weight_rel_err <= 1e-5


@pytest.mark.parametrize("M", [1, 2, 16])
def test_single_token_shape(orc, M):
    check_mx(orc, W.mxfp8_case(M, H=7168, seed=3))


@pytest.mark.parametrize("H", [32, 96, 544, 576, 1120, 7136])
def test_ragged_hidden(orc, H):
    # H % 128 in {32, 64, 96}: a last 128-block holding one, two or three
    # 32-blocks; H = 32 is a single 32-block in all
    for M in (1, 5):
        check_mx(orc, W.mxfp8_case(M, H=H, seed=4))


@pytest.mark.parametrize("scoring,with_bias,renorm", [
    (W.SOFTMAX, False, True), (W.SOFTMAX, True, True), (W.SOFTMAX, False, False),
    (W.SQRT_SOFTPLUS, True, True), (W.SQRT_SOFTPLUS, False, False)])
@pytest.mark.parametrize("E,k", [(256, 8), (100, 6), (16, 16)])
def test_scoring_modes_and_experts(orc, scoring, with_bias, renorm, E, k):
    for M in (1, 24):
        check_mx(orc, W.mxfp8_case(M, H=2048, seed=5, E=E, k=k, scoring=scoring,
                                   with_bias=with_bias, renorm=renorm))


@pytest.mark.parametrize("M", [1, 3, 130, 390])
def test_every_code(orc, M):
    # all finite codes, subnormals and -0 included, at 2^-14: the largest (448)
    # becomes 0.027 and the smallest (2^-9) 2^-23, so the weights have about the
    # workload's N(0, 1/H) size and the logits its O(1) range (rule (b) fixes the
    # weights' 1e-5 bound for logits of that size)
    check_mx(orc, every_code_case(M, H=1024, seed=11, scale=113))


def test_scale_extremes(orc):
    # Blocks at the contract's smallest and largest useful scales next to
    # ordinary ones: rows at scale 10 (E4M3 subnormals at bf16's smallest
    # normal, 2^-126), single blocks pushed up by 2^40, and a row of every
    # code at scale 10.
    case = W.mxfp8_case(4, H=1024, seed=6, E=64, k=8)
    sc = case.scales.copy()
    sc[3, :] = 10
    sc[7, 5] = min(246, int(sc[7, 5]) + 40)
    sc[9, ::3] = 10
    case.scales = sc
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    case.elems = case.elems.copy()
    case.elems[11] = np.resize(finite, 1024)
    case.scales[11, :] = 10
    check_mx(orc, case)


@pytest.mark.parametrize("M", [257, 300, 333, 1000])
@pytest.mark.parametrize("scoring,with_bias", [(W.SOFTMAX, True), (W.SOFTMAX, False),
                                               (W.SQRT_SOFTPLUS, True)])
def test_prefill_ragged(orc, M, scoring, with_bias):
    check_mx(orc, W.mxfp8_case(M, H=1024, seed=M, scoring=scoring, with_bias=with_bias))


@pytest.mark.parametrize("M,H", [(10000, 256), (20000, 128)])
def test_prefill_two_and_one_splits(orc, M, H):
    """10000 rows = 79 tiles (two K splits); 20000 rows = 157 tiles (no split)."""
    check_mx(orc, W.mxfp8_case(M, H=H, seed=M, with_bias=True))


@pytest.mark.parametrize("M,H", [(300, 128), (1000, 128), (390, 256)])
def test_prefill_splits_without_stages(orc, M, H):
    """Four K splits over one or two 64-wide stages: some splits have no stage
    and contribute zero partials, but still take part in the exchange."""
    check_mx(orc, W.mxfp8_case(M, H=H, seed=M + H, with_bias=True))


@pytest.mark.parametrize("E,k,scoring", [(100, 6, W.SQRT_SOFTPLUS), (16, 16, W.SOFTMAX)])
def test_prefill_experts(orc, E, k, scoring):
    check_mx(orc, W.mxfp8_case(300, H=512, seed=E, E=E, k=k, scoring=scoring, with_bias=True))


def test_prefill_scale_extremes(orc):
    case = W.mxfp8_case(390, H=1024, seed=16, E=64, k=8)
    sc = case.scales.copy()
    sc[3, :] = 10
    sc[7, 5] = min(246, int(sc[7, 5]) + 40)
    sc[9, ::3] = 10
    case.scales = sc
    check_mx(orc, case)


def test_prefill_handover_path_matches(orc):
    """Zero exchange wait: every split but the last hands its rows over; results unchanged."""
    case = W.mxfp8_case(520, H=1024, seed=17, with_bias=True)
    args = (bf16_dev(case.x), u8_dev(case.elems), u8_dev(case.scales), f32_dev(case.bias), case.k,
            case.scoring, case.renorm)
    say("mxfp8 prefill hand-over M=520")
    ref = R.router_fwd_mxfp8(*args, return_logits=True)
    try:
        R.set_exchange_timeout_us(0)
        got = R.router_fwd_mxfp8(*args, return_logits=True)
        torch.cuda.synchronize()
    finally:
        R.set_exchange_timeout_us(200)
    for a, g in zip(ref, got):
        assert torch.equal(a.view(torch.int32), g.view(torch.int32))
    check_router(orc, case, host(got[0]), host(got[1]), host(got[2]),
                 ref=orc.router_mxfp8(case.x, case.elems, case.scales, case.bias, case.k,
                                      case.scoring, case.renorm))


@pytest.mark.slow
def test_prefill_full_size_every_row(orc):
    """M=8192, H=7168 with a selection bias: every row against the oracle (rows
    sharded over host threads)."""
    case = W.mxfp8_case(8192, H=7168, seed=18, with_bias=True)
    say(f"mxfp8 {case.name} (every row)")
    gi, gw, gl = run_mx(case)
    ref = oracle_par.router_mxfp8(orc, case.x, case.elems, case.scales, case.bias, case.k,
                                 case.scoring, case.renorm)
    rep = check_router(orc, case, gi, gw, gl, ref=ref)
    assert rep.rows == 8192


def test_fused_equals_unfused(orc):
    # The logits the MXFP8 call returns, routed by router_topk_from_logits,
    # give bit-identical indices and weights: the same device routine.
    for case in (W.mxfp8_case(2, H=4096, seed=7, with_bias=True, scoring=W.SQRT_SOFTPLUS, k=6),
                 W.mxfp8_case(16, H=4096, seed=8), W.mxfp8_case(200, H=512, seed=9, with_bias=True)):
        gi, gw, gl = run_mx(case)
        ti, tw = R.router_topk_from_logits(torch.from_numpy(gl).cuda(), f32_dev(case.bias), case.k,
                                           case.scoring, case.renorm)
        torch.cuda.synchronize()
        assert np.array_equal(host(ti), gi)
        assert np.array_equal(host(tw).view(np.uint32), gw.view(np.uint32))


def test_same_logits_as_mxfp4_on_fp4_representable_weights():
    # E2M1 values are E4M3 values: an MXFP4 gate re-encoded as MXFP8 with the
    # same scales gives the same bf16 weights, the same products in the same
    # MFMA order, hence bit-identical logits and routes on both paths.
    for M, H in ((4, 4096), (150, 1024)):
        c4 = W.mxfp4_case(M, H=H, seed=12, with_bias=True)
        e2m1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
        lo, hi = c4.elems & 0x0F, c4.elems >> 4
        nib = np.stack([lo, hi], axis=-1).reshape(c4.elems.shape[0], H)
        mag = e2m1[nib & 7]
        code8 = np.abs(mag[..., None] - W.E4M3_MAGNITUDES).argmin(axis=-1)
        assert np.array_equal(W.E4M3_MAGNITUDES[code8], mag)
        code8 = (code8 | np.where(nib & 8, 0x80, 0)).astype(np.uint8)
        say(f"mxfp8 vs mxfp4 M={M} H={H}")
        x, sc, b = bf16_dev(c4.x), u8_dev(c4.scales), f32_dev(c4.bias)
        r4 = R.router_fwd_mxfp4(x, u8_dev(c4.elems), sc, b, c4.k, c4.scoring, c4.renorm,
                                return_logits=True)
        r8 = R.router_fwd_mxfp8(x, u8_dev(code8), sc, b, c4.k, c4.scoring, c4.renorm,
                                return_logits=True)
        torch.cuda.synchronize()
        for a, g in zip(r4, r8):
            assert torch.equal(a.view(torch.int32), g.view(torch.int32))


def test_logits_output_does_not_perturb_and_repeats():
    case = W.mxfp8_case(8, H=7168, seed=9, with_bias=True)
    x, we, ws = bf16_dev(case.x), u8_dev(case.elems), u8_dev(case.scales)
    b = f32_dev(case.bias)
    i0, w0 = R.router_fwd_mxfp8(x, we, ws, b, case.k, case.scoring, case.renorm)
    i1, w1, _ = R.router_fwd_mxfp8(x, we, ws, b, case.k, case.scoring, case.renorm, return_logits=True)
    torch.cuda.synchronize()
    ref_i, ref_w = host(i0), host(w0)
    assert np.array_equal(host(i1), ref_i) and np.array_equal(host(w1), ref_w)
    for _ in range(20):
        i2, w2 = R.router_fwd_mxfp8(x, we, ws, b, case.k, case.scoring, case.renorm)
        torch.cuda.synchronize()
        assert np.array_equal(host(i2), ref_i) and np.array_equal(host(w2), ref_w)


def test_interleaved_with_other_formats(orc):
    # bf16, MXFP4 and MXFP8 calls share the decode and prefill workspaces: alternate them.
    for M in (4, 160):
        m8 = W.mxfp8_case(M, H=1024, seed=10)
        m4 = W.mxfp4_case(M, H=1024, seed=10)
        bf = W.decode_case(M, H=1024, seed=10) if M <= R.DECODE_MAX_M else None
        for _ in range(2):
            check_mx(orc, m8)
            gi, gw, gl = R.router_fwd_mxfp4(bf16_dev(m4.x), u8_dev(m4.elems), u8_dev(m4.scales),
                                            f32_dev(m4.bias), m4.k, m4.scoring, m4.renorm,
                                            return_logits=True)
            torch.cuda.synchronize()
            check_router(orc, m4, host(gi), host(gw), host(gl),
                         ref=orc.router_mxfp4(m4.x, m4.elems, m4.scales, m4.bias, m4.k, m4.scoring,
                                              m4.renorm))
            if bf is not None:
                gi, gw, gl = R.router_fwd(bf16_dev(bf.x), bf16_dev(bf.w), f32_dev(bf.bias), bf.k,
                                          bf.scoring, bf.renorm, return_logits=True)
                torch.cuda.synchronize()
                check_router(orc, bf, host(gi), host(gw), host(gl))


def test_empty_batch():
    case = W.mxfp8_case(1, H=256, seed=0)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    i, w = R.router_fwd_mxfp8(x, u8_dev(case.elems), u8_dev(case.scales), None, 8)
    assert i.shape == (0, 8) and w.shape == (0, 8)
