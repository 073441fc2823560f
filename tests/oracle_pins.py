"""Pins for the CPU oracle: checks against facts the mathematics fixes.

Each pin is a function of an oracle instance that raises AssertionError when
the oracle disagrees with a closed form, an exact computation, a brute-force
enumeration, an independent library routine or an invariant.  None of them
retypes the oracle's own code path:

  * logits: exact integer / rational dot products (Python ints, Fractions),
    one-hot gate rows, and numpy's BLAS float64 product;
  * scores: softplus(0) = ln 2, softplus(x) -> x, softplus(x) ~ e^x, numpy's
    logaddexp; softmax of equal logits is 1/E;
  * selection: brute force over every k-subset (E <= 16) against the
    contract "every selected expert precedes every unselected one", a stable
    descending sort, k=1 = first argmax, k=E = the whole order;
  * weights: renormalised weights sum to 1, equal winners get 1/k, softmax
    renormalisation equals a softmax over the winners alone, the bias moves
    the selection but never a weight;
  * table: encounter order equals dict.fromkeys, hand-worked identical and
    disjoint token pairs, structural invariants;
  * BF16 rounding: exact rational rounding to the nearest BF16 (ties to
    even) over random, tie and overflow-edge fp32 patterns;
  * gather + shared add: exact dyadic cases (every fp32 step exact, so only
    the two BF16 roundings act), hand-worked cases for the slot order, the
    separate multiply and add and the intermediate BF16 rounding, all-remote
    = shared, weight-1 single slot = the row, duplicated rows = summed
    weights; compact table rows by hand and by structural invariants.

tests/test_oracle_mutants.py plants plausible mistakes in copies of oracle.c
and requires every planted mistake to fail at least one pin.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np

from gate_projection_top_amd import workloads as W

SOFTMAX, SQRT_SOFTPLUS = 0, 1


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def fraction_to_f32(F: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even)."""
    c = np.float32(float(F))
    best, best_err = None, None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - F)
        if best is None or err < best_err or (
                err == best_err and (int(np.float32(cand).view(np.uint32)) & 1) == 0):
            best, best_err = cand, err
    return np.float32(best)


def bf16_fraction(bits: int) -> Fraction:
    return Fraction(float(W.bf16_bits_to_f32(np.array([bits], np.uint16))[0]))


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|bit-pattern distance| between same-sign fp32 arrays."""
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def precedence_matrix(keys: np.ndarray) -> np.ndarray:
    """P[e, f] = expert e comes before expert f (key larger, or equal and lower index)."""
    k = np.asarray(keys, np.float64)
    E = k.shape[0]
    idx = np.arange(E)
    greater = k[:, None] > k[None, :]
    equal = k[:, None] == k[None, :]
    return greater | (equal & (idx[:, None] < idx[None, :]))


def brute_force_topk(keys: np.ndarray, k: int) -> list:
    """The unique k-subset whose every member precedes every non-member, in order."""
    E = keys.shape[0]
    P = precedence_matrix(keys)
    found = []
    for S in itertools.combinations(range(E), k):
        inside = np.zeros(E, bool)
        inside[list(S)] = True
        if P[np.ix_(inside, ~inside)].all():
            found.append(S)
    assert len(found) == 1, f"contract admits {len(found)} subsets"
    S = list(found[0])
    # order inside the subset: e before f iff P[e, f]; count predecessors
    return sorted(S, key=lambda e: sum(P[f, e] for f in S))


def stable_desc_order(keys: np.ndarray) -> np.ndarray:
    k = np.asarray(keys, np.float64).copy()
    k[k == 0.0] = 0.0
    return np.argsort(-k, kind="stable")


# --------------------------------------------------------------------------
# logits
# --------------------------------------------------------------------------
def pin_logits_small_integers(o):
    """Small integers are exact in bf16; their dot product is an exact integer."""
    rng = np.random.default_rng(11)
    M, H, E = 3, 64, 5
    xi = rng.integers(-8, 9, size=(M, H))
    wi = rng.integers(-8, 9, size=(E, H))
    x = W.f32_to_bf16_bits(xi.astype(np.float32))
    w = W.f32_to_bf16_bits(wi.astype(np.float32))
    lg, ad = o.logits(x, w)
    for t in range(M):
        for e in range(E):
            exact = sum(int(a) * int(b) for a, b in zip(xi[t], wi[e]))
            mag = sum(abs(int(a) * int(b)) for a, b in zip(xi[t], wi[e]))
            assert lg[t, e] == np.float32(exact), (t, e, lg[t, e], exact)
            assert ad[t, e] == float(mag), (t, e, ad[t, e], mag)


def pin_logits_rational(o):
    """Random bf16 operands: the logit is the exact rational dot rounded once to fp32."""
    rng = np.random.default_rng(12)
    M, H, E = 2, 32, 3
    x = W.gaussian_bf16(rng, (M, H), 1.0)
    w = W.gaussian_bf16(rng, (E, H), 0.3)
    lg, ad = o.logits(x, w)
    for t in range(M):
        for e in range(E):
            prods = [bf16_fraction(int(x[t, i])) * bf16_fraction(int(w[e, i])) for i in range(H)]
            exact = sum(prods, Fraction(0))
            assert lg[t, e] == fraction_to_f32(exact), (t, e)
            assert Fraction(ad[t, e]) == sum((abs(p) for p in prods), Fraction(0)), (t, e)


def pin_logits_one_hot(o):
    """A one-hot gate row picks one activation: logit[t,e] = x[t, pos(e)]."""
    rng = np.random.default_rng(13)
    M, H, E = 3, 24, 7
    x = W.gaussian_bf16(rng, (M, H), 1.0)
    pos = rng.choice(H, size=E, replace=False)
    wf = np.zeros((E, H), np.float32)
    wf[np.arange(E), pos] = 1.0
    lg, _ = o.logits(x, W.f32_to_bf16_bits(wf))
    xf = W.bf16_bits_to_f32(x)
    assert np.array_equal(lg, xf[:, pos]), (lg, xf[:, pos])


def pin_logits_blas(o):
    """numpy's float64 matmul (its own BLAS) agrees to rounding on unit-scale data."""
    rng = np.random.default_rng(14)
    M, H, E = 4, 512, 32
    x = W.gaussian_bf16(rng, (M, H), 1.0)
    w = W.gaussian_bf16(rng, (E, H), 1.0 / math.sqrt(H))
    lg, _ = o.logits(x, w)
    ref = W.bf16_bits_to_f32(x).astype(np.float64) @ W.bf16_bits_to_f32(w).astype(np.float64).T
    assert np.all(np.abs(lg - ref) <= 1e-6 * np.maximum(1.0, np.abs(ref))), np.abs(lg - ref).max()


# --------------------------------------------------------------------------
# scores
# --------------------------------------------------------------------------
def pin_softplus_closed_forms(o):
    """softplus(0)=ln2; softplus(40)=40 to double precision; softplus(-30)~e^-30."""
    row = np.array([0.0, 40.0, -30.0, 1.0], np.float32)
    s, u = o.row_scores(row, SQRT_SOFTPLUS)
    assert abs(s[0] - math.sqrt(math.log(2.0))) <= 2e-16, s[0]
    assert abs(s[1] - math.sqrt(40.0)) <= 2e-15, s[1]
    assert abs(s[2] / math.exp(-15.0) - 1.0) <= 1e-12, s[2]
    assert np.array_equal(s, u)
    # softplus(1) = ln(1+e)
    assert abs(s[3] - math.sqrt(math.log(1.0 + math.e))) <= 4e-16, s[3]


def pin_softplus_logaddexp(o):
    """sqrt(logaddexp(0, x)) (numpy's own routine) agrees to double rounding."""
    rng = np.random.default_rng(15)
    row = (rng.standard_normal(256) * 6.0).astype(np.float32)
    s, _ = o.row_scores(row, SQRT_SOFTPLUS)
    ref = np.sqrt(np.logaddexp(0.0, row.astype(np.float64)))
    assert np.all(np.abs(s - ref) <= 8e-16 * ref), np.abs(s / ref - 1).max()


def pin_softmax_closed_forms(o):
    """Equal logits give 1/E; [0, c] gives 1/(1+e^-c); probabilities sum to 1."""
    s, u = o.row_scores(np.full(8, 0.37, np.float32), SOFTMAX)
    assert np.all(s == 0.125) and np.all(u == 1.0)
    c = np.float32(math.log(3.0))
    s, u = o.row_scores(np.array([0.0, c], np.float32), SOFTMAX)
    assert abs(s[1] - 1.0 / (1.0 + math.exp(-float(c)))) <= 2e-16
    assert abs(s[0] - math.exp(-float(c)) / (1.0 + math.exp(-float(c)))) <= 2e-16
    rng = np.random.default_rng(16)
    row = (rng.standard_normal(256) * 3).astype(np.float32)
    s, u = o.row_scores(row, SOFTMAX)
    assert abs(math.fsum(s) - 1.0) < 1e-14
    assert u.max() == 1.0


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------
def _tie_rows(rng, E, n):
    """Rows drawn from a handful of values (so ties are everywhere), with +-0."""
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 2.0, 3.5], np.float32)
    rows = [rng.choice(vals, size=E) for _ in range(n)]
    rows.append(np.full(E, 0.5, np.float32))
    rows.append(np.where(np.arange(E) % 2 == 0, np.float32(-0.0), np.float32(0.0)))
    rows.append((rng.standard_normal(E)).astype(np.float32))
    return np.stack(rows).astype(np.float32)


def pin_topk_brute_force(o):
    """E<=16: the oracle's set is the unique k-subset the contract admits, in order."""
    rng = np.random.default_rng(17)
    for E, ks in ((16, (1, 2, 3, 8, 15, 16)), (6, range(1, 7))):
        rows = _tie_rows(rng, E, 6)
        for k in ks:
            inds, _ = o.topk_from_logits(rows, None, k, SOFTMAX, True)
            for r in range(rows.shape[0]):
                want = brute_force_topk(rows[r], k)
                assert list(inds[r]) == want, (E, k, r, rows[r], inds[r], want)


def pin_topk_stable_sort(o):
    """First k of a stable descending sort (lower index first among equals)."""
    rng = np.random.default_rng(18)
    case = W.adversarial_logits(64, seed=3)
    rows = np.concatenate([case.logits, _tie_rows(rng, 256, 4)])
    for k in (1, 8, 13):
        inds, _ = o.topk_from_logits(rows, None, k, SOFTMAX, True)
        for r in range(rows.shape[0]):
            assert np.array_equal(inds[r], stable_desc_order(rows[r])[:k]), (k, r)


def pin_topk_extremes(o):
    """k=1 is the first argmax; k=E lists every expert in contract order."""
    rng = np.random.default_rng(19)
    rows = _tie_rows(rng, 12, 5)
    i1, _ = o.topk_from_logits(rows, None, 1, SOFTMAX, True)
    assert np.array_equal(i1[:, 0], np.argmax(rows, axis=1))
    iE, _ = o.topk_from_logits(rows, None, 12, SOFTMAX, True)
    for r in range(rows.shape[0]):
        assert sorted(iE[r]) == list(range(12))
        assert list(iE[r]) == brute_force_topk(rows[r], 12)


def pin_unbiased_key_is_exact_score_order(o):
    """No bias: the order is that of the exact scores, i.e. of the logits.

    Softmax and sqrt-softplus are strictly increasing, so a logit one ulp
    above another has the larger exact score, even where both scores round to
    the same fp32 value (which happens near zero, where a logit ulp is far
    below a probability ulp).  The larger logit must win although it sits on
    the higher index.
    """
    lo = np.float32(0.01)
    hi = np.nextafter(lo, np.float32(np.inf))
    row = np.full((1, 16), -5.0, np.float32)
    row[0, 3], row[0, 9] = lo, hi
    s, _ = o.row_scores(row[0], SOFTMAX)
    assert np.float32(s[3]) == np.float32(s[9])  # the fp32 scores do collide
    for scoring in (SOFTMAX, SQRT_SOFTPLUS):
        inds, _ = o.topk_from_logits(row, None, 1, scoring, True)
        assert inds[0, 0] == 9, (scoring, inds)
        inds, _ = o.topk_from_logits(row, None, 2, scoring, True)
        assert list(inds[0]) == [9, 3], (scoring, inds)


def pin_all_equal_rows(o):
    """All-equal logits: experts 0..k-1, weights 1/k (renorm) or 1/E (softmax, no renorm)."""
    row = np.full((1, 256), -0.75, np.float32)
    for scoring in (SOFTMAX, SQRT_SOFTPLUS):
        inds, w = o.topk_from_logits(row, None, 8, scoring, True)
        assert list(inds[0]) == list(range(8)) and np.all(w == np.float32(0.125))
    inds, w = o.topk_from_logits(row, None, 8, SOFTMAX, False)
    assert np.all(w == np.float32(1.0 / 256))


def pin_bias_orders_equal_scores(o):
    """Equal logits + distinct biases: selection follows the bias, weights stay equal."""
    E, k = 32, 6
    bias = (np.arange(E, dtype=np.float32) % 7) * np.float32(0.01) - np.float32(0.03)
    row = np.full((1, E), 0.2, np.float32)
    for scoring in (SOFTMAX, SQRT_SOFTPLUS):
        inds, w = o.topk_from_logits(row, bias, k, scoring, True)
        want = stable_desc_order(bias)[:k]
        assert np.array_equal(inds[0], want), (scoring, inds[0], want)
        assert np.all(w == np.float32(1.0 / k))


def pin_bias_flips_but_weights_unbiased(o):
    """Bias can put a lower-scored expert first; its weight stays the unbiased one."""
    E = 8
    row = np.array([[2.0, 1.0, -3, -3, -3, -3, -3, -3]], np.float32)
    bias = np.zeros(E, np.float32)
    bias[1] = 0.5  # more than the score gap between experts 0 and 1
    for scoring in (SOFTMAX, SQRT_SOFTPLUS):
        inds, w = o.topk_from_logits(row, bias, 2, scoring, True)
        assert list(inds[0]) == [1, 0], (scoring, inds)
        if scoring == SOFTMAX:
            e1 = math.exp(1.0 - 2.0)
            want = [e1 / (e1 + 1.0), 1.0 / (e1 + 1.0)]
        else:
            s0 = math.sqrt(math.log1p(math.exp(2.0)))
            s1 = math.sqrt(math.log1p(math.exp(1.0)))
            want = [s1 / (s0 + s1), s0 / (s0 + s1)]
        assert np.all(ulp_distance(w[0], np.array(want, np.float32)) <= 1), (w, want)


def pin_bias_invariance(o):
    """Two biases that pick the same ordered set give byte-identical weights."""
    case = W.biased_case(4, seed=5, H=256)
    lg, _ = o.logits(case.x, case.w)
    for scoring in (SOFTMAX, SQRT_SOFTPLUS):
        inds, w = o.topk_from_logits(lg, case.bias, case.k, scoring, True)
        for r in range(lg.shape[0]):
            b2 = case.bias.copy()
            losers = np.setdiff1d(np.arange(case.E), inds[r])
            b2[losers] -= np.float32(1.0)     # losers stay losers
            i2, w2 = o.topk_from_logits(lg[r:r + 1], b2, case.k, scoring, True)
            assert np.array_equal(i2[0], inds[r])
            assert np.array_equal(w2[0].view(np.uint32), w[r].view(np.uint32))
        # and bias-free selection of the same row gives the same weight for a shared winner set
        i0, w0 = o.topk_from_logits(lg, None, case.k, scoring, True)
        for r in range(lg.shape[0]):
            if np.array_equal(i0[r], inds[r]):
                assert np.array_equal(w0[r].view(np.uint32), w[r].view(np.uint32))


def pin_renorm_sums_and_softmax_identity(o):
    """Renormalised weights sum to 1; softmax renorm = softmax over the winners alone."""
    case = W.adversarial_logits(32, seed=9)
    for scoring in (SOFTMAX, SQRT_SOFTPLUS):
        inds, w = o.topk_from_logits(case.logits, None, 8, scoring, True)
        assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 1e-6)
    inds, w = o.topk_from_logits(case.logits, None, 8, SOFTMAX, True)
    for r in range(case.logits.shape[0]):
        sel = [float(case.logits[r, e]) for e in inds[r]]
        ex = [math.exp(v) for v in sel]
        tot = math.fsum(ex)
        want = np.array([v / tot for v in ex], np.float32)
        assert np.all(ulp_distance(w[r], want) <= 1), (r, w[r], want)


def pin_softmax_no_renorm_is_probability(o):
    """Without renormalisation a softmax weight is the full-row probability."""
    rng = np.random.default_rng(20)
    rows = (rng.standard_normal((8, 64)) * 2).astype(np.float32)
    inds, w = o.topk_from_logits(rows, None, 4, SOFTMAX, False)
    for r in range(rows.shape[0]):
        ex = [math.exp(float(v)) for v in rows[r]]
        tot = math.fsum(ex)
        want = np.array([ex[e] / tot for e in inds[r]], np.float32)
        assert np.all(ulp_distance(w[r], want) <= 1), (r, w[r], want)
    inds, w = o.topk_from_logits(rows, None, 4, SQRT_SOFTPLUS, False)
    for r in range(rows.shape[0]):
        want = np.array([math.sqrt(math.log1p(math.exp(float(rows[r, e])))) for e in inds[r]],
                        np.float32)
        assert np.all(ulp_distance(w[r], want) <= 1), (r, w[r], want)


# --------------------------------------------------------------------------
# the M=2 unique-route table
# --------------------------------------------------------------------------
def pin_table_hand_cases(o):
    """Identical tokens: k unique, masks 0b11; disjoint tokens: 2k unique, masks 1 then 2."""
    k = 6
    t0 = [7, 3, 200, 41, 0, 99]
    same = np.array([t0, [3, 41, 7, 0, 99, 200]], np.int32)
    ids, mask, s2u, cnt = o.route_table_m2(same)
    assert cnt == k and list(ids[:k]) == t0 and list(ids[k:]) == [-1] * k
    assert list(mask) == [3] * k + [0] * k
    assert list(s2u[:k]) == list(range(k))
    assert list(s2u[k:]) == [t0.index(e) for e in same[1]]
    disjoint = np.array([t0, [1, 2, 4, 5, 6, 8]], np.int32)
    ids, mask, s2u, cnt = o.route_table_m2(disjoint)
    assert cnt == 2 * k and list(ids) == t0 + [1, 2, 4, 5, 6, 8]
    assert list(mask) == [1] * k + [2] * k and list(s2u) == list(range(2 * k))
    partial = np.array([[5, 9], [9, 4]], np.int32)
    ids, mask, s2u, cnt = o.route_table_m2(partial)
    assert cnt == 3 and list(ids) == [5, 9, 4, -1] and list(mask) == [1, 3, 2, 0]
    assert list(s2u) == [0, 1, 1, 2]


def pin_table_invariants(o):
    """Random pairs: dict.fromkeys order, ids[s2u[s]] == slot id, mask bits = token membership."""
    rng = np.random.default_rng(21)
    for _ in range(200):
        k = int(rng.integers(1, 9))
        pool = rng.choice(256, size=int(rng.integers(k, 2 * k + 1)), replace=False)
        inds = np.stack([rng.choice(pool, size=k, replace=False),
                         rng.choice(pool, size=k, replace=False)]).astype(np.int32)
        ids, mask, s2u, cnt = o.route_table_m2(inds)
        slots = list(inds.reshape(-1))
        uniq = list(dict.fromkeys(slots))
        assert cnt == len(uniq) and list(ids[:cnt]) == uniq
        assert np.all(ids[cnt:] == -1) and np.all(mask[cnt:] == 0)
        for s, e in enumerate(slots):
            assert ids[s2u[s]] == e
        for q in range(cnt):
            want = (1 if ids[q] in inds[0] else 0) | (2 if ids[q] in inds[1] else 0)
            assert mask[q] == want
        assert k <= cnt <= 2 * k
        assert sum(bin(int(m)).count("1") for m in mask) == 2 * k


def pin_table_verify_widths(o):
    """Any M: identical tokens share every expert (mask of M ones); disjoint tokens each
    get k entries with mask 1 << t; hand-worked M=3 overlap; the M=2 entry point agrees."""
    k = 4
    base = [17, 3, 250, 64]
    for M in (1, 3, 8, 16):
        same = np.array([np.roll(base, t) for t in range(M)], np.int32)
        ids, mask, s2u, cnt = o.route_table(same)
        assert cnt == k and list(ids[:k]) == base and np.all(ids[k:] == -1)
        assert list(mask[:k]) == [(1 << M) - 1] * k and np.all(mask[k:] == 0)
        assert [base[v] for v in s2u] == list(same.reshape(-1))
        disjoint = np.array([[t * k + j for j in range(k)] for t in range(M)], np.int32)
        ids, mask, s2u, cnt = o.route_table(disjoint)
        assert cnt == M * k and list(ids) == list(range(M * k))
        assert list(mask) == [1 << (s // k) for s in range(M * k)]
        assert list(s2u) == list(range(M * k))
    # token 0 {5, 9}, token 1 {9, 4}, token 2 {4, 5}
    ids, mask, s2u, cnt = o.route_table(np.array([[5, 9], [9, 4], [4, 5]], np.int32))
    assert cnt == 3 and list(ids) == [5, 9, 4, -1, -1, -1]
    assert list(mask) == [0b101, 0b011, 0b110, 0, 0, 0] and list(s2u) == [0, 1, 1, 2, 2, 0]
    rng = np.random.default_rng(5)
    for _ in range(20):
        pair = np.stack([rng.choice(256, 6, replace=False) for _ in range(2)]).astype(np.int32)
        a, b = o.route_table(pair), o.route_table_m2(pair)
        assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3])) and a[3] == b[3]


def pin_table_invariants_any_m(o):
    """Random M in 1..16 with M*k <= 64: dict.fromkeys order, membership masks, slot map,
    M*k mask bits in total."""
    rng = np.random.default_rng(22)
    for _ in range(300):
        M = int(rng.integers(1, 17))
        k = int(rng.integers(1, 64 // M + 1))
        pool = rng.choice(256, size=int(rng.integers(k, min(256, M * k) + 1)), replace=False)
        inds = np.stack([rng.choice(pool, size=k, replace=False) for _ in range(M)]).astype(np.int32)
        ids, mask, s2u, cnt = o.route_table(inds)
        slots = list(inds.reshape(-1))
        uniq = list(dict.fromkeys(slots))
        assert cnt == len(uniq) and list(ids[:cnt]) == uniq
        assert np.all(ids[cnt:] == -1) and np.all(mask[cnt:] == 0)
        for s, e in enumerate(slots):
            assert ids[s2u[s]] == e
        for q in range(cnt):
            want = sum(1 << t for t in range(M) if ids[q] in inds[t])
            assert mask[q] == want
        assert k <= cnt <= M * k
        assert sum(bin(int(m)).count("1") for m in mask) == M * k


# --------------------------------------------------------------------------
# MXFP4 gate weights
# --------------------------------------------------------------------------
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the FP4 E2M1 value table of the MX format


def pin_e2m1_table(o):
    """The 16 E2M1 codes: the format's magnitudes for codes 0..7, sign in bit 3 (code 8 is -0)."""
    for c in range(16):
        v = o.e2m1_value(c)
        sign = -1.0 if c & 8 else 1.0
        assert v == sign * OCP_E2M1[c & 7] and math.copysign(1.0, v) == sign, (c, v)


def _dequant_numpy(elems, scales):
    """Independent dequantisation: nibbles unpacked low-first, table lookup, ldexp per block."""
    E, H = elems.shape[0], elems.shape[1] * 2
    codes = np.empty((E, H), np.int64)
    codes[:, 0::2] = elems & 15
    codes[:, 1::2] = elems >> 4
    mag = np.array(OCP_E2M1)[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    return np.ldexp(mag, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))


def pin_mx_dequant(o):
    """Dequantised weight = table value x 2^(scale-127), element 2j in the low nibble of byte
    j, one scale per 32 elements; scales outside [2, 252] and H % 32 != 0 are refused."""
    rng = np.random.default_rng(31)
    E, H = 5, 96
    elems = rng.integers(0, 256, (E, H // 2)).astype(np.uint8)
    scales = rng.integers(100, 150, (E, H // 32)).astype(np.uint8)
    w = o.dequant_mxfp4(elems, scales)
    assert np.array_equal(w, _dequant_numpy(elems, scales))
    assert w[0, 0] == OCP_E2M1[elems[0, 0] & 7] * (-1 if elems[0, 0] & 8 else 1) * 2.0 ** (int(scales[0, 0]) - 127)
    for bad in (0, 1, 253, 255):
        s2 = scales.copy()
        s2[2, 1] = bad
        try:
            o.dequant_mxfp4(elems, s2)
        except ValueError:
            continue
        raise AssertionError(f"scale {bad} accepted")
    try:
        o.dequant_mxfp4(elems[:, :20], scales[:, :1])  # H = 40
    except ValueError:
        pass
    else:
        raise AssertionError("H % 32 != 0 accepted")


def pin_mx_router_is_bf16_router_on_dequantised(o):
    """The MXFP4 router equals the bf16 router (pinned above) on the dequantised weights,
    which are exact bf16 values: same logits, indices and weight bits, every scoring mode."""
    from gate_projection_top_amd import workloads as W
    modes = [(W.SOFTMAX, False, True), (W.SOFTMAX, True, True), (W.SQRT_SOFTPLUS, True, True),
             (W.SOFTMAX, False, False)]
    for seed, (scoring, with_bias, renorm) in enumerate(modes):
        c = W.mxfp4_case(3, H=256, seed=seed, E=64, k=6, scoring=scoring, with_bias=with_bias,
                         renorm=renorm)
        wd = _dequant_numpy(c.elems, c.scales).astype(np.float32)
        wbits = (wd.view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal((wbits.astype(np.uint32) << 16).view(np.float32), wd)  # exact in bf16
        i1, w1, l1, _ = o.router_mxfp4(c.x, c.elems, c.scales, c.bias, c.k, c.scoring, c.renorm)
        i2, w2, l2, _ = o.router(c.x, wbits, c.bias, c.k, c.scoring, c.renorm)
        assert np.array_equal(i1, i2) and np.array_equal(w1.view(np.uint32), w2.view(np.uint32))
        assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


# --------------------------------------------------------------------------
# routed gather + shared-expert add, and the table's compact rows
# --------------------------------------------------------------------------
def bf16_rne_fraction(f: float) -> int:
    """BF16 bits of a finite fp32 value, by exact rational rounding to the
    nearest multiple of the BF16 spacing at its binade (ties to even)."""
    f = float(np.float32(f))
    sign = 0x8000 if math.copysign(1.0, f) < 0 else 0
    if f == 0.0:
        return sign
    A = abs(Fraction(f))
    _, ex = math.frexp(abs(f))           # |f| = m * 2^ex, m in [0.5, 1)
    e = max(ex - 1, -126)                # binade exponent; subnormal spacing below 2^-126
    spacing = Fraction(2) ** (e - 7)     # 7 fraction bits
    n = round(A / spacing)               # Python rounds a Fraction half to even
    value = n * spacing
    if value >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = int(np.array([float(value)], np.float32).view(np.uint32)[0]) >> 16
    assert bf16_fraction(bits) == value
    return sign | bits


def bf16_bits(v: float) -> int:
    """Bits of a value that BF16 represents exactly."""
    b = int(np.array([v], np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0, v
    return b >> 16


def pin_bf16_round(o):
    rng = np.random.default_rng(40)
    pats = rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, 500, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    near_max = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x00008000, 0x00018000,
                         0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001], np.uint32)
    for u in np.concatenate([pats, ties, near_max, near_max | 0x80000000]):
        f = float(np.array([u], np.uint32).view(np.float32)[0])
        if not math.isfinite(f):
            continue
        got = o.bf16_round(f)
        assert got == bf16_rne_fraction(f), (hex(int(u)), hex(got), hex(bf16_rne_fraction(f)))
    assert o.bf16_round(float("inf")) == 0x7F80 and o.bf16_round(float("-inf")) == 0xFF80
    nan = o.bf16_round(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def _gather(o, y_vals, rows, w, shared_vals):
    y = np.array([[bf16_bits(v) for v in r] for r in y_vals], np.uint16)
    sh = np.array([[bf16_bits(v) for v in r] for r in shared_vals], np.uint16)
    return o.gather_shared_add(y, np.array(rows, np.int32), np.array(w, np.float32), sh)


def pin_gather_exact_dyadic(o):
    """Small dyadic values: every fp32 product and partial sum is exact, so the
    output is the exact routed sum rounded to BF16, plus the shared value,
    rounded to BF16 (both roundings from exact rationals)."""
    rng = np.random.default_rng(41)
    R, D, M, k = 5, 48, 3, 6
    yv = rng.integers(-8, 9, (R, D)).astype(np.float64)
    wchoices = np.array([0.25, 0.5, 0.75, 1.0, 1.5, 2.0, -0.25, -0.5, -0.75, -1.0, -1.5, -2.0])
    for trial in range(6):
        rows = rng.integers(-1, R, (M, k))
        if trial == 0:
            rows[:] = -1                      # all remote
        if trial == 1:
            rows[0, :] = 2                    # one row in every slot of token 0
        w = rng.choice(wchoices, (M, k))
        sv = rng.integers(-16, 17, (M, D)) * 0.5
        out = _gather(o, yv, rows, w, sv)
        for t in range(M):
            for d in range(D):
                S = sum(Fraction(float(w[t, j])) * Fraction(float(yv[rows[t, j], d]))
                        for j in range(k) if rows[t, j] >= 0)
                routed = bf16_fraction(bf16_rne_fraction(float(S)))
                want = bf16_rne_fraction(float(routed + Fraction(float(sv[t, d]))))
                assert int(out[t, d]) == want, (trial, t, d, hex(int(out[t, d])), hex(want))


def pin_gather_hand_cases(o):
    """Worked cases whose expected bits follow from the rounding chain by hand."""
    # fp32 accumulation in slot order: 2^24 + 1 rounds back to 2^24, then -2^24
    # leaves 0 (the exact sum, or the reverse order, gives 1)
    out = _gather(o, [[2.0 ** 12], [1.0], [-(2.0 ** 12)]], [[0, 1, 2]], [[2.0 ** 12, 1.0, 2.0 ** 12]],
                  [[0.0]])
    assert int(out[0, 0]) == 0x0000, hex(int(out[0, 0]))
    # separate multiply and add: fl32((1 + 2^-23)(1 + 2^-7)) drops 2^-30, so the
    # sum is 2^-23 exactly (a fused multiply-add keeps 2^-23 + 2^-30 = 0x3401)
    out = _gather(o, [[1.0 + 2.0 ** -7]], [[0, 0]], [[-1.0, 1.0 + 2.0 ** -23]], [[0.0]])
    assert int(out[0, 0]) == 0x3400, hex(int(out[0, 0]))
    # the routed sum 1 + 2^-8 + 2^-9 first rounds to BF16 1 + 2^-7; adding the
    # shared 2^-8 gives a tie, 1 + 1.5 * 2^-7, which goes to the even 1 + 2^-6
    # (without the intermediate rounding: 1 + 1.25 * 2^-7 -> 1 + 2^-7 = 0x3F81)
    out = _gather(o, [[1.0], [1.0]], [[0, 1]], [[1.0, 2.0 ** -8 + 2.0 ** -9]], [[2.0 ** -8]])
    assert int(out[0, 0]) == 0x3F82, hex(int(out[0, 0]))
    # a remote slot (row -1) adds nothing, wherever it sits
    a = _gather(o, [[3.0], [5.0]], [[0, -1, 1]], [[0.5, 4.0, 0.25]], [[1.0]])
    b = _gather(o, [[3.0], [5.0]], [[0, 1, -1]], [[0.5, 0.25, 9.0]], [[1.0]])
    assert int(a[0, 0]) == int(b[0, 0]) == bf16_bits(3.75), (hex(int(a[0, 0])), hex(int(b[0, 0])))


def pin_gather_invariants(o):
    rng = np.random.default_rng(42)
    R, D, M, k = 4, 40, 2, 6
    y = W.gaussian_bf16(rng, (R, D), 1.0)
    shared = W.gaussian_bf16(rng, (M, D), 1.0)
    w = rng.uniform(0.05, 0.3, (M, k)).astype(np.float32)
    # every slot remote: the output is the shared expert's output
    out = o.gather_shared_add(y, np.full((M, k), -1, np.int32), w, shared)
    sh = W.bf16_bits_to_f32(shared)
    assert np.array_equal(out[sh != 0], shared[sh != 0])
    # one slot with weight 1, shared 0: the output is that expert row (BF16 is exact through the chain)
    zero = np.zeros((1, D), np.uint16)
    out = o.gather_shared_add(y, np.array([[3]], np.int32), np.ones((1, 1), np.float32), zero)
    yr = W.bf16_bits_to_f32(y[3:4])
    assert np.array_equal(out[yr != 0], y[3:4][yr != 0])
    # a duplicated row with weights a and b equals one slot of weight a + b
    # when every product and sum is exact (dyadic weights, small integer rows)
    yi = np.array([[bf16_bits(float(v)) for v in rng.integers(-8, 9, D)]], np.uint16)
    dup = o.gather_shared_add(yi, np.array([[0, 0, -1]], np.int32),
                              np.array([[0.75, 0.5, 3.0]], np.float32), zero)
    one = o.gather_shared_add(yi, np.array([[0, -1, -1]], np.int32),
                              np.array([[1.25, 0.0, 0.0]], np.float32), zero)
    assert np.array_equal(dup, one)
    # a row outside [-1, R) is refused
    for bad in (R, -2):
        try:
            o.gather_shared_add(y, np.array([[bad]], np.int32), np.ones((1, 1), np.float32), zero)
        except ValueError:
            continue
        raise AssertionError(f"row {bad} accepted")


def pin_table_rows_hand_cases(o):
    # token 0 picks 5, 7, 9 and token 1 picks 7, 9, 2: blocks [5: t0] [7: t0 t1] [9: t0 t1] [2: t1]
    ids, mask, s2u, cnt = o.route_table(np.array([[5, 7, 9], [7, 9, 2]]))
    rows = o.table_rows(mask, s2u, cnt, 2, 3)
    assert rows.tolist() == [[0, 1, 3], [2, 4, 5]], rows.tolist()
    # identical tokens: each expert's block holds both tokens
    ids, mask, s2u, cnt = o.route_table(np.array([[3, 4], [3, 4]]))
    assert o.table_rows(mask, s2u, cnt, 2, 2).tolist() == [[0, 2], [1, 3]]
    # disjoint tokens: one row per slot, in slot order
    ids, mask, s2u, cnt = o.route_table(np.array([[1, 2], [3, 4]]))
    assert o.table_rows(mask, s2u, cnt, 2, 2).tolist() == [[0, 1], [2, 3]]
    # a table whose slot names an expert the token did not pick is refused
    try:
        o.table_rows(np.array([1, 1], np.int32), np.array([0, 1, 0, 1], np.int32), 2, 2, 2)
    except ValueError:
        pass
    else:
        raise AssertionError("inconsistent table accepted")


def pin_table_rows_invariants(o):
    rng = np.random.default_rng(43)
    for M in (1, 2, 3, 5, 8, 16):
        for _ in range(6):
            k = int(rng.integers(1, 5))
            E = int(rng.integers(k, 3 * k + 2))
            inds = np.stack([rng.choice(E, k, replace=False) for _ in range(M)]).astype(np.int32)
            ids, mask, s2u, cnt = o.route_table(inds)
            rows = o.table_rows(mask, s2u, cnt, M, k)
            pairs = {}
            for t in range(M):
                for j in range(k):
                    pairs[(int(s2u[t * k + j]), t)] = int(rows[t, j])
            # one row per distinct (expert, token), covering 0..n-1 in (table order, token) order
            assert sorted(pairs.values()) == list(range(len(pairs)))
            assert [pairs[key] for key in sorted(pairs)] == list(range(len(pairs)))
            assert len(pairs) == M * k  # top-k experts are distinct within a token


def _small_int_bf16(rng, shape, lo=-6, hi=7):
    v = rng.integers(lo, hi, shape)
    return v, W.f32_to_bf16_bits(v.astype(np.float32))


def pin_gemm1_hand_table(o):
    """Token 0 picks experts 5, 7, 9 and token 1 picks 7, 9, 2: the compact rows are
    (5,t0) (7,t0) (7,t1) (9,t0) (9,t1) (2,t1); small integers make every product exact."""
    rng = np.random.default_rng(50)
    D, F, E = 24, 5, 10
    xv, x = _small_int_bf16(rng, (2, D))
    wv, w1 = _small_int_bf16(rng, (E, F, D))
    ids, mask, s2u, cnt = o.route_table(np.array([[5, 7, 9], [7, 9, 2]]))
    out, ad = o.expert_gemm1_table(x, w1, ids, mask, cnt)
    order = [(5, 0), (7, 0), (7, 1), (9, 0), (9, 1), (2, 1)]
    want = np.array([[int(np.dot(xv[t], wv[e, f])) for f in range(F)] for e, t in order])
    assert out.shape == want.shape and np.array_equal(out, want.astype(np.float64)), (out, want)
    want_ad = np.array([[int(np.dot(np.abs(xv[t]), np.abs(wv[e, f]))) for f in range(F)] for e, t in order])
    assert np.array_equal(ad, want_ad.astype(np.float64))


def pin_gemm1_one_hot(o):
    """One-hot weight rows pick single activations exactly."""
    rng = np.random.default_rng(51)
    M, D, F, E = 3, 40, 7, 6
    x = W.gaussian_bf16(rng, (M, D), 1.0)
    w1 = np.zeros((E, F, D), np.uint16)
    pick = rng.integers(0, D, (E, F))
    for e in range(E):
        for f in range(F):
            w1[e, f, pick[e, f]] = 0x3F80  # 1.0
    inds = np.array([[4, 1], [1, 5], [0, 4]], np.int32)
    ids, mask, s2u, cnt = o.route_table(inds)
    out, _ = o.expert_gemm1_table(x, w1, ids, mask, cnt)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    r = 0
    for u in range(cnt):
        for t in range(M):
            if (int(mask[u]) >> t) & 1:
                assert np.array_equal(out[r], xf[t, pick[ids[u]]]), (u, t)
                r += 1
    assert r == out.shape[0]


def pin_gemm1_blas_and_table_rows(o):
    """Random bf16 data: each (token, expert) row equals numpy's float64 product,
    at the row the table's slot map gives."""
    rng = np.random.default_rng(52)
    for M, k in ((1, 4), (2, 6), (5, 3)):
        D, F, E = 64, 9, 12
        x = W.gaussian_bf16(rng, (M, D), 1.0)
        w1 = W.gaussian_bf16(rng, (E, F, D), 0.2)
        inds = np.stack([rng.choice(E, k, replace=False) for _ in range(M)]).astype(np.int32)
        ids, mask, s2u, cnt = o.route_table(inds)
        out, _ = o.expert_gemm1_table(x, w1, ids, mask, cnt)
        rows = o.table_rows(mask, s2u, cnt, M, k)
        xf = W.bf16_bits_to_f32(x).astype(np.float64)
        wf = W.bf16_bits_to_f32(w1).astype(np.float64)
        for t in range(M):
            for j in range(k):
                ref = wf[inds[t, j]] @ xf[t]
                got = out[rows[t, j]]
                assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), (M, t, j)


# OCP FP8 E4M3 values worked out by hand from the format's definition (sign,
# 4-bit exponent with bias 7, 3-bit mantissa, subnormals at exponent 0, NaN at
# S.1111.111, no infinities)
E4M3_HAND = {0x00: 0.0, 0x01: 2.0 ** -9, 0x02: 2.0 ** -8, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x0F: 1.875 * 2.0 ** -6, 0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0,
             0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0x80: -0.0, 0x81: -(2.0 ** -9), 0xB8: -1.0,
             0xC4: -3.0, 0xFE: -448.0}


def _e4m3_numpy(codes):
    """E4M3 decoding with numpy's vector arithmetic (no loop over the format)."""
    c = codes.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 15
    fr = (c & 7).astype(np.float64)
    mag = np.where(ex == 0, fr / 8.0 * 2.0 ** -6, (1.0 + fr / 8.0) * np.exp2(ex - 7.0))
    return sign * mag


def pin_e4m3_table(o):
    for code, v in E4M3_HAND.items():
        got = o.e4m3_value(code)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), (hex(code), got, v)
    assert math.isnan(o.e4m3_value(0x7F)) and math.isnan(o.e4m3_value(0xFF))
    finite = [c for c in range(256) if c & 0x7F != 0x7F]
    assert np.array_equal(np.array([o.e4m3_value(c) for c in finite]), _e4m3_numpy(np.array(finite)))
    assert max(abs(o.e4m3_value(c)) for c in finite) == 448.0


def pin_mx8_dequant(o):
    rng = np.random.default_rng(60)
    E, H = 5, 96
    codes = rng.integers(0, 256, (E, H)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    scales = rng.integers(10, 247, (E, H // 32)).astype(np.uint8)
    w = o.dequant_mxfp8(codes, scales)
    ref = _e4m3_numpy(codes) * np.exp2(np.repeat(scales.astype(np.float64), 32, axis=1) - 127.0)
    assert np.array_equal(w, ref)
    for bad_scale in (9, 247):
        sc = scales.copy()
        sc[2, 1] = bad_scale
        try:
            o.dequant_mxfp8(codes, sc)
        except ValueError:
            continue
        raise AssertionError(f"scale {bad_scale} accepted")
    nan_codes = codes.copy()
    nan_codes[1, 7] = 0xFF
    try:
        o.dequant_mxfp8(nan_codes, scales)
    except ValueError:
        pass
    else:
        raise AssertionError("NaN code accepted")


def pin_mx8_router_is_bf16_router_on_dequantised(o):
    """Every dequantised MXFP8 weight is a bf16 value, so the MXFP8 router equals the
    bf16 router on those weights bit for bit."""
    rng = np.random.default_rng(61)
    M, H, E, k = 3, 128, 32, 4
    x = W.gaussian_bf16(rng, (M, H), 1.0)
    codes = rng.integers(0, 256, (E, H)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x2A
    scales = rng.integers(115, 125, (E, H // 32)).astype(np.uint8)
    wd = o.dequant_mxfp8(codes, scales)
    wb = W.f32_to_bf16_bits(wd.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(wb).astype(np.float64), wd)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    for scoring in (SOFTMAX, SQRT_SOFTPLUS):
        a = o.router_mxfp8(x, codes, scales, bias, k, scoring, True)
        b = o.router(x, wb, bias, k, scoring, True)
        for p, q in zip(a, b):
            assert np.array_equal(p, q)


ALL_PINS = [
    pin_logits_small_integers, pin_logits_rational, pin_logits_one_hot, pin_logits_blas,
    pin_softplus_closed_forms, pin_softplus_logaddexp, pin_softmax_closed_forms,
    pin_topk_brute_force, pin_topk_stable_sort, pin_topk_extremes,
    pin_unbiased_key_is_exact_score_order, pin_all_equal_rows,
    pin_bias_orders_equal_scores, pin_bias_flips_but_weights_unbiased, pin_bias_invariance,
    pin_renorm_sums_and_softmax_identity, pin_softmax_no_renorm_is_probability,
    pin_table_hand_cases, pin_table_invariants, pin_table_verify_widths,
    pin_table_invariants_any_m,
    pin_e2m1_table, pin_mx_dequant, pin_mx_router_is_bf16_router_on_dequantised,
    pin_bf16_round, pin_gather_exact_dyadic, pin_gather_hand_cases, pin_gather_invariants,
    pin_table_rows_hand_cases, pin_table_rows_invariants,
    pin_gemm1_hand_table, pin_gemm1_one_hot, pin_gemm1_blas_and_table_rows,
    pin_e4m3_table, pin_mx8_dequant, pin_mx8_router_is_bf16_router_on_dequantised,
]
