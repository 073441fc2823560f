"""Parity rules between the HIP path and the oracle — TEST INFRASTRUCTURE ONLY.

Rule (a), standalone top-k on given logits: indices bit-exact, weights within
2 ulp (integer distance of the fp32 bit patterns; weights are positive).

Rule (b), fused router: logits within 1e-4 * sum_i |x_i w_i| of the oracle's;
weights within 1e-5 relative; indices bit-exact wherever the oracle's
selection is resolved by more than that logit bound; inside the band the
GPU's selection must be a valid top-k of its *own* logits (checked by running
the oracle's selection on the logits the kernel returns, which must then agree
bit for bit, indices and weights within 2 ulp).

Rule (c), unique-route tables: bit-exact against the oracle's table of the
same indices.

Band classifier (per row).  With delta_e = 1e-4 * A[t,e], each key is
bounded by propagating logit_e +- delta_e through the key map:
  no bias:           key = logit;
  sqrt-softplus:     key = s(l) + b, s increasing;
  softmax with bias: key = p + b, p_e scaled by at most exp(+-(delta_e + max delta)).
The cut after rank k is *resolved* iff the smallest lower bound among the
oracle's winners exceeds the largest upper bound among the rest; the order of
two adjacent winners is resolved iff their intervals are disjoint.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SOFTMAX, SQRT_SOFTPLUS = 0, 1
LOGIT_TOL = 1e-4
WEIGHT_RTOL = 1e-5
WEIGHT_ULPS = 2


def ulp_distance(a, b) -> np.ndarray:
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def _sqrt_softplus(x: np.ndarray) -> np.ndarray:
    return np.sqrt(np.logaddexp(0.0, x))


def key_intervals(logits: np.ndarray, absdot: np.ndarray, bias: Optional[np.ndarray],
                  scoring: int):
    """Lower/upper bounds of every selection key under rule (b)'s logit bound."""
    l = logits.astype(np.float64)
    d = LOGIT_TOL * absdot
    if bias is None:
        lo, hi = l - d, l + d
    elif scoring == SQRT_SOFTPLUS:
        lo = _sqrt_softplus(l - d) + bias
        hi = _sqrt_softplus(l + d) + bias
    else:
        m = l.max(axis=1, keepdims=True)
        z = np.exp(l - m)
        p = z / z.sum(axis=1, keepdims=True)
        spread = d + d.max(axis=1, keepdims=True)
        lo = p * np.exp(-spread) + bias
        hi = p * np.exp(spread) + bias
    # fp32 rounding of the key itself (score and sum), with margin
    eps = 4 * np.finfo(np.float32).eps * np.maximum(np.abs(lo), np.abs(hi))
    return lo - eps, hi + eps


@dataclasses.dataclass
class BandInfo:
    cut_resolved: np.ndarray     # bool [M]
    order_resolved: np.ndarray   # bool [M]: cut and every adjacent pair resolved


def classify(inds: np.ndarray, logits: np.ndarray, absdot: np.ndarray,
             bias: Optional[np.ndarray], scoring: int) -> BandInfo:
    lo, hi = key_intervals(logits, absdot, bias, scoring)
    M, E = logits.shape
    k = inds.shape[1]
    cut = np.zeros(M, bool)
    order = np.zeros(M, bool)
    for t in range(M):
        sel = np.zeros(E, bool)
        sel[inds[t]] = True
        if k == E:
            cut[t] = True
        else:
            cut[t] = lo[t, sel].min() > hi[t, ~sel].max()
        pairs = all(lo[t, inds[t, j]] > hi[t, inds[t, j + 1]] for j in range(k - 1))
        order[t] = cut[t] and pairs
    return BandInfo(cut, order)


@dataclasses.dataclass
class RouterReport:
    rows: int
    band_rows: int          # rows whose cut is not resolved by the logit bound
    band_rows_exact: int    # of those, how many matched the oracle exactly anyway
    max_logit_err_ratio: float
    max_weight_rel_err: float


def check_topk(gpu_inds, gpu_w, ref_inds, ref_w, what: str = "topk"):
    """Rule (a)."""
    gpu_inds = np.asarray(gpu_inds)
    if not np.array_equal(gpu_inds, ref_inds):
        bad = np.flatnonzero((gpu_inds != ref_inds).any(axis=1))
        r = int(bad[0])
        raise AssertionError(f"{what}: indices differ in {bad.size} rows; first row {r}: "
                             f"gpu {gpu_inds[r].tolist()} oracle {ref_inds[r].tolist()}")
    d = ulp_distance(gpu_w, ref_w)
    if d.max(initial=0) > WEIGHT_ULPS:
        r, j = np.unravel_index(int(np.argmax(d)), d.shape)
        raise AssertionError(f"{what}: weight [{r},{j}] off by {int(d[r, j])} ulp "
                             f"(gpu {gpu_w[r, j]!r}, oracle {ref_w[r, j]!r})")


def check_router(orc, case, gpu_inds, gpu_w, gpu_logits, ref=None, rows=None) -> RouterReport:
    """Rule (b) for a router case (optionally on a subset of rows).

    gpu_logits is the kernel's own logits output for the same call (needed
    for the in-band self-consistency check).  ref: the oracle's (inds, w,
    logits, absdot) on the same rows, computed here when None.
    """
    x = case.x if rows is None else case.x[rows]
    if ref is None:
        ref = orc.router(x, case.w, case.bias, case.k, case.scoring, case.renorm)
    r_inds, r_w, r_lg, r_ad = ref
    gpu_inds = np.asarray(gpu_inds)
    gpu_w = np.asarray(gpu_w)
    gpu_logits = np.asarray(gpu_logits)
    M = x.shape[0]
    assert gpu_inds.shape == r_inds.shape and gpu_logits.shape == r_lg.shape

    # logits within the bound
    err = np.abs(gpu_logits.astype(np.float64) - r_lg.astype(np.float64))
    bound = LOGIT_TOL * r_ad
    ratio = float((err / np.maximum(bound, 1e-300)).max(initial=0.0))
    if not np.all(err <= bound):
        t, e = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        raise AssertionError(f"{case.name}: logit [{t},{e}] off by {err[t, e]:.3e} "
                             f"> bound {bound[t, e]:.3e}")

    # self-consistency: the GPU's selection is the contract's top-k of its own logits
    s_inds, s_w = orc.topk_from_logits(gpu_logits, case.bias, case.k, case.scoring, case.renorm)
    check_topk(gpu_inds, gpu_w, s_inds, s_w, what=f"{case.name} (own logits)")

    # against the oracle's selection where the band classifier resolves it
    band = classify(r_inds, r_lg, r_ad, case.bias, case.scoring)
    max_wrel = 0.0
    exact_in_band = 0
    for t in range(M):
        same = np.array_equal(gpu_inds[t], r_inds[t])
        if band.order_resolved[t] and not same:
            raise AssertionError(f"{case.name}: row {t} resolved but indices differ: "
                                 f"gpu {gpu_inds[t].tolist()} oracle {r_inds[t].tolist()}")
        if band.cut_resolved[t] and set(gpu_inds[t].tolist()) != set(r_inds[t].tolist()):
            raise AssertionError(f"{case.name}: row {t} cut resolved but sets differ: "
                                 f"gpu {gpu_inds[t].tolist()} oracle {r_inds[t].tolist()}")
        if not band.cut_resolved[t] and same:
            exact_in_band += 1
        if set(gpu_inds[t].tolist()) == set(r_inds[t].tolist()):
            # weights of the same experts, matched by index
            g = dict(zip(gpu_inds[t].tolist(), gpu_w[t].tolist()))
            for e, wr in zip(r_inds[t].tolist(), r_w[t].tolist()):
                rel = abs(g[e] - wr) / abs(wr) if wr != 0 else abs(g[e])
                max_wrel = max(max_wrel, rel)
                if rel > WEIGHT_RTOL:
                    raise AssertionError(f"{case.name}: row {t} expert {e} weight rel err "
                                         f"{rel:.3e} > {WEIGHT_RTOL}")
    n_band = int((~band.cut_resolved).sum())
    return RouterReport(M, n_band, exact_in_band, ratio, max_wrel)


def check_table(orc, gpu_inds, table: dict):
    """Rule (c): the emitted table equals the oracle's table of the same indices
    (gpu_inds: [M, k])."""
    ids, mask, s2u, cnt = orc.route_table(np.asarray(gpu_inds, np.int32))
    got = {k: np.asarray(v) for k, v in table.items()}
    assert np.array_equal(got["unique_ids"], ids), (got["unique_ids"], ids)
    assert np.array_equal(got["token_mask"], mask), (got["token_mask"], mask)
    assert np.array_equal(got["slot_to_unique"], s2u), (got["slot_to_unique"], s2u)
    assert int(got["unique_count"][0]) == cnt, (got["unique_count"], cnt)
