"""Row-sharded oracle calls for the full-size parity tests (test infrastructure).

Tokens are independent, so the oracle's result for a block of rows is the
same whether the rows go through it together or in pieces.  These helpers
split the rows into contiguous chunks, run the (unchanged, single-threaded)
oracle on each chunk in its own host thread (the C library runs without the
interpreter lock) and stitch the results back in row order.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def host_threads(limit: int = 16) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(limit, n))


def _sharded(fn, x, threads):
    M = x.shape[0]
    threads = max(1, min(threads, M))
    bounds = np.linspace(0, M, threads + 1).astype(int)
    chunks = [(bounds[i], bounds[i + 1]) for i in range(threads) if bounds[i + 1] > bounds[i]]
    with ThreadPoolExecutor(max_workers=len(chunks)) as pool:
        parts = list(pool.map(lambda c: fn(x[c[0]:c[1]]), chunks))
    return tuple(np.concatenate([p[i] for p in parts], axis=0) for i in range(len(parts[0])))


def router(orc, x, w, bias, k, scoring, renorm, threads=None):
    """orc.router over row chunks: (inds, weights, logits, absdot) for every row of x."""
    return _sharded(lambda xs: orc.router(xs, w, bias, k, scoring, renorm), x,
                    threads or host_threads())


def router_mxfp4(orc, x, elems, scales, bias, k, scoring, renorm, threads=None):
    return _sharded(lambda xs: orc.router_mxfp4(xs, elems, scales, bias, k, scoring, renorm), x,
                    threads or host_threads())


def router_mxfp8(orc, x, elems, scales, bias, k, scoring, renorm, threads=None):
    return _sharded(lambda xs: orc.router_mxfp8(xs, elems, scales, bias, k, scoring, renorm), x,
                    threads or host_threads())
