"""CPU oracle for the fused MoE router — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``gate_projection_top_amd``) never
imports it and never falls back to it.

The arithmetic lives in ``oracle.c`` (plain single-threaded C99, fp64); this
module builds it with gcc if needed and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SOURCES = [os.path.join(HERE, "oracle.c")]

SOFTMAX = 0
SQRT_SOFTPLUS = 1

# -O2, no fast-math, no FMA contraction: every double operation rounds as written.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(out: str = LIB_PATH, sources=None, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library; return its path."""
    srcs = list(sources) if sources is not None else SOURCES
    cmd = ["gcc", *CFLAGS, *extra_flags, "-I", HERE, *srcs, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes binding of one compiled oracle library."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            build(path)
        self.path = path
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.oracle_logits.argtypes = [P, P, i64, i64, i64, P, P]
        lib.oracle_topk_from_logits.argtypes = [P, P, i64, i64, ci, ci, ci, P, P]
        lib.oracle_router.argtypes = [P, P, P, i64, i64, i64, ci, ci, ci, P, P, P, P]
        lib.oracle_route_table.argtypes = [P, ci, ci, P, P, P, P]
        lib.oracle_e2m1_value.argtypes = [ci]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_dequant_mxfp4.argtypes = [P, P, i64, i64, P]
        lib.oracle_dequant_mxfp4.restype = ci
        lib.oracle_router_mxfp4.argtypes = [P, P, P, P, i64, i64, i64, ci, ci, ci, P, P, P, P]
        lib.oracle_router_mxfp4.restype = ci
        lib.oracle_e4m3_value.argtypes = [ci]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_dequant_mxfp8.argtypes = [P, P, i64, i64, P]
        lib.oracle_dequant_mxfp8.restype = ci
        lib.oracle_router_mxfp8.argtypes = [P, P, P, P, i64, i64, i64, ci, ci, ci, P, P, P, P]
        lib.oracle_router_mxfp8.restype = ci
        lib.oracle_bf16_round.argtypes = [ctypes.c_float]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_gather_shared_add.argtypes = [P, i64, i64, P, P, P, i64, ci, P]
        lib.oracle_gather_shared_add.restype = ci
        lib.oracle_table_rows.argtypes = [P, P, ci, ci, ci, P]
        lib.oracle_table_rows.restype = ci
        lib.oracle_expert_gemm1_table.argtypes = [P, P, i64, i64, i64, P, P, ci, ci, P, P]
        lib.oracle_expert_gemm1_table.restype = ci
        lib.oracle_route_table_m2.argtypes = [P, ci, P, P, P, P]
        lib.oracle_row_scores.argtypes = [P, i64, ci, P, P]
        for f in (lib.oracle_logits, lib.oracle_topk_from_logits, lib.oracle_router,
                  lib.oracle_route_table, lib.oracle_route_table_m2, lib.oracle_row_scores):
            f.restype = ci
        self.lib = lib

    @staticmethod
    def _ptr(a: Optional[np.ndarray]):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    def logits(self, x: np.ndarray, w: np.ndarray):
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        M, H = x.shape
        E = w.shape[0]
        assert w.shape[1] == H
        out = np.empty((M, E), np.float32)
        absdot = np.empty((M, E), np.float64)
        rc = self.lib.oracle_logits(self._ptr(x), self._ptr(w), M, H, E, self._ptr(out),
                                    self._ptr(absdot))
        if rc:
            raise ValueError(f"oracle_logits failed: {rc}")
        return out, absdot

    def topk_from_logits(self, logits: np.ndarray, bias: Optional[np.ndarray], k: int,
                         scoring: int, renorm: bool):
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        M, E = logits.shape
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        inds = np.empty((M, k), np.int32)
        wts = np.empty((M, k), np.float32)
        rc = self.lib.oracle_topk_from_logits(self._ptr(logits), self._ptr(b), M, E, k,
                                              int(scoring), int(bool(renorm)),
                                              self._ptr(inds), self._ptr(wts))
        if rc:
            raise ValueError(f"oracle_topk_from_logits failed: {rc}")
        return inds, wts

    def router(self, x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray], k: int,
               scoring: int, renorm: bool):
        """Return (inds, weights, logits, absdot)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        M, H = x.shape
        E = w.shape[0]
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        inds = np.empty((M, k), np.int32)
        wts = np.empty((M, k), np.float32)
        lg = np.empty((M, E), np.float32)
        ad = np.empty((M, E), np.float64)
        rc = self.lib.oracle_router(self._ptr(x), self._ptr(w), self._ptr(b), M, H, E, k,
                                    int(scoring), int(bool(renorm)), self._ptr(inds),
                                    self._ptr(wts), self._ptr(lg), self._ptr(ad))
        if rc:
            raise ValueError(f"oracle_router failed: {rc}")
        return inds, wts, lg, ad

    def e2m1_value(self, code: int) -> float:
        return float(self.lib.oracle_e2m1_value(int(code)))

    def dequant_mxfp4(self, elems: np.ndarray, scales: np.ndarray) -> np.ndarray:
        """elems uint8 [E, H/2], scales uint8 [E, H/32] -> float64 [E, H]."""
        elems = np.ascontiguousarray(elems, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        E, H = elems.shape[0], elems.shape[1] * 2
        w = np.empty((E, H), np.float64)
        rc = self.lib.oracle_dequant_mxfp4(self._ptr(elems), self._ptr(scales), E, H, self._ptr(w))
        if rc:
            raise ValueError(f"oracle_dequant_mxfp4 failed: {rc}")
        return w

    def router_mxfp4(self, x: np.ndarray, elems: np.ndarray, scales: np.ndarray,
                     bias: Optional[np.ndarray], k: int, scoring: int, renorm: bool):
        """Router on MXFP4 gate weights: (inds, weights, logits, absdot)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        elems = np.ascontiguousarray(elems, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        M, H = x.shape
        E = elems.shape[0]
        assert elems.shape[1] * 2 == H and scales.shape == (E, H // 32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        inds = np.empty((M, k), np.int32)
        wts = np.empty((M, k), np.float32)
        lg = np.empty((M, E), np.float32)
        ad = np.empty((M, E), np.float64)
        rc = self.lib.oracle_router_mxfp4(self._ptr(x), self._ptr(elems), self._ptr(scales),
                                          self._ptr(b), M, H, E, k, int(scoring), int(bool(renorm)),
                                          self._ptr(inds), self._ptr(wts), self._ptr(lg), self._ptr(ad))
        if rc:
            raise ValueError(f"oracle_router_mxfp4 failed: {rc}")
        return inds, wts, lg, ad

    def e4m3_value(self, code: int) -> float:
        return float(self.lib.oracle_e4m3_value(int(code)))

    def dequant_mxfp8(self, elems: np.ndarray, scales: np.ndarray) -> np.ndarray:
        elems = np.ascontiguousarray(elems, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        E, H = elems.shape
        w = np.empty((E, H), np.float64)
        rc = self.lib.oracle_dequant_mxfp8(self._ptr(elems), self._ptr(scales), E, H, self._ptr(w))
        if rc:
            raise ValueError(f"oracle_dequant_mxfp8 failed: {rc}")
        return w

    def router_mxfp8(self, x: np.ndarray, elems: np.ndarray, scales: np.ndarray,
                     bias: Optional[np.ndarray], k: int, scoring: int, renorm: bool):
        """Router on MXFP8 gate weights: (inds, weights, logits, absdot)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        elems = np.ascontiguousarray(elems, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        M, H = x.shape
        E = elems.shape[0]
        assert elems.shape[1] == H and scales.shape == (E, H // 32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        inds = np.empty((M, k), np.int32)
        wts = np.empty((M, k), np.float32)
        lg = np.empty((M, E), np.float32)
        ad = np.empty((M, E), np.float64)
        rc = self.lib.oracle_router_mxfp8(self._ptr(x), self._ptr(elems), self._ptr(scales),
                                          self._ptr(b), M, H, E, k, int(scoring), int(bool(renorm)),
                                          self._ptr(inds), self._ptr(wts), self._ptr(lg), self._ptr(ad))
        if rc:
            raise ValueError(f"oracle_router_mxfp8 failed: {rc}")
        return inds, wts, lg, ad

    def route_table(self, inds: np.ndarray):
        """Unique-route table of inds [M, k] (slots token-major)."""
        inds = np.ascontiguousarray(inds, dtype=np.int32)
        assert inds.ndim == 2
        M, k = inds.shape
        ids = np.empty(M * k, np.int32)
        mask = np.empty(M * k, np.int32)
        s2u = np.empty(M * k, np.int32)
        cnt = np.empty(1, np.int32)
        rc = self.lib.oracle_route_table(self._ptr(inds), M, k, self._ptr(ids), self._ptr(mask),
                                         self._ptr(s2u), self._ptr(cnt))
        if rc:
            raise ValueError(f"oracle_route_table failed: {rc}")
        return ids, mask, s2u, int(cnt[0])

    def route_table_m2(self, inds: np.ndarray):
        inds = np.ascontiguousarray(inds, dtype=np.int32)
        assert inds.shape[0] == 2
        k = inds.shape[1]
        ids = np.empty(2 * k, np.int32)
        mask = np.empty(2 * k, np.int32)
        s2u = np.empty(2 * k, np.int32)
        cnt = np.empty(1, np.int32)
        rc = self.lib.oracle_route_table_m2(self._ptr(inds), k, self._ptr(ids), self._ptr(mask),
                                            self._ptr(s2u), self._ptr(cnt))
        if rc:
            raise ValueError(f"oracle_route_table_m2 failed: {rc}")
        return ids, mask, s2u, int(cnt[0])

    def bf16_round(self, f: float) -> int:
        """BF16 bits of an fp32 value, to nearest, ties to even."""
        return int(self.lib.oracle_bf16_round(float(np.float32(f))))

    def gather_shared_add(self, y: np.ndarray, slot_rows: np.ndarray, weights: np.ndarray,
                          shared: np.ndarray) -> np.ndarray:
        """Routed gather + shared add.  y: bf16 bits [R, D]; slot_rows: int32 [M, k];
        weights: fp32 [M, k]; shared: bf16 bits [M, D].  Returns bf16 bits [M, D]."""
        y = np.ascontiguousarray(y, dtype=np.uint16)
        slot_rows = np.ascontiguousarray(slot_rows, dtype=np.int32)
        weights = np.ascontiguousarray(weights, dtype=np.float32)
        shared = np.ascontiguousarray(shared, dtype=np.uint16)
        R, D = y.shape
        M, k = slot_rows.shape
        assert weights.shape == (M, k) and shared.shape == (M, D)
        out = np.empty((M, D), np.uint16)
        rc = self.lib.oracle_gather_shared_add(self._ptr(y), R, D, self._ptr(slot_rows),
                                               self._ptr(weights), self._ptr(shared), M, k,
                                               self._ptr(out))
        if rc:
            raise ValueError(f"oracle_gather_shared_add failed: {rc}")
        return out

    def table_rows(self, token_mask: np.ndarray, slot_to_unique: np.ndarray, count: int, M: int,
                   k: int) -> np.ndarray:
        """Compact expert-output rows [M, k] that the unique-route table implies."""
        token_mask = np.ascontiguousarray(token_mask, dtype=np.int32)
        slot_to_unique = np.ascontiguousarray(slot_to_unique, dtype=np.int32)
        rows = np.empty(M * k, np.int32)
        rc = self.lib.oracle_table_rows(self._ptr(token_mask), self._ptr(slot_to_unique), int(count),
                                        int(M), int(k), self._ptr(rows))
        if rc:
            raise ValueError(f"oracle_table_rows failed: {rc}")
        return rows.reshape(M, k)

    def expert_gemm1_table(self, x: np.ndarray, w1: np.ndarray, unique_ids: np.ndarray,
                           token_mask: np.ndarray, count: int):
        """Expert GEMM1 on the table's compact rows.  x: bf16 bits [M, D];
        w1: bf16 bits [E, F, D].  Returns (exact [rows, F] float64, absdot [rows, F])."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w1 = np.ascontiguousarray(w1, dtype=np.uint16)
        ids = np.ascontiguousarray(unique_ids, dtype=np.int32)
        mask = np.ascontiguousarray(token_mask, dtype=np.int32)
        M, D = x.shape
        E, F, D2 = w1.shape
        assert D2 == D
        nrows = sum(bin(int(m) & ((1 << M) - 1)).count("1") for m in mask[:count])
        out = np.empty((max(nrows, 1), F), np.float64)
        ad = np.empty((max(nrows, 1), F), np.float64)
        rc = self.lib.oracle_expert_gemm1_table(self._ptr(x), self._ptr(w1), E, F, D, self._ptr(ids),
                                                self._ptr(mask), int(count), M, self._ptr(out),
                                                self._ptr(ad))
        if rc < 0:
            raise ValueError(f"oracle_expert_gemm1_table failed: {rc}")
        return out[:rc], ad[:rc]

    def row_scores(self, row: np.ndarray, scoring: int):
        row = np.ascontiguousarray(row, dtype=np.float32)
        E = row.shape[0]
        s = np.empty(E, np.float64)
        u = np.empty(E, np.float64)
        rc = self.lib.oracle_row_scores(self._ptr(row), E, int(scoring), self._ptr(s), self._ptr(u))
        if rc:
            raise ValueError(f"oracle_row_scores failed: {rc}")
        return s, u


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from oracle.c (built on first use if missing).

    ``ORACLE_LIB`` in the environment names another build of the same source
    (the sanitizer build the CPU tests make) to load instead.
    """
    global _default
    if _default is None:
        _default = Oracle(os.environ.get("ORACLE_LIB") or LIB_PATH)
    return _default
