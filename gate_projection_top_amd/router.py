"""Thin Python binding of librouter (include/router.h).

Argument marshalling only: shapes and dtypes are checked, outputs are
allocated with torch on the input's device, and the C entry point of the same
name is called on the current HIP stream.  Every step of the router runs in
librouter's HIP kernels; there is no CPU or PyTorch fallback.  If the library
is not built, loading raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librouter.so")

SOFTMAX = 0
SQRT_SOFTPLUS = 1

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_MISALIGNED = 3
ERR_HIP = 4
ERR_NO_WORKSPACE = 5
ERR_BUSY = 6
ERR_NOT_INITIALIZED = 7
MAX_STREAMS = 8  # ROUTER_MAX_STREAMS

# router_fwd_route_table limits (ROUTER_TABLE_MAX_M / ROUTER_TABLE_MAX_SLOTS)
TABLE_MAX_M = 16
TABLE_MAX_SLOTS = 64
# router_fwd runs the decode kernel up to this many tokens (ROUTER_DECODE_MAX_M)
DECODE_MAX_M = 256

EXPORTS = ("router_init", "router_fwd", "router_fwd_m2_table", "router_fwd_route_table",
           "router_fwd_mxfp4", "router_fwd_mxfp8", "router_topk_from_logits", "router_gather_shared_add",
           "router_gather_shared_add_table", "router_expert_gemm1_table",
           "router_set_exchange_timeout_us", "router_set_decode_wait_limit_us", "router_status",
           "router_fwd_noalloc", "router_release_stream", "router_strerror")
NOALLOC_MAX_M = 4  # ROUTER_NOALLOC_MAX_M
STATUS_WAIT_LIMIT = 1  # ROUTER_STATUS_WAIT_LIMIT: a decode finisher gave a row up

_lib: Optional[ctypes.CDLL] = None


class RouterError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librouter.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; build it with `python -m gate_projection_top_amd.build` "
            "(or __graft_entry__.build()) — there is no fallback path")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.router_init.argtypes = [i32]
    lib.router_init.restype = i32
    lib.router_fwd.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P]
    lib.router_fwd.restype = i32
    lib.router_fwd_noalloc.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P]
    lib.router_fwd_noalloc.restype = i32
    lib.router_fwd_m2_table.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P]
    lib.router_fwd_m2_table.restype = i32
    lib.router_fwd_route_table.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                           P, P]
    lib.router_fwd_route_table.restype = i32
    lib.router_fwd_mxfp4.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P]
    lib.router_fwd_mxfp4.restype = i32
    lib.router_fwd_mxfp8.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P]
    lib.router_fwd_mxfp8.restype = i32
    lib.router_gather_shared_add.argtypes = [P, i64, P, P, P, i64, i32, i32, P, P]
    lib.router_gather_shared_add.restype = i32
    lib.router_gather_shared_add_table.argtypes = [P, P, P, P, P, P, i32, i32, i32, P, P]
    lib.router_gather_shared_add_table.restype = i32
    lib.router_expert_gemm1_table.argtypes = [P, P, i32, i64, i32, P, P, P, i32, i32, P, P]
    lib.router_expert_gemm1_table.restype = i32
    lib.router_topk_from_logits.argtypes = [P, P, i64, i32, i32, i32, i32, P, P, P]
    lib.router_topk_from_logits.restype = i32
    lib.router_set_exchange_timeout_us.argtypes = [i32]
    lib.router_set_exchange_timeout_us.restype = i32
    lib.router_set_decode_wait_limit_us.argtypes = [i32]
    lib.router_set_decode_wait_limit_us.restype = i32
    lib.router_status.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_uint32)]
    lib.router_status.restype = i32
    lib.router_release_stream.argtypes = [P]
    lib.router_release_stream.restype = i32
    lib.router_strerror.argtypes = [i32]
    lib.router_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().router_strerror(int(code)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    """The device's current stream as a raw handle (the cheap accessor when
    this torch has it)."""
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


_SAME_DEVICE = contextlib.nullcontext()


def _on(device: torch.device):
    """Make `device` current for the call (no switch when it already is)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return _SAME_DEVICE
    return torch.cuda.device(device)


def _check(rc: int, where: str):
    if rc != OK:
        raise RouterError(rc, where)


def _check_tensor(t: torch.Tensor, name: str, dtype: torch.dtype, dim: int):
    if (isinstance(t, torch.Tensor) and t.dtype == dtype and t.dim() == dim and t.is_cuda
            and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def init(device: Optional[int] = None):
    """Allocate the device's workspaces now (required before graph capture)."""
    dev = torch.cuda.current_device() if device is None else int(device)
    _check(load().router_init(dev), "router_init")


def release_stream(stream=None):
    """Give back the workspace the stream (default: the current one) holds on
    the current device; only once the stream's router work has finished."""
    s = torch.cuda.current_stream() if stream is None else stream
    _check(load().router_release_stream(ctypes.c_void_p(s.cuda_stream)), "router_release_stream")


def set_exchange_timeout_us(microseconds: int):
    """Bounded wait of a prefill K split for its siblings (0 forces the hand-over path)."""
    _check(load().router_set_exchange_timeout_us(int(microseconds)), "router_set_exchange_timeout_us")


def set_decode_wait_limit_us(microseconds: int):
    """Bound on a decode finisher's wait for the published logits (0 gives
    every row up unless its logits are already in place at the first look)."""
    _check(load().router_set_decode_wait_limit_us(int(microseconds)), "router_set_decode_wait_limit_us")


def status(device: Optional[int] = None, clear: bool = False) -> int:
    """The device's sticky status bits (synchronises the device first)."""
    dev = -1 if device is None else int(device)
    flags = ctypes.c_uint32(0)
    _check(load().router_status(dev, int(bool(clear)), ctypes.byref(flags)), "router_status")
    return int(flags.value)


def _outputs(M: int, k: int, E: int, device, out_inds, out_weights, want_logits, logits_out):
    inds = out_inds if out_inds is not None else torch.empty((M, k), dtype=torch.int32, device=device)
    wts = out_weights if out_weights is not None else torch.empty((M, k), dtype=torch.float32, device=device)
    _check_tensor(inds, "out_inds", torch.int32, 2)
    _check_tensor(wts, "out_weights", torch.float32, 2)
    if tuple(inds.shape) != (M, k) or tuple(wts.shape) != (M, k):
        raise ValueError("out_inds/out_weights must be [M, k]")
    logits = logits_out
    if logits is None and want_logits:
        logits = torch.empty((M, E), dtype=torch.float32, device=device)
    if logits is not None:
        _check_tensor(logits, "logits_out", torch.float32, 2)
        if tuple(logits.shape) != (M, E):
            raise ValueError("logits_out must be [M, E]")
    return inds, wts, logits


def _check_bias(bias, E):
    if bias is not None:
        _check_tensor(bias, "bias", torch.float32, 1)
        if bias.shape[0] != E:
            raise ValueError("bias must be [E]")


def router_fwd(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], k: int,
               scoring: int = SOFTMAX, renorm: bool = True, *, return_logits: bool = False,
               out_inds=None, out_weights=None, logits_out=None):
    """Fused router.  x: bf16 [M,H]; w: bf16 [E,H]; bias: fp32 [E] or None.

    Returns (inds int32 [M,k], weights fp32 [M,k]) or, with return_logits /
    logits_out, (inds, weights, logits fp32 [M,E]).
    """
    _check_tensor(x, "x", torch.bfloat16, 2)
    _check_tensor(w, "w", torch.bfloat16, 2)
    M, H = x.shape
    E = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("x and w disagree on H")
    _check_bias(bias, E)
    inds, wts, logits = _outputs(M, k, E, x.device, out_inds, out_weights, return_logits, logits_out)
    with _on(x.device):
        rc = load().router_fwd(_ptr(x), _ptr(w), _ptr(bias), M, H, E, int(k), int(scoring),
                               int(bool(renorm)), _ptr(inds), _ptr(wts), _ptr(logits),
                               _stream(x.device))
    _check(rc, "router_fwd")
    return (inds, wts, logits) if logits is not None else (inds, wts)


def router_fwd_noalloc(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                       scoring: int = SOFTMAX, renorm: bool = True, *, return_logits: bool = False,
                       out_inds=None, out_weights=None, logits_out=None):
    """router_fwd through the allocation-free entry point (M <= NOALLOC_MAX_M):
    the library allocates nothing for the call; pass preallocated outputs to
    allocate nothing at all."""
    _check_tensor(x, "x", torch.bfloat16, 2)
    _check_tensor(w, "w", torch.bfloat16, 2)
    M, H = x.shape
    E = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("x and w disagree on H")
    _check_bias(bias, E)
    inds, wts, logits = _outputs(M, k, E, x.device, out_inds, out_weights, return_logits, logits_out)
    with _on(x.device):
        rc = load().router_fwd_noalloc(_ptr(x), _ptr(w), _ptr(bias), M, H, E, int(k), int(scoring),
                                       int(bool(renorm)), _ptr(inds), _ptr(wts), _ptr(logits),
                                       _stream(x.device))
    _check(rc, "router_fwd_noalloc")
    return (inds, wts, logits) if logits is not None else (inds, wts)


def router_fwd_mxfp4(x: torch.Tensor, w_fp4: torch.Tensor, w_scale: torch.Tensor,
                     bias: Optional[torch.Tensor], k: int, scoring: int = SOFTMAX,
                     renorm: bool = True, *, return_logits: bool = False,
                     out_inds=None, out_weights=None, logits_out=None):
    """Fused router on an MXFP4 gate.  x: bf16 [M,H]; w_fp4: uint8 [E,H/2]
    (E2M1 codes, even element in the low nibble); w_scale: uint8 [E,H/32]
    (E8M0 scales, each in [2, 252]); bias: fp32 [E] or None.  H % 32 == 0, and
    H % 128 == 0 when M > DECODE_MAX_M.

    Returns what router_fwd returns.
    """
    _check_tensor(x, "x", torch.bfloat16, 2)
    _check_tensor(w_fp4, "w_fp4", torch.uint8, 2)
    _check_tensor(w_scale, "w_scale", torch.uint8, 2)
    M, H = x.shape
    E = w_fp4.shape[0]
    if H % 32 != 0:
        raise ValueError("the MXFP4 gate needs H % 32 == 0")
    if tuple(w_fp4.shape) != (E, H // 2) or tuple(w_scale.shape) != (E, H // 32):
        raise ValueError("w_fp4 must be [E, H/2] and w_scale [E, H/32]")
    _check_bias(bias, E)
    inds, wts, logits = _outputs(M, k, E, x.device, out_inds, out_weights, return_logits, logits_out)
    with _on(x.device):
        rc = load().router_fwd_mxfp4(_ptr(x), _ptr(w_fp4), _ptr(w_scale), _ptr(bias), M, H, E,
                                     int(k), int(scoring), int(bool(renorm)), _ptr(inds), _ptr(wts),
                                     _ptr(logits), _stream(x.device))
    _check(rc, "router_fwd_mxfp4")
    return (inds, wts, logits) if logits is not None else (inds, wts)


def router_fwd_mxfp8(x: torch.Tensor, w_fp8: torch.Tensor, w_scale: torch.Tensor,
                     bias: Optional[torch.Tensor], k: int, scoring: int = SOFTMAX,
                     renorm: bool = True, *, return_logits: bool = False,
                     out_inds=None, out_weights=None, logits_out=None):
    """Fused router on an MXFP8 gate.  x: bf16 [M,H]; w_fp8: uint8 [E,H]
    (E4M3 codes, none NaN); w_scale: uint8 [E,H/32] (E8M0 scales, each in
    [10, 246]); bias: fp32 [E] or None.  H % 32 == 0, and H % 128 == 0 when
    M > DECODE_MAX_M.

    Returns what router_fwd returns.
    """
    _check_tensor(x, "x", torch.bfloat16, 2)
    _check_tensor(w_fp8, "w_fp8", torch.uint8, 2)
    _check_tensor(w_scale, "w_scale", torch.uint8, 2)
    M, H = x.shape
    E = w_fp8.shape[0]
    if H % 32 != 0:
        raise ValueError("the MXFP8 gate needs H % 32 == 0")
    if tuple(w_fp8.shape) != (E, H) or tuple(w_scale.shape) != (E, H // 32):
        raise ValueError("w_fp8 must be [E, H] and w_scale [E, H/32]")
    _check_bias(bias, E)
    inds, wts, logits = _outputs(M, k, E, x.device, out_inds, out_weights, return_logits, logits_out)
    with _on(x.device):
        rc = load().router_fwd_mxfp8(_ptr(x), _ptr(w_fp8), _ptr(w_scale), _ptr(bias), M, H, E,
                                     int(k), int(scoring), int(bool(renorm)), _ptr(inds), _ptr(wts),
                                     _ptr(logits), _stream(x.device))
    _check(rc, "router_fwd_mxfp8")
    return (inds, wts, logits) if logits is not None else (inds, wts)


def router_fwd_route_table(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                           scoring: int = SOFTMAX, renorm: bool = True, *, return_logits: bool = False,
                           out=None):
    """Router plus the unique-route table of its M tokens, one launch
    (1 <= M <= TABLE_MAX_M, M*k <= TABLE_MAX_SLOTS).

    Returns a dict with inds, weights, unique_ids, token_mask, slot_to_unique,
    unique_count (and logits when return_logits).  `out` may supply any of
    these tensors preallocated.
    """
    _check_tensor(x, "x", torch.bfloat16, 2)
    _check_tensor(w, "w", torch.bfloat16, 2)
    M, H = x.shape
    E = w.shape[0]
    if not 1 <= M <= TABLE_MAX_M or M * int(k) > TABLE_MAX_SLOTS:
        raise ValueError(f"the route table needs 1 <= M <= {TABLE_MAX_M} and M*k <= {TABLE_MAX_SLOTS}")
    if w.shape[1] != H:
        raise ValueError("x and w disagree on H")
    _check_bias(bias, E)
    out = dict(out or {})
    inds, wts, logits = _outputs(M, k, E, x.device, out.get("inds"), out.get("weights"),
                                 return_logits, out.get("logits"))
    n = M * int(k)
    tab = {}
    for name, cnt in (("unique_ids", n), ("token_mask", n), ("slot_to_unique", n),
                      ("unique_count", 1)):
        t = out.get(name)
        if t is None:
            t = torch.empty(cnt, dtype=torch.int32, device=x.device)
        _check_tensor(t, name, torch.int32, 1)
        if t.shape[0] != cnt:
            raise ValueError(f"{name} must have {cnt} entries")
        tab[name] = t
    with _on(x.device):
        rc = load().router_fwd_route_table(
            _ptr(x), _ptr(w), _ptr(bias), M, H, E, int(k), int(scoring), int(bool(renorm)),
            _ptr(inds), _ptr(wts), _ptr(logits), _ptr(tab["unique_ids"]), _ptr(tab["token_mask"]),
            _ptr(tab["slot_to_unique"]), _ptr(tab["unique_count"]), _stream(x.device))
    _check(rc, "router_fwd_route_table")
    res = {"inds": inds, "weights": wts, **tab}
    if logits is not None:
        res["logits"] = logits
    return res


def router_fwd_m2_table(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                        scoring: int = SOFTMAX, renorm: bool = True, *, return_logits: bool = False,
                        out=None):
    """Two-token router plus the unique-route table, one launch (the MTP1
    pair; router_fwd_route_table with M = 2)."""
    _check_tensor(x, "x", torch.bfloat16, 2)
    if x.shape[0] != 2:
        raise ValueError("router_fwd_m2_table needs exactly two tokens")
    _check_tensor(w, "w", torch.bfloat16, 2)
    M, H = x.shape
    E = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("x and w disagree on H")
    _check_bias(bias, E)
    out = dict(out or {})
    inds, wts, logits = _outputs(2, k, E, x.device, out.get("inds"), out.get("weights"),
                                 return_logits, out.get("logits"))
    tab = {}
    for name, n in (("unique_ids", 2 * k), ("token_mask", 2 * k), ("slot_to_unique", 2 * k),
                    ("unique_count", 1)):
        t = out.get(name)
        if t is None:
            t = torch.empty(n, dtype=torch.int32, device=x.device)
        _check_tensor(t, name, torch.int32, 1)
        if t.shape[0] != n:
            raise ValueError(f"{name} must have {n} entries")
        tab[name] = t
    with _on(x.device):
        rc = load().router_fwd_m2_table(
            _ptr(x), _ptr(w), _ptr(bias), H, E, int(k), int(scoring), int(bool(renorm)),
            _ptr(inds), _ptr(wts), _ptr(logits), _ptr(tab["unique_ids"]), _ptr(tab["token_mask"]),
            _ptr(tab["slot_to_unique"]), _ptr(tab["unique_count"]), _stream(x.device))
    _check(rc, "router_fwd_m2_table")
    res = {"inds": inds, "weights": wts, **tab}
    if logits is not None:
        res["logits"] = logits
    return res


def router_topk_from_logits(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                            scoring: int = SOFTMAX, renorm: bool = True, *, out_inds=None,
                            out_weights=None):
    """Scoring + top-k + weights on fp32 logits [M,E] already on the GPU."""
    _check_tensor(logits, "logits", torch.float32, 2)
    M, E = logits.shape
    _check_bias(bias, E)
    inds, wts, _ = _outputs(M, k, E, logits.device, out_inds, out_weights, False, None)
    with _on(logits.device):
        rc = load().router_topk_from_logits(_ptr(logits), _ptr(bias), M, E, int(k), int(scoring),
                                            int(bool(renorm)), _ptr(inds), _ptr(wts),
                                            _stream(logits.device))
    _check(rc, "router_topk_from_logits")
    return inds, wts


def router_gather_shared_add(y: torch.Tensor, slot_rows: torch.Tensor, weights: torch.Tensor,
                             shared: torch.Tensor, *, out: Optional[torch.Tensor] = None):
    """Routed gather + shared-expert add.  y: bf16 [R, D]; slot_rows: int32 [M, k]
    (-1 = no row); weights: fp32 [M, k]; shared: bf16 [M, D].  Returns bf16 [M, D]
    (`out` may be `shared`)."""
    _check_tensor(y, "y", torch.bfloat16, 2)
    _check_tensor(slot_rows, "slot_rows", torch.int32, 2)
    _check_tensor(weights, "weights", torch.float32, 2)
    _check_tensor(shared, "shared", torch.bfloat16, 2)
    R, D = y.shape
    M, k = slot_rows.shape
    if tuple(weights.shape) != (M, k) or tuple(shared.shape) != (M, D):
        raise ValueError("weights must be [M, k] and shared [M, D]")
    if out is None:
        out = torch.empty((M, D), dtype=torch.bfloat16, device=y.device)
    _check_tensor(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, D):
        raise ValueError("out must be [M, D]")
    with _on(y.device):
        rc = load().router_gather_shared_add(_ptr(y), R, _ptr(slot_rows), _ptr(weights), _ptr(shared),
                                             M, k, D, _ptr(out), _stream(y.device))
    _check(rc, "router_gather_shared_add")
    return out


def router_gather_shared_add_table(y: torch.Tensor, table: dict, weights: torch.Tensor,
                                   shared: torch.Tensor, *, out: Optional[torch.Tensor] = None):
    """The gather with rows from a unique-route table (the dict router_fwd_route_table
    returns: token_mask, slot_to_unique, unique_count).  y: bf16 [M*k, D] in the
    table's compact layout; weights: fp32 [M, k]; shared: bf16 [M, D]."""
    _check_tensor(y, "y", torch.bfloat16, 2)
    _check_tensor(weights, "weights", torch.float32, 2)
    _check_tensor(shared, "shared", torch.bfloat16, 2)
    M, k = weights.shape
    D = shared.shape[1]
    if tuple(shared.shape) != (M, D) or y.shape[1] != D or y.shape[0] < M * k:
        raise ValueError("shared must be [M, D] and y at least [M*k, D]")
    mask, s2u, cnt = table["token_mask"], table["slot_to_unique"], table["unique_count"]
    for name, t in (("token_mask", mask), ("slot_to_unique", s2u), ("unique_count", cnt)):
        _check_tensor(t, name, torch.int32, 1)
    if mask.numel() < M * k or s2u.numel() < M * k or cnt.numel() < 1:
        raise ValueError("table arrays are too short for M*k slots")
    if out is None:
        out = torch.empty((M, D), dtype=torch.bfloat16, device=y.device)
    _check_tensor(out, "out", torch.bfloat16, 2)
    with _on(y.device):
        rc = load().router_gather_shared_add_table(_ptr(y), _ptr(mask), _ptr(s2u), _ptr(cnt),
                                                   _ptr(weights), _ptr(shared), M, k, D, _ptr(out),
                                                   _stream(y.device))
    _check(rc, "router_gather_shared_add_table")
    return out


def router_expert_gemm1_table(x: torch.Tensor, w1: torch.Tensor, table: dict, k: int, *,
                              out: Optional[torch.Tensor] = None):
    """Expert GEMM1 on the table's compact rows.  x: bf16 [M, D]; w1: bf16 [E, F, D];
    table: router_fwd_route_table's dict (unique_ids, token_mask, unique_count).
    Returns bf16 [M*k, F] (rows past the layout's last are left as they were)."""
    _check_tensor(x, "x", torch.bfloat16, 2)
    _check_tensor(w1, "w1", torch.bfloat16, 3)
    M, D = x.shape
    E, F, D2 = w1.shape
    if D2 != D:
        raise ValueError("x and w1 disagree on D")
    ids, mask, cnt = table["unique_ids"], table["token_mask"], table["unique_count"]
    for name, t in (("unique_ids", ids), ("token_mask", mask), ("unique_count", cnt)):
        _check_tensor(t, name, torch.int32, 1)
    if ids.numel() < M * k or mask.numel() < M * k or cnt.numel() < 1:
        raise ValueError("table arrays are too short for M*k slots")
    if out is None:
        out = torch.empty((M * k, F), dtype=torch.bfloat16, device=x.device)
    _check_tensor(out, "out", torch.bfloat16, 2)
    if out.shape[0] < M * k or out.shape[1] != F:
        raise ValueError("out must be at least [M*k, F]")
    with _on(x.device):
        rc = load().router_expert_gemm1_table(_ptr(x), _ptr(w1), E, F, D, _ptr(ids), _ptr(mask),
                                              _ptr(cnt), M, int(k), _ptr(out), _stream(x.device))
    _check(rc, "router_expert_gemm1_table")
    return out
