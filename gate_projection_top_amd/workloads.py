"""Seeded synthetic inputs for the fused MoE router.

This module only *builds inputs*: activations, gate matrices, selection biases
and pre-computed logit rows.  It holds none of the router's arithmetic (no dot
products, no scoring, no selection, no renormalisation), so both the HIP path
and the CPU oracle can draw from it without sharing any of the method.

Every generator is a pure function of its seed (numpy PCG64).  bf16 tensors are
returned as their raw uint16 bit patterns (round-to-nearest-even from fp32).

The shapes and distributions follow the workloads the router pages talk about:
a 256-expert gate at hidden sizes 4096 and 7168, top-8 (softmax) and top-6
(sqrt-softplus plus selection bias, the DeepSeek-V4 style), decode verify widths
M in {1, 2, 8} and up to 64, and an 8192-token prefill.  No model weights exist
here, so gate matrices are N(0, 1/H) and activations N(0, 1), which gives logits
of unit scale, as a trained router's pre-activation logits roughly are.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SOFTMAX = 0
SQRT_SOFTPLUS = 1


# --------------------------------------------------------------------------
# bf16 helpers (input encoding only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction, so the NaN case is not handled.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class RouterCase:
    """One router invocation's inputs (host arrays) and its settings."""
    x: np.ndarray            # uint16 [M, H]  bf16 bits
    w: np.ndarray            # uint16 [E, H]  bf16 bits
    bias: Optional[np.ndarray]  # float32 [E] or None
    k: int
    scoring: int
    renorm: bool
    name: str = ""

    @property
    def M(self) -> int:
        return int(self.x.shape[0])

    @property
    def H(self) -> int:
        return int(self.x.shape[1])

    @property
    def E(self) -> int:
        return int(self.w.shape[0])


@dataclasses.dataclass
class LogitsCase:
    """One logits-to-top-k invocation's inputs."""
    logits: np.ndarray       # float32 [M, E]
    bias: Optional[np.ndarray]
    k: int
    scoring: int
    renorm: bool
    row_kind: np.ndarray     # int8 [M]: 0 plain, 1 exact tie, 2 one-ulp chain, 3 all equal
    name: str = ""


def _rng(seed: int, stream: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(stream)]))


def gaussian_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def rms_normalised_bf16(rng: np.random.Generator, M: int, H: int, eps: float = 1e-6) -> np.ndarray:
    """N(0,1) rows scaled to unit RMS (fp64, no gain), then rounded to bf16.

    Stands in for the post-RMSNorm hidden state that feeds a decode router.
    """
    x = rng.standard_normal((M, H))
    x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return f32_to_bf16_bits(x.astype(np.float32))


# --------------------------------------------------------------------------
# Router workloads
# --------------------------------------------------------------------------
def tiny_case(seed: int = 0) -> RouterCase:
    """M=4, H=256, E=16, k=2, softmax, no bias, renorm."""
    rng = _rng(seed, 1)
    M, H, E = 4, 256, 16
    x = gaussian_bf16(rng, (M, H), 1.0)
    w = gaussian_bf16(rng, (E, H), 1.0 / np.sqrt(H))
    return RouterCase(x, w, None, 2, SOFTMAX, True, name=f"tiny/seed{seed}")


def tiny_tie_cases(seed: int = 0) -> list:
    """Four single-token routers whose logits hold exact ties near the k=2 cut.

    Ties are made structurally: two or three experts get *the same* bf16 gate
    row, so any correct dot product gives bitwise-equal logits for them.  The
    shared row is a scaled copy of the token so that the tied logits sit far
    above the N(0,1) background; a further expert with twice that row is
    placed above them when the tie must straddle the cut.

      kind 0: one expert above, pair tied at ranks 2/3, lower index is the smaller one
      kind 1: same, with the copy placed on the lower index
      kind 2: pair tied at the very top (both selected, order by index)
      kind 3: three-way tie at ranks 2/3/4
    """
    rng = _rng(seed, 2)
    H, E = 256, 16
    out = []
    for kind in range(4):
        xf = rng.standard_normal(H).astype(np.float32)
        x = f32_to_bf16_bits(xf)
        xb = bf16_bits_to_f32(x).astype(np.float64)
        w = gaussian_bf16(rng, (E, H), 1.0 / np.sqrt(H))
        c = 6.0 / float(xb @ xb)          # shared row logit ~ +6
        shared = f32_to_bf16_bits((c * xb).astype(np.float32))
        double = f32_to_bf16_bits((2.0 * c * xb).astype(np.float32))
        experts = rng.permutation(E)
        if kind in (0, 1):
            a, b, d = (int(v) for v in experts[:3])
            lo, hi = min(b, d), max(b, d)
            src, dst = (lo, hi) if kind == 0 else (hi, lo)
            w[a] = double
            w[src] = shared
            w[dst] = w[src]
        elif kind == 2:
            b, d = (int(v) for v in experts[:2])
            w[b] = shared
            w[d] = shared
        else:
            a, b, d, f = (int(v) for v in experts[:4])
            w[a] = double
            w[b] = shared
            w[d] = shared
            w[f] = shared
        out.append(RouterCase(x[None, :], w, None, 2, SOFTMAX, True,
                              name=f"tiny-tie/kind{kind}/seed{seed}"))
    return out


def decode_case(M: int, H: int = 4096, seed: int = 0, E: int = 256, k: int = 8) -> RouterCase:
    """Verify-width decode router: unit-RMS activations, softmax, no bias, renorm."""
    rng = _rng(seed, 3)
    x = rms_normalised_bf16(rng, M, H)
    w = gaussian_bf16(rng, (E, H), 1.0 / np.sqrt(H))
    return RouterCase(x, w, None, k, SOFTMAX, True, name=f"decode/M{M}/H{H}/seed{seed}")


def decode_gate_pool(n: int, H: int, seed: int, E: int = 256) -> np.ndarray:
    """n distinct gate matrices (one per MoE layer), uint16 [n, E, H]."""
    rng = _rng(seed, 4)
    return gaussian_bf16(rng, (n, E, H), 1.0 / np.sqrt(H))


def biased_case(M: int, seed: int = 0, H: int = 4096, E: int = 256, k: int = 6,
                force_shared: Optional[bool] = None) -> RouterCase:
    """DeepSeek-V4-style router: sqrt-softplus scores, U(-0.05,0.05) selection bias.

    At M=2, seeds with seed % 10 < 3 (or force_shared=True) overwrite 1..6 gate
    rows with a scaled copy of (x0/|x0|^2 + x1/|x1|^2), which puts those
    experts' logits near +4 for *both* tokens, so the two tokens share them.
    """
    rng = _rng(seed, 5)
    x = gaussian_bf16(rng, (M, H), 1.0)
    w = gaussian_bf16(rng, (E, H), 1.0 / np.sqrt(H))
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    if force_shared is None:
        force_shared = (M == 2 and seed % 10 < 3)
    if force_shared:
        assert M == 2
        xb = bf16_bits_to_f32(x).astype(np.float64)
        xhat = xb[0] / (xb[0] @ xb[0]) + xb[1] / (xb[1] @ xb[1])
        s = int(rng.integers(1, 7))
        rows = rng.choice(E, size=s, replace=False)
        for r in rows:
            alpha = 4.0 + 0.25 * rng.standard_normal()
            w[r] = f32_to_bf16_bits((alpha * xhat).astype(np.float32))
    return RouterCase(x, w, bias, k, SQRT_SOFTPLUS, True, name=f"biased/M{M}/seed{seed}")


def verify_table_case(M: int, seed: int = 0, H: int = 4096, E: int = 256, k: int = 8,
                      biased: bool = False) -> RouterCase:
    """M tokens at a verify width for the unique-route table: the decode router
    (softmax, no bias, k=8) or, with biased=True, the sqrt-softplus router with a
    U(-0.05,0.05) selection bias.  Seeds with seed % 10 < 5 overwrite 1..k gate
    rows with a scaled copy of sum_t x_t/|x_t|^2, which every token then picks,
    and (odd seeds among those) 1..3 more rows with the same construction over
    the first half of the tokens only, so masks cover all-tokens, some-tokens and
    one-token experts."""
    rng = _rng(seed, 9)
    x = gaussian_bf16(rng, (M, H), 1.0)
    w = gaussian_bf16(rng, (E, H), 1.0 / np.sqrt(H))
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32) if biased else None
    if seed % 10 < 5:
        xb = bf16_bits_to_f32(x).astype(np.float64)
        unit = xb / np.einsum("th,th->t", xb, xb)[:, None]
        groups = [np.arange(M)]
        if seed % 2 == 1 and M > 1:
            groups.append(np.arange((M + 1) // 2))
        rows = rng.choice(E, size=int(rng.integers(1, k + 1)) + 3, replace=False)
        at = 0
        for gi, tok in enumerate(groups):
            count = int(rng.integers(1, k + 1)) if gi == 0 else int(rng.integers(1, 4))
            for r in rows[at:at + count]:
                alpha = 4.0 + 0.25 * rng.standard_normal()
                w[r] = f32_to_bf16_bits((alpha * unit[tok].sum(axis=0)).astype(np.float32))
            at += count
    scoring = SQRT_SOFTPLUS if biased else SOFTMAX
    kind = "biased" if biased else "softmax"
    return RouterCase(x, w, bias, k, scoring, True, name=f"table/{kind}/M{M}/k{k}/seed{seed}")


E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # OCP MX FP4 codes 0..7


def quantise_mxfp4(w: np.ndarray):
    """Synthetic MXFP4 weights from real ones [E, H] (H % 32 == 0): per 32-block an E8M0
    scale 2^(ceil(log2(amax / 6))) (so the block's largest magnitude fits E2M1's 6), codes
    by nearest magnitude; even element in the low nibble.  Returns (elems uint8 [E, H/2],
    scales uint8 [E, H/32]).  Input construction only: the router never quantises."""
    E, H = w.shape
    assert H % 32 == 0
    blocks = w.astype(np.float64).reshape(E, H // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    ex = np.ceil(np.log2(np.maximum(amax, 1e-30) / 6.0)).astype(np.int64)
    ex = np.clip(ex, 2 - 127, 252 - 127)
    scaled = blocks / np.ldexp(1.0, ex)[:, :, None]
    mag = np.abs(scaled)
    code = np.abs(mag[..., None] - E2M1_MAGNITUDES).argmin(axis=-1)
    code = code | np.where(scaled < 0, 8, 0)
    code = code.reshape(E, H).astype(np.uint8)
    elems = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    scales = (ex + 127).astype(np.uint8)
    return elems, scales


@dataclasses.dataclass
class MxCase:
    x: np.ndarray        # bf16 bits [M, H]
    elems: np.ndarray    # uint8 [E, H/2] (MXFP4) or [E, H] (MXFP8)
    scales: np.ndarray   # uint8 [E, H/32]
    bias: Optional[np.ndarray]
    k: int
    scoring: int
    renorm: bool
    name: str = ""


def mxfp4_case(M: int, H: int = 4096, seed: int = 0, E: int = 256, k: int = 8,
               scoring: int = SOFTMAX, with_bias: bool = False, renorm: bool = True) -> MxCase:
    """Router on MXFP4 gate weights: X = unit-RMS N(0,1) rows in bf16, W ~ N(0,1/H)
    quantised to MXFP4 (quantise_mxfp4); optional U(-0.05,0.05) selection bias."""
    rng = _rng(seed, 10)
    x = rms_normalised_bf16(rng, M, H)
    w = rng.standard_normal((E, H)) / np.sqrt(H)
    elems, scales = quantise_mxfp4(w)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32) if with_bias else None
    return MxCase(x, elems, scales, bias, k, scoring, renorm,
                  name=f"mxfp4/M{M}/H{H}/E{E}/k{k}/s{scoring}/b{int(with_bias)}/seed{seed}")


def _e4m3_magnitudes() -> np.ndarray:
    """The 127 non-negative finite OCP FP8 E4M3 magnitudes, indexed by code 0..126."""
    c = np.arange(127)
    ex, fr = c >> 3, (c & 7).astype(np.float64)
    return np.where(ex == 0, fr / 8.0 * 2.0 ** -6, (1.0 + fr / 8.0) * np.exp2(ex - 7.0))


E4M3_MAGNITUDES = _e4m3_magnitudes()


def quantise_mxfp8(w: np.ndarray):
    """Synthetic MXFP8 (E4M3) weights from real ones [E, H] (H % 32 == 0): per 32-block an
    E8M0 scale 2^(ceil(log2(amax / 448))) (the block's largest magnitude fits E4M3's 448),
    clamped to scale bytes 10..246, codes by nearest magnitude, sign in bit 7.  Returns
    (elems uint8 [E, H], scales uint8 [E, H/32]).  Input construction only."""
    E, H = w.shape
    assert H % 32 == 0
    blocks = w.astype(np.float64).reshape(E, H // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    ex = np.ceil(np.log2(np.maximum(amax, 1e-30) / 448.0)).astype(np.int64)
    ex = np.clip(ex, 10 - 127, 246 - 127)
    scaled = blocks / np.ldexp(1.0, ex)[:, :, None]
    code = np.abs(np.abs(scaled)[..., None] - E4M3_MAGNITUDES).argmin(axis=-1)
    code = code | np.where(scaled < 0, 0x80, 0)
    return code.reshape(E, H).astype(np.uint8), (ex + 127).astype(np.uint8)


def mxfp8_case(M: int, H: int = 4096, seed: int = 0, E: int = 256, k: int = 8,
               scoring: int = SOFTMAX, with_bias: bool = False, renorm: bool = True) -> MxCase:
    """Router on MXFP8 gate weights: X = unit-RMS N(0,1) rows in bf16, W ~ N(0,1/H)
    quantised to MXFP8 (quantise_mxfp8); optional U(-0.05,0.05) selection bias."""
    rng = _rng(seed, 13)
    x = rms_normalised_bf16(rng, M, H)
    w = rng.standard_normal((E, H)) / np.sqrt(H)
    elems, scales = quantise_mxfp8(w)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32) if with_bias else None
    return MxCase(x, elems, scales, bias, k, scoring, renorm,
                  name=f"mxfp8/M{M}/H{H}/E{E}/k{k}/s{scoring}/b{int(with_bias)}/seed{seed}")


def prefill_case(M: int = 8192, H: int = 7168, seed: int = 0, E: int = 256, k: int = 8) -> RouterCase:
    """Prefill router: softmax scores with U(-0.02,0.02) selection-only bias."""
    rng = _rng(seed, 6)
    x = gaussian_bf16(rng, (M, H), 1.0)
    w = gaussian_bf16(rng, (E, H), 1.0 / np.sqrt(H))
    bias = rng.uniform(-0.02, 0.02, E).astype(np.float32)
    return RouterCase(x, w, bias, k, SOFTMAX, True, name=f"prefill/M{M}/H{H}/seed{seed}")


def shape_case(M: int, H: int, E: int, k: int, scoring: int, with_bias: bool, renorm: bool,
               seed: int = 0) -> RouterCase:
    """Any shape within the limits: X ~ N(0,1), W ~ N(0,1/H) in bf16, and a
    U(-0.05,0.05) selection bias when asked for (edge-case and sweep tests)."""
    rng = _rng(seed, 8)
    x = gaussian_bf16(rng, (M, H), 1.0)
    w = gaussian_bf16(rng, (E, H), 1.0 / np.sqrt(H))
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32) if with_bias else None
    name = (f"shape/M{M}/H{H}/E{E}/k{k}/{'sm' if scoring == SOFTMAX else 'ssp'}"
            f"/{'bias' if with_bias else 'nobias'}/{'renorm' if renorm else 'raw'}/seed{seed}")
    return RouterCase(x, w, bias, k, scoring, renorm, name=name)


def metric_case(seed: int = 0) -> RouterCase:
    """Single-token decode at H=7168 (the latency headline shape)."""
    c = decode_case(1, H=7168, seed=seed)
    c.name = f"decode/M1/H7168/seed{seed}"
    return c


# --------------------------------------------------------------------------
# Logits workloads (adversarial rows for the standalone top-k)
# --------------------------------------------------------------------------
PLAIN, EXACT_TIE, ULP_CHAIN, ALL_EQUAL = 0, 1, 2, 3


def adversarial_logits(M: int, seed: int = 0, E: int = 256, k: int = 8,
                       std: float = float(np.sqrt(2.0))) -> LogitsCase:
    """fp32 logits ~ N(0, 2) with engineered rows around the k-th rank.

    25% of rows: 2-4 entries straddling rank k are set exactly equal.
    25% of rows: 2-4 entries straddling rank k form a chain 1 ulp apart,
                 assigned to the experts in random order (so the larger value
                 sometimes sits on the higher index).
    10% of rows: all entries equal.
    40% of rows: plain.
    Placing the group needs the row's rank order, found with np.argsort; that
    is input construction only (the expected output comes from the oracle).
    """
    rng = _rng(seed, 7)
    logits = (rng.standard_normal((M, E)) * std).astype(np.float32)
    u = rng.random(M)
    kind = np.where(u < 0.25, EXACT_TIE, np.where(u < 0.5, ULP_CHAIN,
                    np.where(u < 0.6, ALL_EQUAL, PLAIN))).astype(np.int8)
    for r in range(M):
        if kind[r] == ALL_EQUAL:
            logits[r, :] = np.float32(rng.standard_normal() * std)
            continue
        if kind[r] == PLAIN:
            continue
        order = np.argsort(-logits[r].astype(np.float64), kind="stable")
        g = int(rng.integers(2, 5))
        g = min(g, E)
        # group occupies ranks [s, s+g) with s <= k-1 < s+g-1, i.e. it straddles the cut
        s_lo = max(0, k - g + 1)
        s_hi = min(k - 1, E - g)
        if s_hi < s_lo:
            continue
        s = int(rng.integers(s_lo, s_hi + 1))
        members = order[s:s + g]
        top = np.float32(logits[r, members[0]])
        if kind[r] == EXACT_TIE:
            logits[r, members] = top
        else:
            chain = [top]
            for _ in range(g - 1):
                chain.append(np.nextafter(chain[-1], np.float32(-np.inf), dtype=np.float32))
            logits[r, rng.permutation(members)] = np.array(chain, dtype=np.float32)
    return LogitsCase(logits, None, k, SOFTMAX, True, kind, name=f"adv-logits/M{M}/seed{seed}")


# --------------------------------------------------------------------------
# Device-side pools for timing (same distributions, generated on the GPU so
# that half-gigabyte pools do not take seconds of host time)
# --------------------------------------------------------------------------
def torch_gaussian_bf16(shape, std: float, seed: int, device):
    """bf16 tensor ~ N(0, std^2) drawn on `device` with a seeded torch generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def torch_rms_normalised_bf16(shape, seed: int, device, eps: float = 1e-6):
    """Unit-RMS rows (last dim) of N(0,1) draws, rounded to bf16, on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x = x / torch.sqrt((x * x).mean(dim=-1, keepdim=True) + eps)
    return x.to(torch.bfloat16)


def torch_uniform_f32(n: int, lo: float, hi: float, seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.rand(n, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def torch_mxfp4_gate(n: int, E: int, H: int, seed: int, device, scale_lo: int = 117, scale_hi: int = 122):
    """n MXFP4 gate matrices on `device`: code bytes uniform over 0..255 (every
    E2M1 code equally likely in both nibbles) [n, E, H/2], and E8M0 scale bytes
    uniform over scale_lo..scale_hi [n, E, H/32] (the block scales that
    quantising N(0, 1/H) weights at H = 4096..7168 produces)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    codes = torch.randint(0, 256, (n, E, H // 2), generator=g, device=device, dtype=torch.uint8)
    scales = torch.randint(scale_lo, scale_hi + 1, (n, E, H // 32), generator=g, device=device,
                           dtype=torch.uint8)
    return codes, scales


# ---------------------------------------------------------------------------
# routed gather + shared-expert add inputs
# ---------------------------------------------------------------------------
GATHER_PATTERNS = ("typical", "same", "disjoint", "overlap", "within_dup", "all_dup", "all_local",
                   "all_remote", "some_remote", "ties")


@dataclasses.dataclass
class GatherCase:
    y: np.ndarray          # bf16 bits [R, D]: expert output rows
    slot_rows: np.ndarray  # int32 [M, k], -1 = no local row
    weights: np.ndarray    # fp32 [M, k]
    shared: np.ndarray     # bf16 bits [M, D]
    name: str = ""


def gather_case(M: int, k: int, D: int, pattern: str = "typical", seed: int = 0,
                R: Optional[int] = None) -> GatherCase:
    """Synthetic expert outputs for the gather: y ~ N(0,1) rows and shared ~ N(0,1)
    in bf16, router-like weights (U(0,1) per slot, scaled to sum to 1 per token,
    fp32), and a slot -> row map of the named route class (the B70 note's test
    classes: same / disjoint / cross-token overlap / within-token duplicate /
    all-duplicate / all-local / all-remote; "ties" uses small integer rows and
    dyadic weights so that many BF16 roundings are exact ties)."""
    assert pattern in GATHER_PATTERNS, pattern
    rng = _rng(seed, 12)
    R = M * k if R is None else R
    y = gaussian_bf16(rng, (R, D), 1.0)
    shared = gaussian_bf16(rng, (M, D), 1.0)
    u = rng.uniform(0.05, 1.0, (M, k))
    w = (u / u.sum(axis=1, keepdims=True)).astype(np.float32)
    if pattern == "typical":
        rows = np.stack([rng.choice(R, k, replace=False) for _ in range(M)])
    elif pattern == "same":
        rows = np.tile(rng.choice(R, k, replace=False), (M, 1))
    elif pattern == "disjoint":
        rows = (np.arange(M * k).reshape(M, k)) % R
    elif pattern == "overlap":
        base = rng.choice(R, k, replace=False)
        rows = np.stack([np.roll(base, t) if t % 2 else base for t in range(M)])
        rows[:, -1] = rng.integers(0, R, M)
    elif pattern == "within_dup":
        rows = np.stack([rng.choice(R, k, replace=False) for _ in range(M)])
        if k > 1:
            rows[:, 1] = rows[:, 0]
    elif pattern == "all_dup":
        rows = np.zeros((M, k), np.int64)
    elif pattern == "all_local":
        rows = np.stack([rng.permutation(R)[:k] for _ in range(M)])
    elif pattern == "all_remote":
        rows = np.full((M, k), -1)
    elif pattern == "some_remote":
        rows = np.stack([rng.choice(R, k, replace=False) for _ in range(M)])
        rows[rng.random((M, k)) < 0.4] = -1
    else:  # ties
        y = f32_to_bf16_bits(rng.integers(-8, 9, (R, D)).astype(np.float32))
        shared = f32_to_bf16_bits((rng.integers(-16, 17, (M, D)) * 0.5).astype(np.float32))
        w = rng.choice(np.array([0.25, 0.5, 0.75, 1.0, 1.5, -0.5], np.float32), (M, k))
        rows = np.stack([rng.choice(R, k, replace=R < k) for _ in range(M)])
    return GatherCase(y, rows.astype(np.int32), w.astype(np.float32), shared,
                      name=f"gather/{pattern}/M{M}/k{k}/D{D}/R{R}/seed{seed}")


def torch_mxfp8_gate(n: int, E: int, H: int, seed: int, device, scale_lo: int = 116, scale_hi: int = 121):
    """n MXFP8 gate matrices on `device`: E4M3 code bytes uniform over the finite codes
    [n, E, H] and E8M0 scale bytes uniform over scale_lo..scale_hi [n, E, H/32]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    codes = torch.randint(0, 256, (n, E, H), generator=g, device=device, dtype=torch.uint8)
    codes = torch.where((codes & 0x7F) == 0x7F, codes ^ 0x01, codes)  # NaN patterns -> +-1.75*2^8
    scales = torch.randint(scale_lo, scale_hi + 1, (n, E, H // 32), generator=g, device=device,
                           dtype=torch.uint8)
    return codes, scales
