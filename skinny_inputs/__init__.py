"""Seeded synthetic inputs for the skinny BF16 decode projection.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It only draws numbers and packs them as BF16 bit patterns; it holds
none of the projection's arithmetic (no products, no sums, no output rounding).

Workloads follow the decode projections the pages describe: the packed
Q/K/V/G/F_A/beta weight [6288, 7168] and the F_B weight [1536, 128] of the TP8
KDA projection ("Kimi-K3 low_latency_gemm", ``run_kda_projection_overlap``
parameters), plus the square-ish [3584, 7168] shape that page names as the one
re-measured on SM107, a tiny [256, 512] case and a long-K [7168, 18432] case.
No trained weights are used; values are drawn from the stated distributions.

Seeds: ``1_000_000 * config + 1000 * role + index`` with role 1 for weight copy
``index`` and role 2 for the activation block (index 0).  Draws use NumPy's
PCG64 (``np.random.default_rng``): normal draws are ``standard_normal`` in
float32 times sigma, uniform draws are ``random`` in float32 mapped to [-1, 1).
Float32 values become BF16 by round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

ROLE_WEIGHT = 1
ROLE_X = 2


@dataclass(frozen=True)
class Workload:
    """One decode projection workload: weight [n, k], activations [<=64, k]."""

    cid: int
    name: str
    n: int
    k: int
    copies: int              # distinct weight copies rotated per call
    m_values: tuple          # token counts that are timed
    x_rows: int              # rows of the activation block (prefixes give each M)
    w_dist: tuple            # ("normal", sigma) or ("uniform",)
    x_dist: tuple
    out_dtypes: tuple        # "bf16" and/or "f32"

    @property
    def weight_bytes(self) -> int:
        return 2 * self.n * self.k


WORKLOADS = {
    1: Workload(1, "tiny_256x512", 256, 512, 1, (1,), 1,
                ("uniform",), ("uniform",), ("f32",)),
    2: Workload(2, "square_3584x7168", 3584, 7168, 8, (1, 2, 4, 8, 16, 32), 64,
                ("normal", 0.02), ("normal", 1.0), ("bf16",)),
    3: Workload(3, "packed_qkvg_6288x7168", 6288, 7168, 4, (1, 2, 4, 8, 16, 32), 64,
                ("normal", 0.02), ("normal", 1.0), ("bf16",)),
    4: Workload(4, "short_k_1536x128", 1536, 128, 1, (1, 2, 4, 8, 16, 32, 64), 64,
                ("normal", 0.1), ("normal", 1.0), ("f32", "bf16")),
    5: Workload(5, "long_k_7168x18432", 7168, 18432, 2, (4, 8, 16, 32, 64), 64,
                ("normal", 0.01), ("normal", 1.0), ("bf16",)),
}


def seed_for(cid: int, role: int, index: int) -> int:
    return 1_000_000 * cid + 1000 * role + index


def f32_to_bf16_bits(a) -> np.ndarray:
    """Pack float32 values as BF16 bit patterns, rounding to nearest even.

    Inputs are finite here; NaN handling is not needed for generation.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(a) -> np.ndarray:
    """Pack float32 values as FP16 bit patterns (NumPy's nearest-even cast)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b) -> np.ndarray:
    """Widen FP16 bit patterns to float32 (exact)."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def draw(seed: int, shape, dist, dtype: str = "bf16") -> np.ndarray:
    """Draw float32 values of the given distribution and return BF16 (or,
    dtype "f16", FP16) bits."""
    rng = np.random.default_rng(seed)
    if dist[0] == "normal":
        v = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(dist[1])
    elif dist[0] == "uniform":
        v = rng.random(size=shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return f32_to_f16_bits(v) if dtype == "f16" else f32_to_bf16_bits(v)


def weight(cid: int, copy: int = 0) -> np.ndarray:
    """BF16 bits of weight copy ``copy`` of workload ``cid``: uint16 [n, k]."""
    w = WORKLOADS[cid]
    return draw(seed_for(cid, ROLE_WEIGHT, copy), (w.n, w.k), w.w_dist)


def activations(cid: int) -> np.ndarray:
    """BF16 bits of the activation block of workload ``cid``: uint16 [rows, k].

    The input for M tokens is the first M rows, so outputs at different M are
    prefixes of one another.
    """
    w = WORKLOADS[cid]
    return draw(seed_for(cid, ROLE_X, 0), (w.x_rows, w.k), w.x_dist)


def random_case(seed: int, m: int, n: int, k: int, w_sigma: float = 0.05,
                x_sigma: float = 1.0, dtype: str = "bf16"):
    """A generic normal (x, W) pair of BF16 (or FP16) bits for parity sweeps."""
    x = draw(seed * 2 + 1, (m, k), ("normal", x_sigma), dtype)
    wt = draw(seed * 2 + 2, (n, k), ("normal", w_sigma), dtype)
    return x, wt


def residual_case(seed: int, m: int, n: int, out: str = "bf16", sigma: float = 1.0):
    """A normal residual [m, n]: BF16 bits (out "bf16") or float32 values."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(size=(m, n), dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(v) if out == "bf16" else v


# ----------------------------------------------------------------------------
# Structured probes.  Each only builds inputs; expected outputs come from the
# oracle (and the tests' own closed forms), never from here.
# ----------------------------------------------------------------------------

def small_int_case(seed: int, m: int, n: int, k: int, lo: int = -3, hi: int = 3, dtype: str = "bf16"):
    """Integer-valued BF16 (or FP16) inputs in [lo, hi] (exact in both)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=(m, k)).astype(np.float32)
    wt = rng.integers(lo, hi + 1, size=(n, k)).astype(np.float32)
    if dtype == "f16":
        return f32_to_f16_bits(x), f32_to_f16_bits(wt)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(wt)


def _int_bits_table(values, dtype: str = "bf16") -> np.ndarray:
    v = np.asarray(values, dtype=np.float32)
    return f32_to_f16_bits(v) if dtype == "f16" else f32_to_bf16_bits(v)


def int_block_rows(k: int, block_elems: int = 1 << 27) -> int:
    """Rows per independently seeded block of int_weight_blocks (about
    block_elems elements per block, 128 Mi by default)."""
    return max(1, block_elems // k)


def int_weight_blocks(seed: int, n: int, k: int, values=(-3, -2, -1, 0, 1, 2, 3), block_elems: int = 1 << 27):
    """Yield (row0, bits) for the row blocks of an [n, k] BF16 weight whose
    entries are drawn uniformly from the small integers `values` (exact in
    BF16).  Block b (rows b * int_block_rows(k, block_elems) on) has its own generator
    seeded (seed, b), so a weight of billions of elements is built block by
    block and any block can be drawn again alone (int_weight_rows)."""
    table = _int_bits_table(values)
    per = int_block_rows(k, block_elems)
    for b, row0 in enumerate(range(0, n, per)):
        rows = min(per, n - row0)
        rng = np.random.default_rng([seed, b])
        idx = rng.integers(0, len(values), size=(rows, k), dtype=np.uint8)
        yield row0, table[idx]


def int_weight_rows(seed: int, n: int, k: int, rows, values=(-3, -2, -1, 0, 1, 2, 3),
                    block_elems: int = 1 << 27) -> np.ndarray:
    """Rows `rows` (any order) of the weight int_weight_blocks(seed, n, k,
    values, block_elems) yields, drawn again from their blocks only: uint16
    [len(rows), k]."""
    rows = np.asarray(rows, dtype=np.int64)
    per = int_block_rows(k, block_elems)
    table = _int_bits_table(values)
    out = np.empty((rows.shape[0], k), dtype=np.uint16)
    for b in np.unique(rows // per):
        row0 = int(b) * per
        nrows = min(per, n - row0)
        rng = np.random.default_rng([seed, int(b)])
        block = table[rng.integers(0, len(values), size=(nrows, k), dtype=np.uint8)]
        sel = np.nonzero(rows // per == b)[0]
        out[sel] = block[rows[sel] - row0]
    return out


def int_matrix(seed: int, m: int, k: int, values=(-3, -2, -1, 0, 1, 2, 3)) -> np.ndarray:
    """An [m, k] BF16 matrix of entries drawn uniformly from `values`."""
    rng = np.random.default_rng(seed)
    return _int_bits_table(values)[rng.integers(0, len(values), size=(m, k), dtype=np.uint8)]


def tie_case(n: int, k: int, m: int = 1):
    """Inputs whose exact dot products are odd integers above 256.

    Row n of W holds ones on its first ``257 + 2 * (n % 64)`` positions
    (requires k >= 383), x is all ones, so out[m][n] = 257 + 2 * (n % 64):
    every value lies halfway between two BF16 neighbours (spacing 2 there).
    """
    if k < 257 + 2 * 63:
        raise ValueError("tie probe needs k >= 383")
    wt = np.zeros((n, k), dtype=np.float32)
    for r in range(n):
        wt[r, : 257 + 2 * (r % 64)] = 1.0
    x = np.ones((m, k), dtype=np.float32)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(wt)


def k_probe_case(seed: int, m: int, n: int, k: int):
    """W row r has one nonzero, at column f(r); x is random normal.

    The first rows hit both ends and the middle of the K range; after them
    f(r) = 9973 * r mod k.  9973 is odd, so when k is a multiple of 512 any
    512 consecutive rows cover every residue of k modulo 8, 64 and 512, and
    every split and wave boundary is hit by some row.
    Returns (x_bits, w_bits, cols, scales).
    """
    rng = np.random.default_rng(seed)
    cols = np.empty(n, dtype=np.int64)
    edge = [0, k - 1, k // 2, k // 2 - 1, 7, 8, 63, 64, 511 % k, 512 % k]
    for r in range(n):
        cols[r] = edge[r] % k if r < len(edge) else (r * 9973) % k
    scales = np.float32(2.0) ** rng.integers(-3, 4, size=n).astype(np.float32)
    wt = np.zeros((n, k), dtype=np.float32)
    wt[np.arange(n), cols] = scales
    x = rng.standard_normal(size=(m, k), dtype=np.float32)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(wt), cols, scales


def fingerprint(bits: np.ndarray) -> str:
    """SHA-256 of the little-endian BF16 bits, for determinism checks."""
    return hashlib.sha256(np.ascontiguousarray(bits, dtype="<u2").tobytes()).hexdigest()
