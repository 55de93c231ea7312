"""CPU oracle for the skinny BF16 decode projection -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP library and never
imports it.

``gemm(x_bits, w_bits)`` returns ``(O, S)`` in float64, where
``O = x @ W^T`` (``out[M, N] = x[M, K] @ weight[N, K]^T``: class
PreparedWarpSplitK on the page
"vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.warp_splitk") and
``S = |x| @ |W|^T`` elementwise over the products, the scale of the parity
bound.  The arithmetic is in ``oracle.c`` (plain loops, OpenMP over rows of W).

The checker (``check``) applies the stated bound:
  fp32 output:  |g - O| <= 1e-3 * S + 1e-6
  BF16 output:  the same plus 2^-8 * |O| (one BF16 rounding of the result).

``dtype="f16"`` reads x and W as FP16 instead of BF16 (the two weight types
of class PreparedProjection on the page
"vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.projection").
``gemm_residual`` is ``O + R`` for a residual R given as values: the
``residual`` of try_low_latency_gemm on the page
"vllm.models.kimi_k3.nvidia.low_latency_gemm", read as an addend of the
product.  With a residual the checker also allows the one fp32 rounding of
the addition (2^-23 * |O + R|).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int)


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str = _LIB) -> ctypes.CDLL:
    """Load a built oracle library (building it if it is missing)."""
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    lib.oracle_gemm.argtypes = [_u16p, _u16p, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, _f64p, _f64p]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_t.argtypes = [_u16p, _u16p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, _f64p, _f64p]
    lib.oracle_gemm_t.restype = ctypes.c_int
    lib.oracle_gemm_sampled_t.argtypes = [_u16p, _u16p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, _i32p, _i32p, ctypes.c_long,
                                          _f64p, _f64p]
    lib.oracle_gemm_sampled_t.restype = ctypes.c_int
    lib.oracle_decode_f16.argtypes = [_u16p, ctypes.c_long, _f64p]
    lib.oracle_decode_f16.restype = None
    lib.oracle_gemm_sampled.argtypes = [_u16p, _u16p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, _i32p, _i32p, ctypes.c_long,
                                        _f64p, _f64p]
    lib.oracle_gemm_sampled.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [_f64p, ctypes.c_long, _u16p]
    lib.oracle_round_bf16.restype = None
    lib.oracle_decode_bf16.argtypes = [_u16p, ctypes.c_long, _f64p]
    lib.oracle_decode_bf16.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    return lib


_lib = None


def _get():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def _u16(a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a, a.ctypes.data_as(_u16p)


def _f16_flag(dtype: str) -> int:
    if dtype not in ("bf16", "f16"):
        raise ValueError(dtype)
    return int(dtype == "f16")


def gemm(x_bits, w_bits, lib=None, dtype: str = "bf16"):
    """(O, S) = (x @ W^T, |x| @ |W|^T products summed) in float64.

    x_bits: uint16 [M, K] bits; w_bits: uint16 [N, K] bits, BF16 or (dtype
    "f16") FP16.
    """
    lib = lib or _get()
    x, xp = _u16(x_bits)
    w, wp = _u16(w_bits)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"shape mismatch: x {x.shape}, W {w.shape}")
    m, k = x.shape
    n = w.shape[0]
    o = np.zeros((m, n), dtype=np.float64)
    s = np.zeros((m, n), dtype=np.float64)
    rc = lib.oracle_gemm_t(xp, wp, m, n, k, _f16_flag(dtype), o.ctypes.data_as(_f64p),
                           s.ctypes.data_as(_f64p))
    if rc != 0:
        raise RuntimeError("oracle_gemm failed")
    return o, s


def gemm_residual(x_bits, w_bits, r, lib=None, dtype: str = "bf16"):
    """(O + R, S): the product plus a residual R [M, N] given as values."""
    o, s = gemm(x_bits, w_bits, lib=lib, dtype=dtype)
    r = np.asarray(r, dtype=np.float64)
    if r.shape != o.shape:
        raise ValueError(f"residual {r.shape} vs product {o.shape}")
    return o + r, s


def gemm_sampled(x_bits, w_bits, mi, ni, lib=None, dtype: str = "bf16"):
    """Elements (mi[i], ni[i]) of (O, S), for checks at sizes too big to do whole."""
    lib = lib or _get()
    x, xp = _u16(x_bits)
    w, wp = _u16(w_bits)
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("K mismatch")
    mi = np.ascontiguousarray(mi, dtype=np.int32)
    ni = np.ascontiguousarray(ni, dtype=np.int32)
    o = np.zeros(mi.shape[0], dtype=np.float64)
    s = np.zeros(mi.shape[0], dtype=np.float64)
    rc = lib.oracle_gemm_sampled_t(xp, wp, m, n, k, _f16_flag(dtype), mi.ctypes.data_as(_i32p),
                                   ni.ctypes.data_as(_i32p), mi.shape[0],
                                   o.ctypes.data_as(_f64p), s.ctypes.data_as(_f64p))
    if rc != 0:
        raise RuntimeError("oracle_gemm_sampled failed (index out of range?)")
    return o, s


def round_bf16(values, lib=None) -> np.ndarray:
    """Round float64 values to BF16 bits, nearest-even, in one step."""
    lib = lib or _get()
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    lib.oracle_round_bf16(v.ctypes.data_as(_f64p), v.size, out.ctypes.data_as(_u16p))
    return out


def decode_bf16(bits, lib=None) -> np.ndarray:
    """BF16 bits to float64 (exact)."""
    lib = lib or _get()
    b, bp = _u16(bits)
    out = np.zeros(b.shape, dtype=np.float64)
    lib.oracle_decode_bf16(bp, b.size, out.ctypes.data_as(_f64p))
    return out


def decode_f16(bits, lib=None) -> np.ndarray:
    """FP16 bits to float64 (exact)."""
    lib = lib or _get()
    b, bp = _u16(bits)
    out = np.zeros(b.shape, dtype=np.float64)
    lib.oracle_decode_f16(bp, b.size, out.ctypes.data_as(_f64p))
    return out


def threads(lib=None) -> int:
    return (lib or _get()).oracle_threads()


def set_threads(n: int, lib=None) -> None:
    """Threads the oracle's later calls use (timing only; results do not depend on it)."""
    (lib or _get()).oracle_set_threads(int(n))


# ----------------------------------------------------------------------------
# Checker
# ----------------------------------------------------------------------------

REL = 1e-3
ABS = 1e-6
BF16_REL = 2.0 ** -8
F32_ADD_REL = 2.0 ** -23


@dataclass
class Report:
    ok: bool
    worst_ratio: float        # max |g - O| / bound
    worst_rel_s: float        # max |g - O| / S  (diagnostic)
    n_bad: int
    first_bad: tuple | None
    nan: int

    def __str__(self):
        return (f"ok={self.ok} worst err/bound={self.worst_ratio:.3e} "
                f"worst err/S={self.worst_rel_s:.3e} bad={self.n_bad} "
                f"nan={self.nan} first_bad={self.first_bad}")


def bound(o, s, mode: str, residual: bool = False):
    """The allowed |g - O| per element for output mode "f32" or "bf16"
    (O including the residual when there is one)."""
    b = REL * np.asarray(s, dtype=np.float64) + ABS
    if residual:
        b = b + F32_ADD_REL * np.abs(np.asarray(o, dtype=np.float64))
    if mode == "bf16":
        b = b + BF16_REL * np.abs(np.asarray(o, dtype=np.float64))
    elif mode != "f32":
        raise ValueError(mode)
    return b


def check(g, o, s, mode: str, residual: bool = False) -> Report:
    """Compare a result g (float values, already decoded) with the oracle."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    if g.shape != o.shape:
        raise ValueError(f"shape {g.shape} vs oracle {o.shape}")
    err = np.abs(g - o)
    b = bound(o, s, mode, residual)
    nan = int(np.count_nonzero(~np.isfinite(g)))
    bad = ~(err <= b)
    n_bad = int(np.count_nonzero(bad))
    first = None
    if n_bad:
        idx = np.argwhere(bad)[0]
        first = (tuple(int(i) for i in idx), float(g[tuple(idx)]), float(o[tuple(idx)]))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = float(np.nanmax(err / b)) if err.size else 0.0
        rel_s = float(np.nanmax(np.where(s > 0, err / s, 0.0))) if err.size else 0.0
    return Report(ok=(n_bad == 0 and nan == 0), worst_ratio=ratio, worst_rel_s=rel_s,
                  n_bad=n_bad, first_bad=first, nan=nan)
