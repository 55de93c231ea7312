"""Pins that tie the CPU oracle to facts other than itself.

Each pin takes a loaded oracle library, so the same pins also run against
deliberately broken copies of the oracle (tests/test_oracle.py) to show that a
plausible mistake -- a dropped term, a wrong sign or index, a transposed
operand, a wrong rounding rule -- makes at least one of them fail.

The quantity pinned is out[M, N] = x[M, K] @ weight[N, K]^T (class
PreparedWarpSplitK, page "vllm.models.kimi_k3.nvidia.specialized_decode.
cutedsl.gemm.warp_splitk"), plus S = sum_k |x_k * W_nk|, the scale of the
parity bound.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

import oracle
import skinny_inputs as si


def _bits_of_ints(a):
    return si.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def pin_bruteforce_integers(lib):
    """Exact equality with Python integer arithmetic on every shape 1..4."""
    rng = np.random.default_rng(7)
    for m, n, k in itertools.product(range(1, 5), repeat=3):
        xi = rng.integers(-8, 9, size=(m, k))
        wi = rng.integers(-8, 9, size=(n, k))
        o, s = oracle.gemm(_bits_of_ints(xi), _bits_of_ints(wi), lib=lib)
        for a in range(m):
            for b in range(n):
                want = sum(int(xi[a, c]) * int(wi[b, c]) for c in range(k))
                want_s = sum(abs(int(xi[a, c]) * int(wi[b, c])) for c in range(k))
                assert o[a, b] == want, (m, n, k, a, b, o[a, b], want)
                assert s[a, b] == want_s, (m, n, k, a, b, s[a, b], want_s)


def pin_onehot(lib):
    """W[n][k] = 2^e_n [k == pi(n)] gives O[m][n] = 2^e_n x[m][pi(n)] exactly."""
    rng = np.random.default_rng(11)
    for m, n, k in ((3, 5, 7), (2, 9, 16), (5, 16, 40), (1, 3, 3)):
        pi = rng.permutation(k)[:n]
        e = rng.integers(-4, 5, size=n)
        w = np.zeros((n, k), dtype=np.float32)
        w[np.arange(n), pi] = np.ldexp(1.0, e)
        x = si.draw(100 + m * n * k, (m, k), ("normal", 1.0))
        o, _ = oracle.gemm(x, si.f32_to_bf16_bits(w), lib=lib)
        xf = si.bf16_bits_to_f32(x).astype(np.float64)
        want = xf[:, pi] * np.ldexp(1.0, e)[None, :]
        assert np.array_equal(o, want), (m, n, k)


def pin_linearity(lib):
    """O is additive over disjoint K supports and scales by powers of two."""
    rng = np.random.default_rng(13)
    m, n, k = 4, 24, 96
    x = si.draw(201, (m, k), ("normal", 1.0))
    w = si.draw(202, (n, k), ("normal", 0.1))
    mask = rng.random(k) < 0.5
    x1 = np.where(mask[None, :], x, np.uint16(0))
    x2 = np.where(mask[None, :], np.uint16(0), x)
    o, s = oracle.gemm(x, w, lib=lib)
    o1, _ = oracle.gemm(x1, w, lib=lib)
    o2, _ = oracle.gemm(x2, w, lib=lib)
    assert np.all(np.abs(o - (o1 + o2)) <= 1e-12 * s + 1e-300)
    # 2^j x: BF16 exponent shift, exact
    for j in (-3, 1, 5):
        xs = si.f32_to_bf16_bits(si.bf16_bits_to_f32(x) * np.float32(2.0 ** j))
        oj, sj = oracle.gemm(xs, w, lib=lib)
        assert np.array_equal(oj, o * 2.0 ** j)
        assert np.array_equal(sj, s * 2.0 ** j)
    # O is also linear in W's rows: negating W negates O, leaves S
    wn = w ^ np.uint16(0x8000)
    on, sn = oracle.gemm(x, wn, lib=lib)
    assert np.array_equal(on, -o) and np.array_equal(sn, s)


def pin_numpy(lib, cids=(1, 4)):
    """Agreement with NumPy float64 matmul (an independent code path)."""
    for cid in cids:
        w = si.weight(cid)
        x = si.activations(cid)
        o, s = oracle.gemm(x, w, lib=lib)
        x64 = si.bf16_bits_to_f32(x).astype(np.float64)
        w64 = si.bf16_bits_to_f32(w).astype(np.float64)
        ref = x64 @ w64.T
        ref_s = np.abs(x64) @ np.abs(w64).T
        assert np.all(np.abs(o - ref) <= 1e-12 * ref_s), cid
        assert np.all(np.abs(s - ref_s) <= 1e-12 * ref_s), cid


def pin_sampled_matches_full(lib):
    """The sampled entry point returns the full product's elements exactly."""
    x, w = si.random_case(5, 7, 33, 120)
    o, s = oracle.gemm(x, w, lib=lib)
    rng = np.random.default_rng(3)
    mi = rng.integers(0, 7, size=50)
    ni = rng.integers(0, 33, size=50)
    os_, ss = oracle.gemm_sampled(x, w, mi, ni, lib=lib)
    assert np.array_equal(os_, o[mi, ni]) and np.array_equal(ss, s[mi, ni])


def _bf16_value(bits: int) -> Fraction:
    """Exact value of a finite BF16 bit pattern, from the format's definition."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0:
        mag = Fraction(frac, 128) * Fraction(2) ** -126
    else:
        mag = (1 + Fraction(frac, 128)) * Fraction(2) ** (exp - 127)
    return sign * mag


def _rne_bruteforce(v: float) -> int:
    """Nearest BF16 by exact comparison with both neighbours, ties to even."""
    target = Fraction(v)
    if v == 0:
        return 0x8000 if np.signbit(v) else 0
    sign = 0x8000 if v < 0 else 0
    mag = abs(target)
    # bisect over the ordered positive finite patterns 0x0000..0x7F7F
    lo, hi = 0, 0x7F7F
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if _bf16_value(mid) <= mag:
            lo = mid
        else:
            hi = mid
    a, b = _bf16_value(lo), _bf16_value(hi)
    if mag >= b:
        return sign | hi
    da, db = mag - a, b - mag
    if da < db or (da == db and lo % 2 == 0):
        return sign | lo
    return sign | hi


def pin_round_bf16(lib):
    """One-step nearest-even rounding to BF16 against an exact brute force."""
    fixed = {1.0: 0x3F80, -2.0: 0xC000, 257.0: 0x4380, 259.0: 0x4382,
             261.0: 0x4382, 263.0: 0x4384, 0.0: 0x0000, 2.0 ** -133: 0x0001,
             3 * 2.0 ** -134: 0x0002, 1.0 + 2.0 ** -8: 0x3F80,
             1.0 + 3 * 2.0 ** -8: 0x3F82}
    got = oracle.round_bf16(np.array(list(fixed)), lib=lib)
    for (v, want), g in zip(fixed.items(), got):
        assert int(g) == want, (v, hex(int(g)), hex(want))
    rng = np.random.default_rng(17)
    vals = np.concatenate([
        rng.standard_normal(300) * np.exp2(rng.integers(-30, 30, 300)),
        (rng.integers(-2000, 2000, 100) + 0.5) * 2.0 ** -7,   # exact ties near 1..16
        rng.standard_normal(50) * 2.0 ** -128,                # subnormal range
    ])
    got = oracle.round_bf16(vals, lib=lib)
    for v, g in zip(vals, got):
        assert int(g) == _rne_bruteforce(float(v)), (v, hex(int(g)))


def pin_decode(lib):
    """BF16 widening against the format's definition."""
    pats = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x4380, 0x3E4D],
                    dtype=np.uint16)
    got = oracle.decode_bf16(pats, lib=lib)
    for p, g in zip(pats, got):
        assert Fraction(float(g)) == _bf16_value(int(p)), hex(int(p))


def pin_decode_f16(lib):
    """FP16 widening against NumPy's own float16 on every bit pattern, and
    against the format's definition on a few."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_f16(pats, lib=lib)
    ref = pats.view(np.float16).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), hex(int(pats[~same][0]))
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))
    for p, want in ((0x3C00, 1.0), (0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24), (0x0400, 2.0 ** -14),
                    (0x7BFF, 65504.0), (0xC500, -5.0)):
        assert oracle.decode_f16(np.array([p], dtype=np.uint16), lib=lib)[0] == want, hex(p)


def pin_f16_products(lib):
    """FP16 inputs: exact against Python integers on small shapes, and within
    1e-12 S of NumPy float64 on a random case."""
    rng = np.random.default_rng(23)
    for m, n, k in ((1, 1, 1), (2, 3, 4), (3, 5, 17), (4, 2, 33)):
        xi = rng.integers(-8, 9, size=(m, k))
        wi = rng.integers(-8, 9, size=(n, k))
        o, s = oracle.gemm(si.f32_to_f16_bits(xi), si.f32_to_f16_bits(wi), lib=lib, dtype="f16")
        want = xi @ wi.T
        assert np.array_equal(o, want.astype(np.float64)), (m, n, k)
        assert np.array_equal(s, (np.abs(xi) @ np.abs(wi).T).astype(np.float64)), (m, n, k)
    x, w = si.random_case(29, 5, 40, 300, dtype="f16")
    o, s = oracle.gemm(x, w, lib=lib, dtype="f16")
    ref = x.view(np.float16).astype(np.float64) @ w.view(np.float16).astype(np.float64).T
    assert np.all(np.abs(o - ref) <= 1e-12 * s)
    mi, ni = np.array([0, 4, 2]), np.array([39, 0, 17])
    os_, ss = oracle.gemm_sampled(x, w, mi, ni, lib=lib, dtype="f16")
    assert np.array_equal(os_, o[mi, ni]) and np.array_equal(ss, s[mi, ni])


def pin_residual(lib):
    """O + R: exact against Python integers, and R = 0 gives the product."""
    rng = np.random.default_rng(31)
    m, n, k = 3, 7, 20
    xi = rng.integers(-5, 6, size=(m, k))
    wi = rng.integers(-5, 6, size=(n, k))
    ri = rng.integers(-100, 101, size=(m, n))
    o, s = oracle.gemm_residual(_bits_of_ints(xi), _bits_of_ints(wi), ri.astype(np.float64), lib=lib)
    assert np.array_equal(o, (xi @ wi.T + ri).astype(np.float64))
    o0, s0 = oracle.gemm(_bits_of_ints(xi), _bits_of_ints(wi), lib=lib)
    oz, sz = oracle.gemm_residual(_bits_of_ints(xi), _bits_of_ints(wi), np.zeros((m, n)), lib=lib)
    assert np.array_equal(oz, o0) and np.array_equal(sz, s0) and np.array_equal(s, s0)


ALL_PINS = (pin_bruteforce_integers, pin_onehot, pin_linearity, pin_numpy,
            pin_sampled_matches_full, pin_round_bf16, pin_decode, pin_decode_f16,
            pin_f16_products, pin_residual)


def run_all(lib):
    """Return the names of the pins that fail for this library."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    return failed
