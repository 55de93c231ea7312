"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Exact probes first -- integer inputs make every fp32 partial sum exact, so any
correct kernel, in any summation order, must reproduce the oracle bit for bit
(and the nearest-even BF16 rounding of it) -- then the seeded workloads under
the stated bound |g - O| <= 1e-3 S + 1e-6 (+ 2^-8 |O| for BF16 output).
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np
import pytest

import oracle
import skinny_inputs as si
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import skinny_bf16_decode_amd as sk
    sk.load_library()
    return sk


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_exact(sk, plan, x_bits, o, m, label):
    """Run plan on the first m rows, compare bitwise with the exact result."""
    import torch
    x = gu.dev_bf16(x_bits[:m])
    out = gu.out_buffer(plan.n, plan.out_dtype)
    plan.run(x, out[:m])   # rows [0, m) of a packed [64, N] buffer are a packed [m, N] view
    torch.cuda.synchronize()
    assert gu.sentinel_intact(out, m), f"{label}: rows >= M were written"
    got = gu.host_bits(out)[:m]
    if plan.out_dtype == torch.float32:
        want = o[:m].astype(np.float32).view(np.uint32)
    else:
        want = oracle.round_bf16(o[:m])
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)[0]
        raise AssertionError(f"{label}: first mismatch at {tuple(bad)}: got {got[tuple(bad)]:#x} "
                             f"want {want[tuple(bad)]:#x} (exact {o[tuple(bad)]})")


EXACT_SHAPES = [(200, 1032), (48, 4104), (64, 128)]


@pytest.mark.parametrize("shape", EXACT_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("od", ["f32", "bf16"])
def test_integer_probe_every_tactic(sk, shape, od):
    """Every candidate tactic, forced, is exact on integer inputs -- at its full
    token tile and at a ragged M below it.  Shapes have ragged row tiles and K
    not a multiple of the wave stride (K/8 = 129, 513, 16)."""
    import torch
    n, k = shape
    out_dtype = torch.float32 if od == "f32" else torch.bfloat16
    x_bits, w_bits = si.small_int_case(1000 + n + k, 64, n, k)
    o, _ = oracle.gemm(x_bits, w_bits)
    assert np.all(np.abs(o) < 2 ** 24)
    w = gu.dev_bf16(w_bits)
    tactics = sk.enumerate_tactics(n, k)
    _say(f"[exact] {n}x{k} {od}: {len(tactics)} tactics")
    for t in tactics:
        plan = sk.Prepared(w, out_dtype, table=gu.forced_table(t))
        for m in sorted({t.mt, max(1, t.mt - 3), max(1, t.mt // 2 + 1)}):
            _check_exact(sk, plan, x_bits, o, m, f"{t} M={m}")
        plan.close()


def test_random_shapes_random_tactics_exact(sk):
    """Seeded random shapes (N not a multiple of any tile, K = 8 j up to 4800),
    each with a tactic drawn from its own candidate list and a random M up to
    the tactic's tile, on integer inputs: fp32 out bit-identical to the oracle,
    BF16 out to its nearest-even rounding, rows >= M untouched.  Covers range
    and tile arithmetic at sizes the fixed probes do not."""
    import torch
    rng = np.random.default_rng(20261203)
    paths = set()
    for case in range(160):
        n = int(rng.integers(1, 3000))
        k = 8 * int(rng.integers(1, 601))
        tactics = sk.enumerate_tactics(n, k)
        t = tactics[int(rng.integers(0, len(tactics)))]
        m = int(rng.integers(1, t.mt + 1))
        od = torch.float32 if case % 2 else torch.bfloat16
        x_bits, w_bits = si.small_int_case(50_000 + case, 64, n, k)
        o, _ = oracle.gemm(x_bits[:m], w_bits)
        plan = sk.Prepared(gu.dev_bf16(w_bits), od, table=gu.forced_table(t))
        _check_exact(sk, plan, x_bits, o, m, f"case {case}: {n}x{k} M={m} {od} {t}")
        plan.close()
        paths.add(t.path)
    _say(f"[random shapes] paths {sorted(paths)}")
    assert len(paths) == 8                      # every path the enumeration offers


@pytest.mark.parametrize("shape", [(1, 8), (15, 8), (17, 24), (3, 128)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_degenerate_shapes_every_tactic(sk, shape):
    """The smallest shapes: one weight row, one 16-byte chunk per row (K = 8),
    fewer rows than any tile.  Every candidate tactic, forced, at its full
    tile and a ragged M, then the tuned plan at every M = 1..64, exact on
    integer inputs with rows >= M untouched."""
    import torch
    n, k = shape
    x_bits, w_bits = si.small_int_case(9100 + n * 1000 + k, 64, n, k)
    o, _ = oracle.gemm(x_bits, w_bits)
    w = gu.dev_bf16(w_bits)
    tactics = sk.enumerate_tactics(n, k)
    _say(f"[degenerate {n}x{k}] {len(tactics)} tactics")
    for i, t in enumerate(tactics):
        od = torch.float32 if i % 2 else torch.bfloat16
        plan = sk.Prepared(w, od, table=gu.forced_table(t))
        for m in sorted({t.mt, max(1, t.mt // 2 + 1)}):
            _check_exact(sk, plan, x_bits, o, m, f"{n}x{k} {t} M={m} {od}")
        plan.close()
    plan = sk.Prepared(w, torch.float32)
    for m in range(1, 65):
        _check_exact(sk, plan, x_bits, o, m, f"{n}x{k} tuned M={m}")
    plan.close()


def test_nan_and_inf_propagate_every_tactic(sk):
    """A NaN in one x row makes its whole output row NaN; a +Inf in another
    makes out[.][n] +Inf, -Inf or NaN as W[n] at that column is positive,
    negative or zero; the other rows stay exact -- for every candidate
    tactic at its own token tile (a 1- or 2-token tile runs once per special
    row), BF16 and fp32 out.  The K-split exchange stores values XOR a
    signalling-NaN pattern with zero meaning empty; NaN and Inf partials must
    pass through it like any other value."""
    import torch
    n, k = 72, 520
    x_bits, w_bits = si.small_int_case(9300, 66, n, k)
    x_bits = x_bits.copy()
    x_bits[0, 5] = 0x7FC0                        # NaN
    x_bits[1, 9] = 0x7F80                        # +Inf
    o, _ = oracle.gemm(x_bits[2:], w_bits)      # the other rows are finite
    wcol = si.bf16_bits_to_f32(w_bits[:, 9])
    want_inf = np.where(wcol > 0, np.inf, np.where(wcol < 0, -np.inf, np.nan))
    w = gu.dev_bf16(w_bits)
    x = gu.dev_bf16(x_bits)
    tactics = sk.enumerate_tactics(n, k)
    _say(f"[nan/inf] {len(tactics)} tactics, {sum(t.split > 1 for t in tactics)} with a K split")
    assert {t.path for t in tactics} >= {0, 1, 3, 8, 9, 10, 11, 12}
    assert any(t.split > 1 for t in tactics)

    def check(plan, od, first, m, label):
        out = gu.out_buffer(n, od)
        plan.run(x[first:first + m], out[:m])
        torch.cuda.synchronize()
        assert gu.sentinel_intact(out, m), f"{label}: rows >= M written"
        got = out[:m].float().cpu().numpy().astype(np.float64)
        bits = gu.host_bits(out)[:m]
        for r in range(m):
            src = first + r
            if src == 0:
                assert np.all(np.isnan(got[r])), f"{label}: NaN row"
            elif src == 1:
                assert np.array_equal(np.isnan(got[r]), np.isnan(want_inf)), f"{label}: Inf row NaN pattern"
                fin = ~np.isnan(want_inf)
                assert np.array_equal(got[r][fin], want_inf[fin]), f"{label}: Inf row signs"
            elif od == torch.float32:
                assert np.array_equal(got[r], o[src - 2]), f"{label}: finite row {src}"
            else:
                assert np.array_equal(bits[r], oracle.round_bf16(o[src - 2])), f"{label}: finite row {src}"

    for i, t in enumerate(tactics):
        od = torch.float32 if i % 2 else torch.bfloat16
        plan = sk.Prepared(w, od, table=gu.forced_table(t))
        check(plan, od, 0, t.mt, f"{t} {od}")
        if t.mt < 2:
            check(plan, od, 1, 1, f"{t} {od} (Inf row)")
        plan.close()


def test_k_probe_every_tactic(sk):
    """One nonzero per weight row, at a column that sweeps every residue
    modulo 8, 64 and 512: any chunk dropped or duplicated at a lane, wave or
    split boundary shows up as a wrong output."""
    import torch
    n, k = 600, 1536
    x_bits, w_bits, cols, scales = si.k_probe_case(5, 64, n, k)
    o, _ = oracle.gemm(x_bits, w_bits)
    want_cf = si.bf16_bits_to_f32(x_bits).astype(np.float64)[:, cols] * scales.astype(np.float64)
    assert np.array_equal(o, want_cf)
    w = gu.dev_bf16(w_bits)
    tactics = sk.enumerate_tactics(n, k)
    _say(f"[kprobe] {len(tactics)} tactics")
    for t in tactics:
        plan = sk.Prepared(w, torch.float32, table=gu.forced_table(t))
        _check_exact(sk, plan, x_bits, o, t.mt, f"{t}")
        plan.close()


@pytest.mark.parametrize("path", ["tuned", "dot2", "mfma"])
def test_tie_probe_rounds_to_nearest_even(sk, path):
    """Exact sums 257, 259, 261, ... lie halfway between BF16 neighbours;
    nearest-even gives 256, 260, 260, ..., truncation 256, 258, 260, ..."""
    import torch
    n, k = 128, 512
    x_bits, w_bits = si.tie_case(n, k, m=64)
    o, _ = oracle.gemm(x_bits, w_bits)
    w = gu.dev_bf16(w_bits)
    if path == "tuned":
        plan = sk.Prepared(w, torch.bfloat16)
    elif path == "dot2":
        plan = sk.Prepared(w, torch.bfloat16, table=gu.forced_table(sk.Tactic(0, 8, 4, 1, 1, 1)))
    else:
        plan = sk.Prepared(w, torch.bfloat16, table=[sk.Tactic(1, 64, 16, 2, 1, 2)] * 64)
    for m in (1, 5, 8, 16, 33, 64):
        _check_exact(sk, plan, x_bits, o, m, f"tie {path} M={m}")
    plan.close()


def _bound_check(got, o, s, mode, label):
    rep = oracle.check(got, o, s, mode)
    _say(f"  {label}: {rep}")
    assert rep.ok, f"{label}: {rep}"
    # Beyond the stated bound: an fp32 accumulator over these lengths sits far
    # inside it.  Allow 1e-4 S for accumulation, plus the output rounding
    # (half a BF16 ulp, <= 2^-8 |O|) in BF16 mode.
    tight = 1e-4 * np.asarray(s) + 1e-6
    if mode == "bf16":
        tight = tight + 2.0 ** -8 * np.abs(np.asarray(o))
    worst = float(np.max(np.abs(np.asarray(got) - np.asarray(o)) / tight)) if np.size(o) else 0.0
    assert worst <= 1.0, f"{label}: error level above the fp32-accumulation expectation ({worst:.3f})"


@pytest.mark.parametrize("cid", [1, 4])
def test_small_workloads_all_m(sk, cid):
    """Tuned plans on the tiny and short-K workloads, every M = 1..64 (the
    activation block is cycled for the tiny workload, which has one row)."""
    import torch
    wl = si.WORKLOADS[cid]
    w_bits = si.weight(cid)
    x_bits = si.activations(cid)
    if x_bits.shape[0] < 64:
        x_bits = np.ascontiguousarray(np.resize(x_bits, (64, wl.k)))
    o, s = oracle.gemm(x_bits, w_bits)
    w = gu.dev_bf16(w_bits)
    for od in wl.out_dtypes:
        out_dtype = torch.float32 if od == "f32" else torch.bfloat16
        plan = sk.Prepared(w, out_dtype)
        for m in range(1, 65):
            x = gu.dev_bf16(x_bits[:m])
            out = gu.out_buffer(wl.n, out_dtype)
            plan.run(x, out[:m])
            torch.cuda.synchronize()
            assert gu.sentinel_intact(out, m), (cid, od, m)
            _bound_check(gu.values(out)[:m], o[:m], s[:m], od, f"cfg{cid} {od} M={m} {plan.describe(m)}")
        plan.close()


@pytest.mark.parametrize("cid", [2, 3])
def test_decode_workloads(sk, cid):
    """The [3584, 7168] and [6288, 7168] workloads at full size, tuned, at the
    timed token counts and at ragged ones, against the whole oracle."""
    import torch
    wl = si.WORKLOADS[cid]
    w_bits = si.weight(cid)
    x_bits = si.activations(cid)
    t0 = time.time()
    o, s = oracle.gemm(x_bits, w_bits)
    _say(f"[cfg{cid}] oracle {time.time() - t0:.1f}s")
    w = gu.dev_bf16(w_bits)
    t0 = time.time()
    plan = sk.Prepared(w, torch.bfloat16)
    _say(f"[cfg{cid}] prepare {time.time() - t0:.2f}s")
    for m in sorted(set(wl.m_values) | {3, 7, 13, 31, 47, 64}):
        x = gu.dev_bf16(x_bits[:m])
        out = gu.out_buffer(wl.n, torch.bfloat16)
        plan.run(x, out[:m])
        torch.cuda.synchronize()
        assert gu.sentinel_intact(out, m), (cid, m)
        _bound_check(gu.values(out)[:m], o[:m], s[:m], "bf16", f"cfg{cid} M={m} {plan.describe(m)}")
    # a second prepare of the same shape reuses the tuned table
    t0 = time.time()
    plan2 = sk.Prepared(w, torch.bfloat16)
    dt = time.time() - t0
    _say(f"[cfg{cid}] second prepare {dt:.3f}s")
    assert all(plan.tactic(m) == plan2.tactic(m) for m in range(1, 65))
    plan.close()
    plan2.close()


def test_long_k_split_workload(sk):
    """[7168, 18432] at its timed token counts, tuned, and with a forced
    four-way cross-workgroup K split on the DOT2 and MFMA paths: the whole
    output against the oracle."""
    import torch
    cid = 5
    wl = si.WORKLOADS[cid]
    w_bits = si.weight(cid)
    x_bits = si.activations(cid)
    t0 = time.time()
    o, sv = oracle.gemm(x_bits, w_bits)
    _say(f"[cfg5] oracle {time.time() - t0:.1f}s")
    w = gu.dev_bf16(w_bits)
    plans = {"tuned": sk.Prepared(w, torch.bfloat16),
             "split4": sk.Prepared(w, torch.bfloat16, table=[
                 sk.Tactic(0, 8, 4, 4, 1, 4) if m <= 8 else sk.Tactic(1, 64, 16, 4, 2, 4)
                 for m in range(1, 65)])}
    for m in wl.m_values:
        for name, plan in plans.items():
            x = gu.dev_bf16(x_bits[:m])
            out = gu.out_buffer(wl.n, torch.bfloat16)
            plan.run(x, out[:m])
            torch.cuda.synchronize()
            assert gu.sentinel_intact(out, m)
            _bound_check(gu.values(out)[:m], o[:m], sv[:m], "bf16", f"cfg5 {name} M={m} {plan.describe(m)}")
    for p in plans.values():
        p.close()


def test_deterministic_and_graph_replay(sk):
    """Bitwise-identical results across repeated runs and across 100 replays
    of a captured graph (the split-K exchange nodes must be empty again after
    every call)."""
    import torch
    n, k = 1024, 4096
    x_bits, w_bits = si.random_case(77, 64, n, k)
    w = gu.dev_bf16(w_bits)
    table = [sk.Tactic(0, 8, 2, 2, 1, 4) if m <= 8 else sk.Tactic(1, 32, 16, 2, 1, 4)
             for m in range(1, 33)] + [sk.Tactic(1, 64, 16, 2, 1, 2)] * 32
    plan = sk.Prepared(w, torch.bfloat16, table=table)
    x = gu.dev_bf16(x_bits)
    ref = {}
    for m in (5, 24, 64):
        out = gu.out_buffer(n, torch.bfloat16)
        plan.run(x[:m], out[:m])
        torch.cuda.synchronize()
        ref[m] = gu.host_bits(out).copy()
        for _ in range(20):
            out2 = gu.out_buffer(n, torch.bfloat16)
            plan.run(x[:m], out2[:m])
            torch.cuda.synchronize()
            assert np.array_equal(gu.host_bits(out2), ref[m]), m
    o, s = oracle.gemm(x_bits, w_bits)
    for m in ref:
        _bound_check(si.bf16_bits_to_f32(ref[m][:m]).astype(np.float64), o[:m], s[:m], "bf16",
                     f"graph-ref M={m}")
    # graph capture of three calls on one stream
    outs = {m: gu.out_buffer(n, torch.bfloat16) for m in ref}
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for m in ref:
                plan.run(x[:m], outs[m][:m])
    for rep in range(100):
        for m in ref:
            outs[m][:m].fill_(0)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for m in ref:
            assert np.array_equal(gu.host_bits(outs[m]), ref[m]), (rep, m)
    plan.close()


# Kernels the tuner picks for the packed 6288x7168 decode weight, by token
# count: DOT2 at M = 1, DOT2 over equal row ranges at M = 2, the ranged MFMAX
# at 16 tokens and at 32 with a two-way K split; and the barrier-free MFMAW at
# 4, 8 (with a two-way K split), 32 and 64 tokens.
DECODE_KERNEL_SETS = {
    "dot2_mfmax": lambda sk: {1: sk.Tactic(0, 1, 2, 8, 1, 1), 2: sk.Tactic(sk.PATH_DOT2R, 2, 4, 1, 2, 1),
                              16: sk.Tactic(3, 16, 32, 2, 2, 1), 32: sk.Tactic(3, 32, 64, 4, 2, 2)},
    "mfmaw": lambda sk: {4: sk.Tactic(sk.PATH_MFMAW, 16, 32, 2, 2, 1), 8: sk.Tactic(sk.PATH_MFMAW, 16, 32, 2, 2, 2),
                         32: sk.Tactic(sk.PATH_MFMAW, 32, 32, 2, 2, 1), 64: sk.Tactic(sk.PATH_MFMAW, 64, 32, 4, 2, 1)},
}


def shipped_table(sk, n, k, od="bf16"):
    """The 64-entry table the benchmark loads for an [n, k] weight (BF16 in,
    `od` out, 256 CUs), from the file shipped with the package; the BF16-out
    table when none ships for `od`."""
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "skinny_bf16_decode_amd", "tables", "mi355x_tuned.txt")
    with open(path) as f:
        lines = [line.split() for line in f]
    for want in (od, "bf16"):
        for p in lines:
            if p[3:8] == ["256", str(n), str(k), "bf16", want]:
                return [sk.Tactic(*map(int, e.split("."))) for e in p[8:]]
    raise AssertionError(f"no shipped table for {n}x{k}")


# the weights with a shipped table, by workload id
SHIPPED = {2: (3584, 7168), 3: (6288, 7168), 4: (1536, 128), 5: (7168, 18432)}


@pytest.mark.parametrize("cid", sorted(SHIPPED))
def test_shipped_tables_exact_full_size(sk, cid):
    """The shipped table of each weight (the fp32-out table for fp32 out
    where one ships), forced, on integer inputs at the full shape (x, W in
    {-3..3}, so every partial sum is exact in fp32):
    every M = 1..64 -- each kernel the table uses, at each M it serves --
    bit for bit, fp32 out equal to the oracle and BF16 out to its nearest-even
    rounding."""
    import torch
    n, k = SHIPPED[cid]
    x_bits, w_bits = si.small_int_case(9000 + cid, 64, n, k)
    t0 = time.time()
    o, _ = oracle.gemm(x_bits, w_bits)
    _say(f"[shipped exact {n}x{k}] oracle {time.time() - t0:.1f}s")
    assert np.all(np.abs(o) < 2 ** 24)
    w = gu.dev_bf16(w_bits)
    for od in (torch.bfloat16, torch.float32):
        table = shipped_table(sk, n, k, "f32" if od == torch.float32 else "bf16")
        plan = sk.Prepared(w, od, table=table)
        for m in range(1, 65):
            _check_exact(sk, plan, x_bits, o, m, f"{n}x{k} {od} M={m} {table[m - 1]}")
        plan.close()


@pytest.mark.parametrize("cid", sorted(SHIPPED))
def test_shipped_tables_random_full_size(sk, cid):
    """The shipped table of each decode weight on its seeded workload at the
    full shape: the whole output within the stated bound at the benchmark's
    token counts and at ragged ones, bit-identical over repeats and over graph
    replays with eager work between them (the launch configuration
    bench.py times)."""
    import torch
    wl = si.WORKLOADS[cid]
    n, k = SHIPPED[cid]
    w_bits, x_bits = si.weight(cid, 0), si.activations(cid)
    t0 = time.time()
    o, sv = oracle.gemm(x_bits, w_bits)
    _say(f"[shipped random {n}x{k}] oracle {time.time() - t0:.1f}s")
    w, x = gu.dev_bf16(w_bits), gu.dev_bf16(x_bits)
    plan = sk.Prepared(w, torch.bfloat16, table=shipped_table(sk, n, k))
    ms = sorted(set(wl.m_values) | {3, 7, 13, 31, 47, 64})
    ref = {}
    for m in ms:
        out = gu.out_buffer(n, torch.bfloat16)
        plan.run(x[:m], out[:m])
        torch.cuda.synchronize()
        assert gu.sentinel_intact(out, m), f"M={m}: rows >= M were written"
        ref[m] = gu.host_bits(out).copy()
        _bound_check(si.bf16_bits_to_f32(ref[m][:m]).astype(np.float64), o[:m], sv[:m], "bf16",
                     f"shipped {n}x{k} M={m} {plan.describe(m)}")
        for _ in range(3):
            out2 = gu.out_buffer(n, torch.bfloat16)
            plan.run(x[:m], out2[:m])
            torch.cuda.synchronize()
            assert np.array_equal(gu.host_bits(out2), ref[m]), f"M={m}: repeat differs"
    timed = list(wl.m_values)
    outs = {m: gu.out_buffer(n, torch.bfloat16) for m in timed}
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for m in timed:
                plan.run(x[:m], outs[m][:m])
    for rep in range(5):
        for m in timed:
            outs[m][:m].fill_(0)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for m in timed:
            assert np.array_equal(gu.host_bits(outs[m]), ref[m]), (rep, m)
    del g
    plan.close()


@pytest.mark.parametrize("kernels", sorted(DECODE_KERNEL_SETS))
def test_decode_kernels_repeat_and_graph_replay(sk, kernels):
    """Kernel sets of the packed 6288x7168 decode weight, forced, at full
    size: bitwise identical over repeats and over graph replays with eager
    work between them, and the whole output within the bound."""
    import torch
    wl = si.WORKLOADS[3]
    w_bits, x_bits = si.weight(3, 0), si.activations(3)
    n = wl.n
    w = gu.dev_bf16(w_bits)
    x = gu.dev_bf16(x_bits)
    o_all, s_all = oracle.gemm(x_bits, w_bits)
    forced = DECODE_KERNEL_SETS[kernels](sk)
    table = []
    for m in range(1, 65):
        fits = [t for mm, t in sorted(forced.items()) if mm >= m]
        table.append(fits[0] if fits else sk.Tactic(3, 64, 128, 8, 1, 4))
    _say(f"[decode kernels {kernels}] {forced}")
    plan = sk.Prepared(w, torch.bfloat16, table=table)
    for m, t in forced.items():
        assert plan.tactic(m) == t, (m, plan.tactic(m))
    ref = {}
    for m in forced:
        out = gu.out_buffer(n, torch.bfloat16)
        plan.run(x[:m], out[:m])
        torch.cuda.synchronize()
        assert gu.sentinel_intact(out, m), f"M={m}: rows >= M were written"
        ref[m] = gu.host_bits(out).copy()
        for _ in range(10):
            out2 = gu.out_buffer(n, torch.bfloat16)
            plan.run(x[:m], out2[:m])
            torch.cuda.synchronize()
            assert np.array_equal(gu.host_bits(out2), ref[m]), f"M={m}: repeat differs"
        got = si.bf16_bits_to_f32(ref[m][:m]).astype(np.float64)
        _bound_check(got, o_all[:m], s_all[:m], "bf16", f"decode kernel M={m} {forced[m]}")
    outs = {m: gu.out_buffer(n, torch.bfloat16) for m in forced}
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for m in forced:
                plan.run(x[:m], outs[m][:m])
    for rep in range(5):
        for m in forced:
            outs[m][:m].fill_(0)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for m in forced:
            assert np.array_equal(gu.host_bits(outs[m]), ref[m]), (rep, m)
    plan.close()


def test_run_errors(sk):
    import torch
    n, k = 64, 256
    _, w_bits = si.random_case(3, 1, n, k)
    w = gu.dev_bf16(w_bits)
    plan = sk.Prepared(w, torch.float32, table=[sk.Tactic(1, 64, 16, 1, 1, 1)] * 64)
    x = gu.dev_bf16(np.zeros((66, k), dtype=np.uint16))
    out = torch.zeros((66, n), dtype=torch.float32, device="cuda")
    with pytest.raises(sk.UnsupportedTokens):
        plan.run(x[:65], out[:65])
    with pytest.raises(sk.UnsupportedTokens):
        plan.run_ptr(x.data_ptr(), out.data_ptr(), 0)
    with pytest.raises(ValueError):
        plan.run_ptr(x.data_ptr() + 2, out.data_ptr(), 4)      # x not 16-byte aligned
    with pytest.raises(ValueError):
        plan.run_ptr(x.data_ptr(), out.data_ptr() + 2, 4)      # fp32 out not 4-byte aligned
    assert plan.supports(64) and not plan.supports(65) and not plan.supports(0)
    with pytest.raises(ValueError):
        sk.Prepared(w, torch.float32, table=[sk.Tactic(0, 1, 1, 1, 1, 1)] * 64)   # tile < M
    plan.close()


def test_forced_tactic_environment(sk, monkeypatch):
    """SKINNY_FORCE_TACTIC: no tuning and no table file; the plan runs the
    named tactic for every M up to its tile and the 64-token MFMA tactic
    above it, for runs with and without a residual, exact on integer inputs."""
    import torch
    n, k = 600, 1536
    x_bits, w_bits = si.small_int_case(77, 64, n, k)
    o, _ = oracle.gemm(x_bits, w_bits)
    forced, above = sk.Tactic(9, 32, 64, 4, 3, 2), sk.Tactic(1, 64, 16, 1, 1, 1)
    monkeypatch.setenv("SKINNY_FORCE_TACTIC", "9.32.64.4.3.2")
    monkeypatch.delenv("SKINNY_TABLE_CACHE", raising=False)
    plan = sk.Prepared(gu.dev_bf16(w_bits), torch.float32)
    for m in range(1, 65):
        want = repr(forced if m <= 32 else above)
        assert repr(plan.tactic(m, False)) == want and repr(plan.tactic(m, True)) == want, m
    for m in (1, 17, 32, 33, 64):
        _check_exact(sk, plan, x_bits, o, m, f"forced M={m}")
    plan.close()


def test_tune_command_appends_then_loads(sk, tmp_path):
    """python -m skinny_bf16_decode_amd.tune tunes a shape the file does not
    hold and appends its two tables; run again on the same file, it loads
    them instead of tuning and appends nothing."""
    import os
    import subprocess
    path = tmp_path / "tables.txt"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    cmd = [sys.executable, "-m", "skinny_bf16_decode_amd.tune", "--file", str(path), "--out", "f32", "328x520"]
    env = dict(os.environ, SKINNY_LOG="1")
    env.pop("SKINNY_TABLE_CACHE", None)
    first = subprocess.run(cmd, cwd=root, env=env, capture_output=True, text=True, timeout=240)
    assert first.returncode == 0, first.stderr[-2000:]
    assert "tuned N=328 K=520" in first.stderr and "328x520 bf16->f32" in first.stdout
    lines = path.read_text().splitlines()
    assert [ln.split()[4:8] for ln in lines] == [["328", "520", "bf16", "f32"], ["328", "520", "bf16", "f32+res"]]
    second = subprocess.run(cmd, cwd=root, env=env, capture_output=True, text=True, timeout=240)
    assert second.returncode == 0, second.stderr[-2000:]
    assert "table loaded from" in second.stderr and "tuned N=328" not in second.stderr
    assert path.read_text().splitlines() == lines


def test_table_cache_file_round_trip(sk, tmp_path):
    """SKINNY_TABLE_CACHE: a tuning process appends its two tables (without
    and with a residual); a second process loads both instead of tuning and
    chooses the same tactics."""
    import os
    import subprocess
    path = tmp_path / "tables.txt"
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import numpy as np, torch, skinny_inputs as si, skinny_bf16_decode_amd as sk\n"
        "from tests import gpu_util as gu\n"
        "x, w = si.random_case(9, 1, 640, 2048)\n"
        "plan = sk.Prepared(gu.dev_bf16(w), torch.bfloat16)\n"
        "print('|'.join(repr(plan.tactic(m, r)) for r in (False, True) for m in range(1, 65)))\n"
    ) % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))),)
    env = dict(os.environ, SKINNY_TABLE_CACHE=str(path), SKINNY_LOG="1")
    first = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240)
    assert first.returncode == 0, first.stderr[-2000:]
    assert "tuned N=640 K=2048" in first.stderr
    lines = path.read_text().splitlines()
    assert len(lines) == 2 and all(ln.startswith("skinny-table v2 gfx950 ") for ln in lines)
    assert [ln.split()[4:8] for ln in lines] == [["640", "2048", "bf16", "bf16"],
                                                 ["640", "2048", "bf16", "bf16+res"]], lines
    second = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240)
    assert second.returncode == 0, second.stderr[-2000:]
    assert "table loaded from" in second.stderr and "residual table loaded from" in second.stderr
    assert "tuned N=640" not in second.stderr
    assert first.stdout.strip().splitlines()[-1] == second.stdout.strip().splitlines()[-1]
    assert len(path.read_text().splitlines()) == 2


def test_residual_table(sk):
    """Runs with a residual take the plan's residual table: at every M its
    tactic is one of the plain table's tactics with a tile >= M, and the
    residual runs are exact on integer inputs at every M (fp32 out equals
    O + R bit for bit), in place and separate."""
    import torch
    n, k = 1000, 4096
    x_bits, w_bits = si.small_int_case(33, 64, n, k)
    o, _ = oracle.gemm(x_bits, w_bits)
    rng = np.random.default_rng(5)
    r = rng.integers(-8, 9, size=(64, n)).astype(np.float32)
    plan = sk.Prepared(gu.dev_bf16(w_bits), torch.float32)
    plain = {repr(plan.tactic(m)) for m in range(1, 65)}
    x = gu.dev_bf16(x_bits)
    res = torch.from_numpy(r).cuda()
    for m in range(1, 65):
        t = plan.tactic(m, residual=True)
        assert repr(t) in plain and t.mt >= m, (m, t)
        out = torch.full((64, n), float("nan"), dtype=torch.float32, device="cuda")
        plan.run(x[:m], out[:m], residual=res[:m])
        got = out.cpu().numpy()
        assert np.array_equal(got[:m], (o[:m] + r[:m]).astype(np.float32)), m
        assert np.isnan(got[m:]).all()
        acc = res.clone()
        plan.run(x[:m], acc[:m], residual=acc[:m])
        assert np.array_equal(acc.cpu().numpy()[:m], (o[:m] + r[:m]).astype(np.float32)), m
    plan.close()


@pytest.mark.parametrize("remap", ["1", "0"])
def test_split_k_exchange_exact(sk, remap, monkeypatch):
    """Every split-K candidate, with the split workgroups of a tile placed on
    one XCD (default) and dealt over all XCDs (SKINNY_XCD_REMAP=0): the swap
    exchange must be exact on integer inputs, and leave every node empty (a
    second call gives the same bits)."""
    import torch
    monkeypatch.setenv("SKINNY_XCD_REMAP", remap)
    n, k = 392, 4096
    x_bits, w_bits = si.small_int_case(31, 64, n, k)
    o, _ = oracle.gemm(x_bits, w_bits)
    w = gu.dev_bf16(w_bits)
    tactics = [t for t in sk.enumerate_tactics(n, k) if t.split > 1]
    _say(f"[split remap={remap}] {len(tactics)} tactics")
    assert {t.path for t in tactics} >= {0, 1, 3, 8, 9, 10, 11, 12}
    for t in tactics:
        plan = sk.Prepared(w, torch.float32, table=gu.forced_table(t))
        for rep in range(2):
            _check_exact(sk, plan, x_bits, o, t.mt, f"{t} remap={remap} call {rep}")
        plan.close()


@pytest.mark.parametrize("n", [65535, 70001])
def test_row_ranges_around_2_16_tiles(sk, n):
    """Equal row ranges of one row each: 65535 ranges take the kernels' 32-bit
    row-range arithmetic, 70001 its 64-bit form.  DOT2R with and without a
    two-way K split (XCD remap and one exchange node per range), exact on
    integer inputs."""
    import torch
    k = 64
    x_bits, w_bits = si.small_int_case(7000 + n, 64, n, k)
    o, _ = oracle.gemm(x_bits, w_bits)
    w = gu.dev_bf16(w_bits)
    for t in (sk.Tactic(sk.PATH_DOT2R, 1, 1, 1, 1, 1), sk.Tactic(sk.PATH_DOT2R, 2, 1, 1, 1, 2)):
        _say(f"[ranges {n}] {t}")
        plan = sk.Prepared(w, torch.float32, table=gu.forced_table(t))
        for m in sorted({1, t.mt}):
            _check_exact(sk, plan, x_bits, o, m, f"{t} N={n} M={m}")
        plan.close()
