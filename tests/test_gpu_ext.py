"""Parity of the extended entry points (through the C ABI) with the CPU
oracle: FP16 inputs and pitched weights (class PreparedProjection and
matrix_view, page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.
projection"), pitched x / out, and the fused residual (the `residual` of
try_low_latency_gemm, page "vllm.models.kimi_k3.nvidia.low_latency_gemm").

As in test_gpu_parity: integer inputs make every fp32 partial sum exact, so
those cases are compared bit for bit; random cases use the stated bound.
"""
from __future__ import annotations

import os
import sys

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


def dev_f16(bits):
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.float16).cuda()


def _want_bits(o, out_dtype):
    import torch
    if out_dtype == torch.float32:
        return o.astype(np.float32).view(np.uint32)
    return oracle.round_bf16(o)


def _tight(got, o, s, mode, label, residual=False):
    """Beyond the stated bound: fp32 accumulation sits far inside it.  Allow
    1e-4 S, plus the output rounding in BF16 mode and the residual add."""
    tight = 1e-4 * np.asarray(s) + 1e-6
    if mode == "bf16":
        tight = tight + 2.0 ** -8 * np.abs(np.asarray(o))
    if residual:
        tight = tight + 2.0 ** -23 * np.abs(np.asarray(o))
    worst = float(np.max(np.abs(np.asarray(got) - np.asarray(o)) / tight))
    assert worst <= 1.0, f"{label}: error level above the fp32-accumulation expectation ({worst:.3f})"


def _one_per_path(sk, n, k):
    """The first enumerated tactic of every (path, token tile, split > 1) kind,
    and for MFMAW of every stage form (unroll: 8 or 16 chunks, one or two
    stages in flight)."""
    seen, pick = set(), []
    for t in sk.enumerate_tactics(n, k):
        key = (t.path, t.mt, t.split > 1, t.unroll if t.path == sk.PATH_MFMAW else 0)
        if key not in seen:
            seen.add(key)
            pick.append(t)
    return pick


def test_f16_integer_probe_every_tactic(sk):
    """Every candidate tactic, forced, on FP16 integer inputs: exact."""
    import torch
    n, k = 200, 1032
    x_bits, w_bits = si.small_int_case(77, 64, n, k, dtype="f16")
    o, _ = oracle.gemm(x_bits, w_bits, dtype="f16")
    w = dev_f16(w_bits)
    tactics = sk.enumerate_tactics(n, k)
    _say(f"[f16 exact] {len(tactics)} tactics")
    for t in tactics:
        plan = sk.Prepared(w, torch.float32, table=gu.forced_table(t))
        for m in sorted({t.mt, max(1, t.mt - 3)}):
            out = gu.out_buffer(n, torch.float32)
            plan.run(dev_f16(x_bits[:m]), out[:m])
            torch.cuda.synchronize()
            assert gu.sentinel_intact(out, m), f"{t} M={m}: rows >= M written"
            got = gu.host_bits(out)[:m]
            want = _want_bits(o[:m], torch.float32)
            assert np.array_equal(got, want), f"{t} M={m}"
        plan.close()


@pytest.mark.parametrize("od", ["f32", "bf16"])
def test_f16_decode_workload_within_bound(sk, od):
    """FP16 weights and activations of the square decode shape (W N(0, 0.02),
    x N(0, 1)), tuned, at every listed M."""
    import torch
    n, k = 3584, 7168
    out_dtype = torch.float32 if od == "f32" else torch.bfloat16
    w_bits = si.draw(si.seed_for(2, 1, 0), (n, k), ("normal", 0.02), "f16")
    x_bits = si.draw(si.seed_for(2, 2, 0), (64, k), ("normal", 1.0), "f16")
    o, s = oracle.gemm(x_bits[:32], w_bits, dtype="f16")
    plan = sk.Prepared(dev_f16(w_bits), out_dtype)
    x = dev_f16(x_bits)
    for m in (1, 2, 4, 8, 16, 32):
        out = gu.out_buffer(n, out_dtype)
        plan.run(x[:m], out[:m])
        torch.cuda.synchronize()
        assert gu.sentinel_intact(out, m)
        got = gu.values(out)[:m]
        rep = oracle.check(got, o[:m], s[:m], od)
        _say(f"[f16 {od}] M={m} {plan.describe(m)}: {rep}")
        assert rep.ok, (m, str(rep))
        _tight(got, o[:m], s[:m], od, f"M={m}")
    plan.close()


@pytest.mark.parametrize("od", ["f32", "bf16"])
@pytest.mark.parametrize("inplace", [False, True], ids=["separate", "inplace"])
def test_residual_exact(sk, od, inplace):
    """out = x W^T + R on integer inputs and an integer residual, for one
    tactic of every path (with and without a K split): exact.  In place, out
    holds R on entry."""
    import torch
    n, k = 392, 2048
    out_dtype = torch.float32 if od == "f32" else torch.bfloat16
    x_bits, w_bits = si.small_int_case(41, 64, n, k)
    rng = np.random.default_rng(43)
    r_int = rng.integers(-200, 201, size=(64, n))
    o, _ = oracle.gemm_residual(x_bits, w_bits, r_int.astype(np.float64))
    w = gu.dev_bf16(w_bits)
    if out_dtype == torch.float32:
        r_dev = torch.from_numpy(r_int.astype(np.float32)).cuda()
    else:
        r_dev = gu.dev_bf16(si.f32_to_bf16_bits(r_int.astype(np.float32)))
    tactics = _one_per_path(sk, n, k)
    assert {t.path for t in tactics} == {0, 1, 3, 8, 9, 10, 11, 12}
    _say(f"[residual {od} {'inplace' if inplace else 'separate'}] {len(tactics)} tactics")
    for t in tactics:
        plan = sk.Prepared(w, out_dtype, table=gu.forced_table(t))
        name = plan.describe(t.mt).split()[0]
        assert name.startswith(sk.PATH_NAMES[t.path]), (t, name)   # every path has its name
        for m in sorted({t.mt, max(1, t.mt - 3)}):
            out = gu.out_buffer(n, out_dtype)
            x = gu.dev_bf16(x_bits[:m])
            if inplace:
                out[:m].copy_(r_dev[:m])
                plan.run(x, out[:m], residual=out[:m])
            else:
                plan.run(x, out[:m], residual=r_dev[:m])
            torch.cuda.synchronize()
            assert gu.sentinel_intact(out, m), f"{t} M={m}"
            got = gu.host_bits(out)[:m]
            assert np.array_equal(got, _want_bits(o[:m], out_dtype)), f"{t} M={m}"
        plan.close()


def test_residual_random_within_bound(sk):
    """A BF16 residual on the packed decode shape, tuned plan."""
    import torch
    n, k = 6288, 7168
    w_bits = si.weight(3)
    x_bits = si.activations(3)
    r_bits = si.residual_case(47, 32, n)
    r_val = si.bf16_bits_to_f32(r_bits).astype(np.float64)
    o, s = oracle.gemm_residual(x_bits[:32], w_bits, r_val)
    plan = sk.Prepared(gu.dev_bf16(w_bits), torch.bfloat16)
    x = gu.dev_bf16(x_bits)
    r = gu.dev_bf16(r_bits)
    for m in (1, 8, 32):
        out = gu.out_buffer(n, torch.bfloat16)
        plan.run(x[:m], out[:m], residual=r[:m])
        torch.cuda.synchronize()
        got = gu.values(out)[:m]
        rep = oracle.check(got, o[:m], s[:m], "bf16", residual=True)
        _say(f"[residual bf16] M={m}: {rep}")
        assert rep.ok, (m, str(rep))
        _tight(got, o[:m], s[:m], "bf16", f"M={m}", residual=True)
    plan.close()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_pitched_views_exact(sk, dtype):
    """W with row pitch K + 24, x with K + 40, out with N + 7: the padding of
    W and x holds garbage that must not be read into the result, and out's
    padding columns must stay untouched."""
    import torch
    n, k = 300, 1536
    ldw, ldx, ldo = k + 24, k + 40, n + 7
    x_bits, w_bits = si.small_int_case(53, 64, n, k, dtype=dtype)
    o, _ = oracle.gemm(x_bits, w_bits, dtype=dtype)
    junk = 0x7E00 if dtype == "f16" else 0x7FC0          # NaN patterns in the pads
    wp = np.full((n, ldw), junk, dtype=np.uint16)
    wp[:, :k] = w_bits
    xp = np.full((64, ldx), junk, dtype=np.uint16)
    xp[:, :k] = x_bits
    to_dev = dev_f16 if dtype == "f16" else gu.dev_bf16
    w = to_dev(wp)[:, :k]
    x = to_dev(xp)[:, :k]
    assert w.stride() == (ldw, 1) and x.stride() == (ldx, 1)
    tactics = _one_per_path(sk, n, k)
    for t in tactics:
        plan = sk.Prepared(w, torch.float32, table=gu.forced_table(t))
        for m in sorted({t.mt, max(2, t.mt - 3)}):
            buf = gu.out_buffer(ldo, torch.float32)
            out = buf[:, :n]
            plan.run(x[:m], out[:m])
            torch.cuda.synchronize()
            bits = gu.host_bits(buf)
            assert np.all(bits[:m, n:] == gu.SENTINEL_F32), f"{t} M={m}: padding columns written"
            assert np.all(bits[m:] == gu.SENTINEL_F32), f"{t} M={m}: rows >= M written"
            assert np.array_equal(bits[:m, :n], _want_bits(o[:m], torch.float32)), f"{t} M={m}"
        plan.close()


def _shipped_f16_table(sk, n, k, od):
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "skinny_bf16_decode_amd", "tables", "mi355x_tuned.txt")
    with open(path) as f:
        for line in f:
            p = line.split()
            if p[3:8] == ["256", str(n), str(k), "f16", od]:
                return [sk.Tactic(*map(int, e.split("."))) for e in p[8:]]
    raise AssertionError(f"no shipped FP16 table for {n}x{k} {od}")


@pytest.mark.parametrize("shape", [(6288, 7168), (3584, 7168), (7168, 18432), (1536, 128)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_f16_shipped_tables_exact_full_size(sk, shape):
    """The shipped FP16-input tables, forced at their full shape on integer
    FP16 inputs: every M = 1..64, BF16 out bit-identical to RNE(O) and (where
    an fp32-out table ships) fp32 out to O."""
    import torch
    n, k = shape
    x_bits, w_bits = si.small_int_case(4242 + n, 64, n, k, dtype="f16")
    o, _ = oracle.gemm(x_bits, w_bits, dtype="f16")
    w, x = dev_f16(w_bits), dev_f16(x_bits)
    for od, name in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        if od == torch.float32 and shape != (1536, 128):
            continue
        table = _shipped_f16_table(sk, n, k, name)
        plan = sk.Prepared(w, od, table=table)
        for m in range(1, 65):
            out = gu.out_buffer(n, od)
            plan.run(x[:m], out[:m])
            torch.cuda.synchronize()
            assert gu.sentinel_intact(out, m), (shape, name, m)
            assert np.array_equal(gu.host_bits(out)[:m], _want_bits(o[:m], od)), (shape, name, m, table[m - 1])
        plan.close()


def _random_extended_cases(sk, seed, cases, n_hi, k8_hi, max_elems, case_seed):
    """Seeded random combinations of the extended entry points: a random
    shape (N < n_hi, K = 8 j with j < k8_hi and N K <= max_elems), a tactic
    drawn from the shape's own candidates, a random M up to its tile, BF16 or
    FP16 inputs, row-pitched W, x and out (NaN patterns in the padding of W
    and x, sentinels in out's), no residual, a separate one or out itself,
    BF16 or fp32 out.  Integer inputs and an integer residual keep every sum
    exact, so out must be RNE(O + R) (BF16) or O + R (fp32) bit for bit, on
    two calls in a row (the split-K exchange nodes are empty again after
    each launch).  Returns the (path, input type, residual) kinds seen."""
    import torch
    rng = np.random.default_rng(seed)
    seen = set()
    for case in range(cases):
        n = int(rng.integers(1, n_hi))
        k = 8 * int(rng.integers(1, max(2, min(k8_hi, max_elems // (8 * n) + 1))))
        dtype = "f16" if rng.integers(0, 2) else "bf16"
        od = torch.float32 if rng.integers(0, 2) else torch.bfloat16
        mode = ("none", "separate", "inplace")[int(rng.integers(0, 3))]
        ldw, ldx, ldo = k + 8 * int(rng.integers(0, 4)), k + 8 * int(rng.integers(0, 4)), n + int(rng.integers(0, 9))
        tactics = sk.enumerate_tactics(n, k)
        t = tactics[int(rng.integers(0, len(tactics)))]
        m = int(rng.integers(1, t.mt + 1))
        x_bits, w_bits = si.small_int_case(case_seed + case, m, n, k, dtype=dtype)
        r_int = rng.integers(-100, 101, size=(m, n)) if mode != "none" else np.zeros((m, n), dtype=np.int64)
        o, _ = oracle.gemm_residual(x_bits, w_bits, r_int.astype(np.float64), dtype=dtype)
        junk = 0x7E00 if dtype == "f16" else 0x7FC0
        wp = np.full((n, ldw), junk, dtype=np.uint16)
        wp[:, :k] = w_bits
        xp = np.full((m, ldx), junk, dtype=np.uint16)
        xp[:, :k] = x_bits
        to_dev = dev_f16 if dtype == "f16" else gu.dev_bf16
        w, x = to_dev(wp)[:, :k], to_dev(xp)[:, :k]
        plan = sk.Prepared(w, od, table=gu.forced_table(t))
        buf = gu.out_buffer(ldo, od)
        out = buf[:, :n]
        r_dev = torch.from_numpy(r_int.astype(np.float32)).cuda().to(od)
        label = f"case {case}: {n}x{k} ldw={ldw} ldx={ldx} ldo={ldo} M={m} {dtype}->{od} residual={mode} {t}"
        for call in range(2):
            res = None
            if mode == "inplace":
                out[:m].copy_(r_dev)
                res = out[:m]
            elif mode == "separate":
                res = r_dev
            plan.run(x, out[:m], residual=res)
            torch.cuda.synchronize()
            bits = gu.host_bits(buf)
            sentinel = gu.SENTINEL_F32 if od == torch.float32 else gu.SENTINEL_BF16
            assert np.all(bits[:m, n:] == sentinel), f"{label} call {call}: padding columns written"
            assert np.all(bits[m:] == sentinel), f"{label} call {call}: rows >= M written"
            assert np.array_equal(bits[:m, :n], _want_bits(o, od)), f"{label} call {call}"
        plan.close()
        seen.add((t.path, dtype, mode))
        if (case + 1) % 100 == 0:
            _say(f"  {case + 1}/{cases} cases exact")
    return seen


def test_random_extended_calls_exact(sk):
    """80 random combinations of the extended entry points on shapes up to
    1500 x 2400 (see _random_extended_cases)."""
    seen = _random_extended_cases(sk, 1203, 80, 1500, 301, 1 << 62, 70_000)
    _say(f"[random extended] {len(seen)} (path, input, residual) kinds")


def test_random_extended_calls_large_shapes_exact(sk):
    """The same on shapes up to 20000 rows, K up to 20000 and 1.4e8 weight
    elements (the long-K weight has 1.32e8), where row ranges, splits and
    32-bit offsets reach their full size.  SKINNY_RANDOM_LARGE_CASES sets the
    count (default 40)."""
    cases = int(os.environ.get("SKINNY_RANDOM_LARGE_CASES", "40"))
    seen = _random_extended_cases(sk, 20261204, cases, 20001, 2501, 140_000_000, 80_000)
    _say(f"[random extended, large] {len(seen)} (path, input, residual) kinds, "
         f"paths {sorted({p for p, _, _ in seen})}")


def test_prepare_from_threads(sk, monkeypatch):
    """skinny_prepare from four threads at once, two per shape, with no
    stored table: the first prepare of a shape tunes (capturing its timing
    graphs on its own stream) while the other threads allocate and wait for
    the table cache; every plan must get the same table per shape and give
    exact results on integer inputs."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    monkeypatch.delenv("SKINNY_TABLE_CACHE", raising=False)
    shapes = [(264, 520), (1544, 136)]          # shapes no other test tunes: nothing cached yet
    cases = {}
    for i, (n, k) in enumerate(shapes):
        x_bits, w_bits = si.small_int_case(300 + i, 64, n, k)
        o, _ = oracle.gemm(x_bits, w_bits)
        cases[(n, k)] = (gu.dev_bf16(x_bits), gu.dev_bf16(w_bits), o)
    torch.cuda.synchronize()

    def prepare(shape):
        torch.cuda.set_device(0)
        x, w, _ = cases[shape]
        plan = sk.Prepared(w, torch.float32)
        return shape, plan, [repr(plan.tactic(m)) for m in range(1, 65)]

    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(prepare, [shapes[0], shapes[1], shapes[0], shapes[1]]))
    tables = {}
    for shape, plan, table in results:
        assert tables.setdefault(shape, table) == table, f"{shape}: two threads got different tables"
        x, _, o = cases[shape]
        for m in (1, 7, 16, 33, 64):
            out = gu.out_buffer(shape[0], torch.float32)
            plan.run(x[:m], out[:m])
            torch.cuda.synchronize()
            assert gu.sentinel_intact(out, m), (shape, m)
            assert np.array_equal(gu.host_bits(out)[:m], o[:m].astype(np.float32).view(np.uint32)), (shape, m)
        plan.close()


def test_concurrent_plans_on_streams(sk):
    """Four threads, each with its own plan (a K-split tactic, so each plan's
    exchange workspace is in use) and its own stream, launch 24 runs each
    without waiting, at changing M, into 24 output buffers; all four streams
    run at once.  Every output must be exact on integer inputs afterwards: no
    plan sees another's partials."""
    import threading
    import torch
    n, k = 600, 1536
    tactics = [sk.Tactic(9, 32, 64, 4, 3, 2), sk.Tactic(1, 64, 16, 2, 1, 4), sk.Tactic(10, 16, 28, 2, 2, 3),
               sk.Tactic(3, 32, 64, 4, 2, 2)]
    cases = []
    for i, t in enumerate(tactics):
        x_bits, w_bits = si.small_int_case(9400 + i, 64, n, k)
        o, _ = oracle.gemm(x_bits, w_bits)
        plan = sk.Prepared(gu.dev_bf16(w_bits), torch.float32, table=gu.forced_table(t))
        outs = [gu.out_buffer(n, torch.float32) for _ in range(24)]
        cases.append((t, gu.dev_bf16(x_bits), plan, outs, o))
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            torch.cuda.set_device(0)
            t, x, plan, outs, _ = cases[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for j, out in enumerate(outs):
                    m = 1 + (j * 7 + i) % t.mt
                    plan.run(x[:m], out[:m], stream=stream)
            stream.synchronize()
        except Exception as e:                  # reported by the main thread
            errors.append((i, e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (t, _, plan, outs, o) in enumerate(cases):
        for j, out in enumerate(outs):
            m = 1 + (j * 7 + i) % t.mt
            assert gu.sentinel_intact(out, m), f"{t} run {j}: rows >= M written"
            got = gu.host_bits(out)[:m]
            assert np.array_equal(got, o[:m].astype(np.float32).view(np.uint32)), f"{t} run {j} M={m}"
        plan.close()


def test_run_ex_argument_errors(sk):
    """Pitches below the row length, unaligned pitches and a residual that
    overlaps out without being it are refused before any launch."""
    import ctypes
    import torch
    n, k = 64, 256
    lib = sk.load_library()
    w = gu.dev_bf16(si.small_int_case(1, 1, n, k)[1])
    plan = sk.Prepared(w, torch.float32, table=[sk.Tactic(1, 64, 16, 1, 1, 1)] * 64)
    x = torch.zeros((4, k + 8), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((8, n + 8), dtype=torch.float32, device="cuda")
    p = plan._plan
    xp, op = ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr())
    assert lib.skinny_run_ex(p, xp, k - 8, None, 0, op, n, 4, None) == 2        # ldx < K
    assert lib.skinny_run_ex(p, xp, k + 4, None, 0, op, n, 4, None) == 2        # ldx % 8
    assert lib.skinny_run_ex(p, xp, k, None, 0, op, n - 1, 4, None) == 2        # ldo < N
    r = ctypes.c_void_p(out.data_ptr() + 4 * 3)                                 # overlaps out
    assert lib.skinny_run_ex(p, xp, k, r, n, op, n, 4, None) == 1
    assert lib.skinny_run_ex(p, xp, k, op, n + 8, op, n, 4, None) == 1          # out, other pitch
    assert lib.skinny_run_ex(p, xp, k, op, n, op, n, 4, None) == 0              # in place: fine
    assert lib.skinny_run_ex(p, xp, k, None, 0, op, n, 65, None) == 4
    torch.cuda.synchronize()
    plan.close()
    with pytest.raises(ValueError):
        sk.Prepared(w[:, :250], torch.float32)                                  # K % 8 != 0


def test_kda_projection_two_streams(sk):
    """The KDA decode projection with its F_A/beta -> F_B branch on a second
    stream: every output matches the oracle (F_B against the oracle applied
    to the F_A output the GPU produced), and equals, bit for bit, the same
    products run on one stream -- also when captured in a graph and replayed."""
    import torch
    from skinny_bf16_decode_amd import kda
    w_bits = si.weight(3)
    fb_bits = si.weight(4)
    x_bits = si.activations(3)
    proj = kda.KdaProjection(gu.dev_bf16(w_bits), gu.dev_bf16(fb_bits))
    aux = torch.cuda.Stream()
    events = (torch.cuda.Event(), torch.cuda.Event())
    x = gu.dev_bf16(x_bits)
    rows_fab = kda.F_A_ROWS + kda.BETA_ROWS
    for m in (1, 8, 32):
        out = proj.outputs(m)
        proj.run(x[:m], out, aux, events)
        torch.cuda.synchronize()
        o, s = oracle.gemm(x_bits[:m], w_bits[:kda.QKVG_ROWS + rows_fab])
        rep = oracle.check(gu.values(out.qkvg), o[:, :kda.QKVG_ROWS], s[:, :kda.QKVG_ROWS], "bf16")
        assert rep.ok, f"qkvg M={m}: {rep}"
        rep = oracle.check(gu.values(out.fab), o[:, kda.QKVG_ROWS:], s[:, kda.QKVG_ROWS:], "bf16")
        assert rep.ok, f"F_A/beta M={m}: {rep}"
        fa_bits = gu.host_bits(out.fab)[:, :kda.F_A_ROWS]
        o2, s2 = oracle.gemm(np.ascontiguousarray(fa_bits), fb_bits)
        rep = oracle.check(gu.values(out.f_b), o2, s2, "bf16")
        assert rep.ok, f"F_B M={m}: {rep}"
        _say(f"[kda] M={m}: qkvg/fab/f_b within bound")
        ref = [gu.host_bits(t).copy() for t in (out.qkvg, out.fab, out.f_b)]
        ser = proj.outputs(m)
        proj.run_serial(x[:m], ser)
        torch.cuda.synchronize()
        for a, b in zip(ref, (ser.qkvg, ser.fab, ser.f_b)):
            assert np.array_equal(a, gu.host_bits(b))
        stream = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        gout = proj.outputs(m)
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                proj.run(x[:m], gout, aux, events)
        for rep_i in range(3):
            for t in (gout.qkvg, gout.fab, gout.f_b):
                t.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for a, b in zip(ref, (gout.qkvg, gout.fab, gout.f_b)):
                assert np.array_equal(a, gu.host_bits(b)), f"graph replay {rep_i} M={m}"
        pk, fbo = proj.packed_outputs(m)
        proj.run_packed(x[:m], pk, fbo)
        torch.cuda.synchronize()
        rows = kda.QKVG_ROWS + rows_fab
        rep = oracle.check(gu.values(pk)[:, :rows], o, s, "bf16")
        assert rep.ok, f"packed M={m}: {rep}"
        fa_bits = np.ascontiguousarray(gu.host_bits(pk)[:, kda.QKVG_ROWS:kda.QKVG_ROWS + kda.F_A_ROWS])
        o3, s3 = oracle.gemm(fa_bits, fb_bits)
        rep = oracle.check(gu.values(fbo), o3, s3, "bf16")
        assert rep.ok, f"packed F_B M={m}: {rep}"
    proj.close()
