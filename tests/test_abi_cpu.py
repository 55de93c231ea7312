"""The C ABI on the CPU: the library loads, exports every function the
header declares, rejects bad arguments before touching the device, and the
tactic logic (legality, candidate list, per-M table rule) behaves as stated.
No kernel is launched here."""
from __future__ import annotations

import ctypes
import sys
import os
import re
import subprocess

import pytest

import skinny_bf16_decode_amd as sk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skinny.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(skinny_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "skinny_prepare" in names and "skinny_run" in names
    lib = sk.load_library()
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", sk.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (skinny_[a-z_0-9]+)$", out, flags=re.M))
    assert set(names) <= exported, set(names) - exported


def _prepare(ptr, n, k, od=0):
    lib = sk.load_library()
    plan = ctypes.c_void_p(123)
    st = lib.skinny_prepare(ctypes.c_void_p(ptr), n, k, od, ctypes.byref(plan))
    return st, plan


@pytest.mark.parametrize("ptr,n,k,od,want", [
    (0, 256, 512, 0, 1),            # W NULL
    (0x1000, 0, 512, 0, 1),         # N <= 0
    (0x1000, 256, 0, 0, 1),         # K <= 0
    (0x1000, 256, 512, 7, 1),       # bad out dtype
    (0x1000, 256, 513, 0, 2),       # K % 8
    (0x1000, 65536, 65536, 0, 2),   # N*K >= 2^31
    (0x1001, 256, 512, 0, 3),       # misaligned W
    (0x1008, 256, 512, 1, 3),
])
def test_prepare_rejects_before_any_device_call(ptr, n, k, od, want):
    st, plan = _prepare(ptr, n, k, od)
    assert st == want, sk.last_error()
    assert plan.value is None          # *plan cleared on failure
    assert sk.last_error()


@pytest.mark.parametrize("n,k,ldw,idt,od,want", [
    (256, 512, 504, 0, 0, 2),       # ldw < K
    (256, 512, 516, 0, 0, 2),       # ldw % 8
    (256, 512, 512, 2, 0, 1),       # bad in dtype
    (256, 512, 512, -1, 1, 1),
    (256, 512, 1 << 26, 0, 0, 2),   # 16 rows of W past 2 GiB
    (256, 512, 1 << 24, 0, 0, 2),   # 64 rows of W (the largest tile) reach the out-of-range load offset
])
def test_prepare_ex_rejects_before_any_device_call(n, k, ldw, idt, od, want):
    lib = sk.load_library()
    plan = ctypes.c_void_p(123)
    st = lib.skinny_prepare_ex(ctypes.c_void_p(0x1000), n, k, ldw, idt, od, ctypes.byref(plan))
    assert st == want, sk.last_error()
    assert plan.value is None
    plan = ctypes.c_void_p(123)
    st = lib.skinny_prepare_tactics_ex(ctypes.c_void_p(0x1000), n, k, ldw, idt, od, None, ctypes.byref(plan))
    assert st == want, sk.last_error()


def test_run_ex_null_plan():
    lib = sk.load_library()
    assert lib.skinny_run_ex(None, ctypes.c_void_p(0x1000), 512, None, 0, ctypes.c_void_p(0x1000), 256, 4,
                             None) == 1


def test_prepare_null_plan_pointer():
    lib = sk.load_library()
    assert lib.skinny_prepare(ctypes.c_void_p(0x1000), 16, 64, 0, None) == 1


def test_run_argument_errors():
    lib = sk.load_library()
    assert lib.skinny_run(None, ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1000), 4, None) == 1
    assert lib.skinny_supports(None, 4) == 0
    assert lib.skinny_describe(None, 4, ctypes.create_string_buffer(8), 8) == 1


def test_status_strings():
    lib = sk.load_library()
    for code in range(8):
        assert lib.skinny_status_string(code)
    assert lib.skinny_status_string(99) == b"unknown status"


def T(*a):
    return sk.Tactic(*a)


def test_tactic_check_rules():
    ok = [T(0, 8, 4, 4, 1, 1), T(0, 1, 16, 1, 1, 8), T(1, 64, 16, 4, 1, 2), T(1, 16, 64, 8, 2, 1)]
    for t in ok:
        sk.tactic_check(t, 6288, 7168)
    bad = [T(0, 3, 1, 1, 1, 1),          # no such token tile
           T(0, 8, 16, 1, 1, 1),         # mt * rows > 64
           T(0, 1, 1, 3, 1, 1),          # waves not a power of two
           T(0, 1, 1, 16, 1, 1),         # too many waves
           T(0, 1, 1, 1, 3, 1),          # unroll
           T(0, 1, 1, 1, 1, 0),          # split < 1
           T(0, 1, 1, 1, 1, 17),         # split > 16
           T(1, 16, 24, 1, 1, 1),        # rows not a multiple of 16
           T(1, 64, 64, 8, 1, 1),        # LDS over the limit
           T(2, 16, 16, 1, 1, 1)]        # no such path
    for t in bad:
        with pytest.raises(ValueError):
            sk.tactic_check(t, 6288, 7168)
    with pytest.raises(ValueError):
        sk.tactic_check(T(0, 1, 1, 1, 1, 4), 16, 16)     # split > chunks of a row
    with pytest.raises(ValueError):
        sk.tactic_check(T(0, 1, 1, 1, 1, 1), 16, 12)     # K % 8


def test_enumeration_is_legal_and_covers_every_tile():
    for n, k in ((256, 512), (3584, 7168), (6288, 7168), (1536, 128), (7168, 18432), (200, 1032)):
        cands = sk.enumerate_tactics(n, k)
        assert cands, (n, k)
        for t in cands:
            sk.tactic_check(t, n, k)
        assert {t.mt for t in cands} == {1, 2, 4, 8, 16, 32, 64}
        assert len(set(cands)) == len(cands)
    assert sk.load_library().skinny_enumerate_tactics(0, 64, None, 0) == -1


def test_row_range_tactics():
    """The equal-row-range forms: MFMAX with unroll 2 and DOT2R (path 8, the
    DOT2 kernels) are enumerated and legal; MFMAX takes unroll 1 or 2 only, and
    DOT2R follows DOT2's rules on rows and unroll."""
    cands = sk.enumerate_tactics(6288, 7168)
    assert any(t.path == 3 and t.unroll == 2 for t in cands)
    assert any(t.path == 3 and t.unroll == 1 for t in cands)
    assert any(t.path == sk.PATH_DOT2R for t in cands)
    sk.tactic_check(T(3, 16, 32, 2, 2, 1), 6288, 7168)
    sk.tactic_check(T(sk.PATH_DOT2R, 2, 4, 1, 2, 1), 6288, 7168)
    with pytest.raises(ValueError):
        sk.tactic_check(T(3, 16, 32, 2, 3, 1), 6288, 7168)        # MFMAX unroll 3
    with pytest.raises(ValueError):
        sk.tactic_check(T(sk.PATH_DOT2R, 2, 3, 1, 1, 1), 6288, 7168)   # no DOT2 kernel with 3 rows
    with pytest.raises(ValueError):
        sk.tactic_check(T(12, 16, 16, 1, 1, 1), 6288, 7168)       # no such path
    # many workgroups per CU balance themselves: no DOT2R with more than
    # eight per CU of the part enumerated for (256 CUs unless told otherwise)
    for cus in (256, 80):
        for t in sk.enumerate_tactics(6288, 7168, cus=cus):
            if t.path == sk.PATH_DOT2R:
                assert -(-6288 // t.rows) * t.split <= 8 * cus


@pytest.mark.parametrize("path", [2, 4, 5, 6, 7])
def test_retired_paths_are_refused(path):
    """Kernel families measured and removed keep their path numbers reserved:
    a tactic naming one is refused (so a stored table that names one is
    ignored and the shape tuned afresh), and none is enumerated."""
    with pytest.raises(ValueError, match="removed"):
        sk.tactic_check(T(path, 16, 32, 2, 1, 1), 6288, 7168)
    assert all(t.path == 0 or t.path not in (2, 4, 5, 6, 7) for t in sk.enumerate_tactics(6288, 7168))


def test_enumeration_follows_the_cu_count():
    """The launch-shape rules take the device's CU count: a part with fewer
    CUs gets fewer K-split DOT2R candidates (its rows already fill it) and
    MFMA4 instances sized to its larger per-CU row ranges."""
    full = sk.enumerate_tactics(6288, 7168)
    assert full == sk.enumerate_tactics(6288, 7168, cus=256)
    small = sk.enumerate_tactics(6288, 7168, cus=64)
    for t in small:
        sk.tactic_check(t, 6288, 7168)
    m4 = lambda c: {t.rows for t in c if t.path == sk.PATH_MFMA4 and t.split == 1}
    # one range per CU without a K split: 24-25 rows on 256 CUs, 49-50 on 64
    assert 28 in m4(full) and 52 not in m4(full)
    assert 52 in m4(small)
    assert sk.load_library().skinny_enumerate_tactics_ex(6288, 7168, 0, None, 0) == -1


@pytest.mark.parametrize("path,tiles", [(sk.PATH_MFMA4, {4, 8, 16, 32}), (sk.PATH_DOT2W, {1, 2, 4, 8})])
def test_row_group_stream_tactics(path, tiles):
    """MFMA4 (path 10) and DOT2W (path 11), the row-group stream kernels:
    ranges of at most 4, 8, 16, 28, 52 or 56 rows, at most 4 waves, 2 or 3
    stages of 16 chunks in flight, K split 1..8 and no more parts than
    stages; the enumerator keeps the instance whose 4-row groups the equal
    ranges fill (none left empty)."""
    cands = [t for t in sk.enumerate_tactics(6288, 7168) if t.path == path]
    assert {t.mt for t in cands} == tiles
    assert {t.unroll for t in cands} == {2, 3}
    for t in cands:
        per_round = -(-256 // t.split)
        ranges = -(-(-(-6288 // t.rows)) // per_round) * per_round
        most = -(-6288 // ranges)
        assert t.rows - 4 < most <= t.rows, t
        assert t.waves <= 4
    assert any(t.rows == 28 and t.split == 1 for t in cands)      # 24-25 rows per CU
    assert any(t.rows == 52 and t.split == 2 for t in cands)      # 49 rows, two K halves
    big = max(tiles)
    sk.tactic_check(T(path, big, 28, 4, 3, 1), 6288, 7168)
    sk.tactic_check(T(path, big // 2, 56, 1, 2, 8), 6288, 7168)
    for bad in (T(path, big, 52, 4, 2, 1),            # 13 row groups x the largest tile: not compiled
                T(path, big // 2, 24, 4, 2, 1),       # no 6-group instance
                T(path, big // 2, 28, 8, 2, 1),       # more than 4 waves
                T(path, big // 2, 28, 4, 1, 1),       # 2 or 3 stages in flight
                T(path, big // 2, 28, 4, 4, 1),
                T(path, 3 * big // 8, 28, 4, 2, 1),   # not a compiled token tile
                T(path, big // 2, 28, 4, 2, 9)):      # more than 8 K parts
        with pytest.raises(ValueError):
            sk.tactic_check(bad, 6288, 7168)
    with pytest.raises(ValueError):
        sk.tactic_check(T(path, big // 2, 28, 1, 2, 3), 64, 256)   # 2 stages of 16 chunks


def test_barrier_free_row_range_tactics():
    """MFMAW (path 9): ranges of at most 16, 32 or 64 rows (row groups of
    16), with its compiled wave counts only, stages of 8 (unroll 1, 3) or 16
    chunks (unroll 2, 4), two (unroll 1, 2) or one (3, 4) in flight, and a K
    split no larger than its stage count; every wave of every candidate owns
    at least two stages of its K part."""
    cands = [t for t in sk.enumerate_tactics(6288, 7168) if t.path == sk.PATH_MFMAW]
    assert {t.mt for t in cands} == {16, 32, 64}
    assert {t.unroll for t in cands} == {1, 2, 3, 4}
    assert {t.rows for t in cands} == {16, 32, 64}
    for t in cands:
        assert t.rows % 16 == 0
        sc = 16 if t.unroll in (2, 4) else 8
        assert (7168 // 8) // t.split >= 2 * t.waves * sc
    sk.tactic_check(T(sk.PATH_MFMAW, 32, 64, 4, 2, 2), 6288, 7168)
    sk.tactic_check(T(sk.PATH_MFMAW, 16, 32, 2, 2, 1), 6288, 7168)
    for bad in (T(sk.PATH_MFMAW, 32, 64, 8, 2, 1),    # spills: not compiled
                T(sk.PATH_MFMAW, 16, 48, 4, 2, 1),    # no 3-group instance
                T(sk.PATH_MFMAW, 16, 24, 4, 2, 1),    # not whole row groups
                T(sk.PATH_MFMAW, 16, 32, 4, 5, 1),    # stages of 8 or 16 chunks, one or two deep
                T(sk.PATH_MFMAW, 16, 32, 4, 3, 1),    # no one-deep instance of two row groups, 16 tokens
                T(sk.PATH_MFMAW, 16, 32, 4, 2, 9),    # 128 chunks: 8 stages of 16
                T(sk.PATH_MFMAW, 16, 32, 4, 1, 17)):  # 16 stages of 8
        with pytest.raises(ValueError):
            sk.tactic_check(bad, 6288, 1024)


def test_token_group_tactics():
    """MFMAT (path 12): the 16-token MFMA kernels over token groups, serving
    at most 32 or 64 tokens.  Candidates only for weights of at most 16 MiB
    (their groups re-read each row tile from L2), with the MFMA kernels'
    rows, waves and unroll."""
    small = [t for t in sk.enumerate_tactics(1536, 128) if t.path == sk.PATH_MFMAT]
    assert {t.mt for t in small} == {32, 64}
    assert {t.rows for t in small} == {16, 32, 64}
    plain = {(t.rows, t.waves, t.unroll) for t in sk.enumerate_tactics(1536, 128)
             if t.path == sk.PATH_MFMA and t.mt == 16 and t.split == 1}
    assert {(t.rows, t.waves, t.unroll) for t in small if t.split == 1} == plain
    assert any(t.path == sk.PATH_MFMAT for t in sk.enumerate_tactics(140, 7168))
    assert any(t.path == sk.PATH_MFMAT for t in sk.enumerate_tactics(256, 512))
    for n, k in ((6288, 7168), (3584, 7168), (7168, 18432), (1024, 8200)):   # 16 MiB and more
        assert not any(t.path == sk.PATH_MFMAT for t in sk.enumerate_tactics(n, k)), (n, k)
    assert any(t.path == sk.PATH_MFMAT for t in sk.enumerate_tactics(1024, 8192))   # exactly 16 MiB
    sk.tactic_check(T(sk.PATH_MFMAT, 64, 16, 4, 1, 1), 1536, 128)
    sk.tactic_check(T(sk.PATH_MFMAT, 32, 64, 2, 2, 2), 140, 7168)
    for bad in (T(sk.PATH_MFMAT, 16, 16, 4, 1, 1),     # one group: that is MFMA
                T(sk.PATH_MFMAT, 48, 16, 4, 1, 1),     # 32 or 64 tokens only
                T(sk.PATH_MFMAT, 64, 48, 4, 1, 1),     # no 48-row MFMA instance
                T(sk.PATH_MFMAT, 64, 64, 4, 4, 1),     # no 64-row MFMA instance with unroll 4
                T(sk.PATH_MFMAT, 64, 16, 4, 1, 5)):    # 128 K: 4 steps of 32
        with pytest.raises(ValueError):
            sk.tactic_check(bad, 1536, 128)


def test_table_rule_with_a_fake_timer():
    """table[M] = fastest candidate whose token tile >= M; ties to the
    smaller tile, then the lower index; failed candidates are skipped."""
    cands = sk.enumerate_tactics(6288, 7168)
    # fake timer: cost grows with the tile, plus a per-candidate jitter
    times = [10.0 + 0.1 * t.mt + 0.001 * ((i * 7919) % 101) for i, t in enumerate(cands)]
    table = sk.select_table(cands, times)
    for m in range(1, 65):
        legal = [(times[i], cands[i].mt, i) for i in range(len(cands)) if cands[i].mt >= m]
        want = cands[min(legal)[2]]
        assert table[m - 1] == want, m
        assert table[m - 1].mt >= m
    # smallest tile >= M wins under a cost that grows with the tile
    tiles = [1, 2, 4, 4, 8, 8, 8, 8] + [16] * 8 + [32] * 16 + [64] * 32
    assert [t.mt for t in table] == tiles


def test_table_rule_prefers_a_faster_bigger_tile_and_skips_failures():
    a, b, c = T(0, 1, 1, 1, 1, 1), T(0, 8, 4, 1, 1, 1), T(1, 64, 16, 1, 1, 1)
    table = sk.select_table([a, b, c], [5.0, 4.0, 9.0])
    assert table[0] == b                     # tile 8 faster than tile 1 at M=1
    assert all(t == c for t in table[8:])
    table = sk.select_table([a, b, c], [5.0, -1.0, 9.0])   # b could not run
    assert table[0] == a and table[1] == c
    # equal times: the smaller tile
    table = sk.select_table([c, b], [4.0, 4.0])
    assert table[0] == b
    with pytest.raises(ValueError):
        sk.select_table([a], [1.0])          # nothing serves M = 2..64


def test_python_binding_has_no_fallback(tmp_path):
    """Loading from a path with no library raises instead of computing elsewhere."""
    import importlib
    mod = importlib.import_module("skinny_bf16_decode_amd")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError):
            mod.load_library(str(tmp_path / "libskinny.so"))
    finally:
        mod._lib = saved


def test_bench_names_the_kernel_of_every_tactic():
    """bench.py matches launches to the rocprofv3 traffic record by kernel
    name; every enumerated tactic must map to its BF16 instance."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    for t in sk.enumerate_tactics(6288, 7168):
        name = bench.kernel_name(t)
        assert name and re.fullmatch(r"k_(dot2|mfma|mfmax|mfmaw|rgs)<((\d+|true|false), )+false>",
                                     name), (t, name)
    assert bench.kernel_name(T(sk.PATH_MFMA4, 16, 28, 4, 3, 1)) == "k_rgs<true, 4, 7, 3, false>"
    assert bench.kernel_name(T(sk.PATH_MFMA4, 4, 52, 2, 2, 2)) == "k_rgs<true, 1, 13, 2, false>"
    assert bench.kernel_name(T(sk.PATH_DOT2W, 8, 28, 4, 2, 1)) == "k_rgs<false, 8, 7, 2, false>"
    assert bench.kernel_name(T(3, 32, 64, 4, 2, 2)) == "k_mfmax<2, 4, false>"
    assert bench.kernel_name(T(sk.PATH_DOT2R, 2, 4, 1, 2, 1)) == "k_dot2<2, 4, 2, false>"
    assert bench.kernel_name(T(sk.PATH_MFMAW, 32, 64, 4, 2, 2)) == "k_mfmaw<2, 4, 4, 16, 2, false>"
    assert bench.kernel_name(T(sk.PATH_MFMAW, 16, 32, 2, 1, 1)) == "k_mfmaw<1, 2, 2, 8, 2, false>"
    assert bench.kernel_name(T(sk.PATH_MFMAW, 32, 64, 4, 3, 2)) == "k_mfmaw<2, 4, 4, 8, 1, false>"
    assert bench.kernel_name(T(sk.PATH_MFMAW, 32, 32, 4, 4, 1)) == "k_mfmaw<2, 2, 4, 16, 1, false>"
    assert bench.kernel_name(T(sk.PATH_MFMAT, 64, 32, 4, 2, 1)) == "k_mfma<1, 2, 2, false>"
    for t in sk.enumerate_tactics(1536, 128):
        assert bench.kernel_name(t), t


def test_shipped_table_is_legal_and_profiled():
    """The tactic tables bench.py loads by default: one line per (chip,
    shape, input type, output type, residual or not), every entry legal for
    its shape with a token tile >= M (the library ignores a line that fails
    this, and tunes instead), and for BF16 inputs the shape's committed HBM
    traffic record names the kernel of every token count its benchmark step
    runs (which adds no residual).  FP16-input tables ship for the same
    shapes."""
    import json
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    with open(bench.SHIPPED_TABLES) as f:
        lines = [ln.split() for ln in f if ln.strip()]
    assert lines
    heads = set()
    for ln in lines:
        assert ln[:3] == ["skinny-table", "v2", "gfx950"] and len(ln) == 8 + 64
        n, k = int(ln[4]), int(ln[5])
        heads.add(tuple(ln[:8]))
        for m, field in enumerate(ln[8:], start=1):
            t = T(*map(int, field.split(".")))
            sk.tactic_check(t, n, k)
            assert t.mt >= m
    assert len(heads) == len(lines)
    assert any(ln[4:8] == ["6288", "7168", "bf16", "bf16"] for ln in lines)
    assert any(ln[4:8] == ["6288", "7168", "f16", "bf16"] for ln in lines)
    import skinny_inputs as si
    profiled = 0
    for ln in lines:
        wl = next((w for w in si.WORKLOADS.values() if [str(w.n), str(w.k)] == ln[4:6]), None)
        if wl is None:
            continue                                     # a sub-plan of the KDA projection
        if ln[7].endswith("+res"):
            continue                                     # runs with a residual: not in the profiled sweeps
        if ln[6] != "bf16":
            continue                                     # FP16 inputs: the profiled sweeps run BF16
        path = bench.traffic_record_path(wl, ln[7])
        if wl.cid == 1 and not os.path.exists(path):
            continue                                     # the tiny shape has no M sweep to profile
        profiled += 1
        with open(path) as f:
            rec = json.load(f)
        for m in wl.m_values:
            name = bench.kernel_name(T(*map(int, ln[8 + m - 1].split("."))))
            assert name in rec["kernels"], (wl.name, m, name)
    assert profiled >= 3


def test_launch_constant_division_is_exact(tmp_path):
    """The kernels divide by n_tiles, split and the XCD count through
    host-made multipliers (Granlund-Montgomery); the host form of the same
    formula equals plain unsigned division on every divisor below 2^17 at
    the quotient boundaries and extremes, and on random 32-bit pairs."""
    here = os.path.dirname(os.path.abspath(__file__))
    exe = str(tmp_path / "fastdiv_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", exe, os.path.join(here, "fastdiv_check.cpp")], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout + r.stderr


def test_c_program_uses_the_abi(tmp_path):
    """tests/c_abi/abi_from_c.c, a C99 program, compiles against the header
    with -pedantic -Werror, links against libskinny.so and runs its host-only
    checks (argument errors before any device call, the tactic and table
    rules) without a GPU."""
    src = os.path.join(ROOT, "tests", "c_abi", "abi_from_c.c")
    exe = str(tmp_path / "abi_from_c")
    lib_dir = os.path.dirname(sk.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                    os.path.join(ROOT, "include"), src, "-o", exe, "-L", lib_dir, "-lskinny",
                    f"-Wl,-rpath,{lib_dir}"], check=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("abi ok "), run.stdout
    assert int(run.stdout.split()[2]) > 100


@pytest.mark.parametrize("value", ["garbage", "9.32.64.4.3", "9.32.64.4.3.2 ", "9.3.64.4.3.2",
                                   "2.1.1.1.1.1", "9.32.64.4.3.99"])
def test_forced_tactic_is_checked_before_any_device_call(monkeypatch, value):
    """SKINNY_FORCE_TACTIC is parsed with the table lines' strict syntax and
    checked like any tactic; a bad value is refused before the device is
    touched (with no GPU here, reaching the device would give
    SKINNY_ERR_DEVICE instead)."""
    monkeypatch.setenv("SKINNY_FORCE_TACTIC", value)
    st, plan = _prepare(0x1000, 6288, 7168)
    assert st == 1, (st, sk.last_error())
    assert plan.value is None
    assert sk.last_error()


def test_tune_command_checks_shapes_before_the_gpu():
    """python -m skinny_bf16_decode_amd.tune: shapes parse as NxK under the
    library's shape rules; a bad one is refused before the GPU is touched."""
    from skinny_bf16_decode_amd import tune
    assert tune.parse_shape("6288x7168") == (6288, 7168)
    assert tune.parse_shape("1X8") == (1, 8)
    for bad in ("6288", "6288x", "x7168", "6288x7169", "0x512", "64x0", "-1x8", "6288*7168", "1x2x3", "a x8"):
        with pytest.raises(ValueError):
            tune.parse_shape(bad)
    with pytest.raises(SystemExit) as e:
        tune.main(["--file", "/nonexistent/t.txt", "6288x7169"])
    assert e.value.code == 2
