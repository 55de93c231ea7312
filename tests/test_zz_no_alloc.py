"""The allocation-free entry point skinny_run_static (through the C ABI)
against the plan entry point skinny_run_ex with the same tactic.

skinny_run_static takes the weight and one tactic instead of a plan and
exchanges split-K partials through a device array the library holds per GPU
(SKINNY_STATIC_SCRATCH_BYTES); nothing is allocated.  Two calls in a row --
the second on a smaller weight and fewer tokens -- must each give the same
bits as the plan run (same kernel, same reduction order), lie within the
stated bound of the CPU oracle, and leave rows >= M untouched; the second
call also shows that the first left every exchange node empty.
"""
from __future__ import annotations

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


def _one(sk, n, k, m, tactic, seed):
    import torch
    x_bits, w_bits = si.random_case(seed, 64, n, k)
    o, s = oracle.gemm(x_bits[:m], w_bits)
    w, x = gu.dev_bf16(w_bits), gu.dev_bf16(x_bits[:m])
    plan = sk.Prepared(w, torch.bfloat16, table=gu.forced_table(tactic))
    ref = gu.out_buffer(n, torch.bfloat16)
    plan.run(x, ref[:m])
    got = gu.out_buffer(n, torch.bfloat16)
    sk.run_static(w, tactic, x, got[:m])
    torch.cuda.synchronize()
    plan.close()
    assert gu.sentinel_intact(got, m), f"{tactic} M={m}: rows >= M were written"
    assert np.array_equal(gu.host_bits(got), gu.host_bits(ref)), f"{tactic} M={m}: differs from skinny_run_ex"
    rep = oracle.check(gu.values(got)[:m], o, s, "bf16")
    _say(f"  N={n} K={k} M={m} {tactic}: {rep}")
    assert rep.ok, rep


def test_static_run_matches_plan_run_twice(sk):
    # a two-way K split on the square decode shape (128 ranges x 2 parts,
    # 512 KiB of exchange nodes), then a smaller product with a three-way
    # split of a row-group stream kernel: both use the static scratch
    _one(sk, 3584, 7168, 32, sk.Tactic(sk.PATH_MFMAW, 32, 32, 4, 1, 2), 801)
    _one(sk, 1000, 4096, 13, sk.Tactic(sk.PATH_MFMA4, 16, 16, 2, 2, 3), 802)


def test_static_run_token_groups_and_one_stage(sk):
    # token groups: 3 groups of 16 tokens over 9 row tiles with an 8-way K
    # split, each (group, tile) with nodes of its own in the static scratch;
    # then the one-stage split-2 MFMAW the packed decode weight runs at M = 32
    _one(sk, 140, 7168, 40, sk.Tactic(sk.PATH_MFMAT, 64, 16, 4, 1, 8), 804)
    _one(sk, 6288, 7168, 32, sk.Tactic(sk.PATH_MFMAW, 32, 64, 4, 3, 2), 805)


def test_static_run_random_split_tactics(sk):
    """Seeded random shapes, each with a split-K tactic drawn from its own
    candidates, run through skinny_run_static and through a plan: the same
    bits, exact against the oracle on integer inputs, rows >= M untouched.
    The calls follow one another on the one static array, so each also
    shows that the previous left every exchange node empty."""
    import torch
    rng = np.random.default_rng(31)
    done = 0
    while done < 40:
        n = int(rng.integers(1, 2500))
        k = 8 * int(rng.integers(2, 600))
        split = [t for t in sk.enumerate_tactics(n, k) if t.split > 1]
        if not split:
            continue
        t = split[int(rng.integers(0, len(split)))]
        m = int(rng.integers(1, t.mt + 1))
        od = torch.float32 if done % 2 else torch.bfloat16
        x_bits, w_bits = si.small_int_case(90_000 + done, m, n, k)
        o, _ = oracle.gemm(x_bits, w_bits)
        w, x = gu.dev_bf16(w_bits), gu.dev_bf16(x_bits)
        got = gu.out_buffer(n, od)
        try:
            sk.run_static(w, t, x, got[:m])
        except ValueError as e:                 # an exchange larger than the static array
            assert "static scratch" in str(e), e
            continue
        plan = sk.Prepared(w, od, table=gu.forced_table(t))
        ref = gu.out_buffer(n, od)
        plan.run(x, ref[:m])
        torch.cuda.synchronize()
        plan.close()
        label = f"{n}x{k} M={m} {od} {t}"
        assert gu.sentinel_intact(got, m), f"{label}: rows >= M written"
        assert np.array_equal(gu.host_bits(got), gu.host_bits(ref)), f"{label}: differs from skinny_run_ex"
        want = o.astype(np.float32).view(np.uint32) if od == torch.float32 else oracle.round_bf16(o)
        assert np.array_equal(gu.host_bits(got)[:m], want), f"{label}: differs from the oracle"
        done += 1


def test_static_run_without_split_and_limits(sk):
    """No split: no scratch at all.  A tactic whose exchange would exceed the
    static scratch is refused before any launch."""
    import torch
    _one(sk, 640, 2048, 5, sk.Tactic(0, 8, 2, 2, 1, 1), 803)
    n, k = 7168, 18432
    w = torch.zeros((n, k), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((64, k), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((64, n), dtype=torch.bfloat16, device="cuda")
    big = sk.Tactic(sk.PATH_MFMAX, 64, 64, 4, 1, 8)       # 112 tiles x 7 nodes x 4096 values x 4 B
    with pytest.raises(ValueError, match="static scratch"):
        sk.run_static(w, big, x, out)
    with pytest.raises(ValueError):
        sk.run_static(w, sk.Tactic(0, 8, 2, 2, 1, 1), x[:9], out[:9])   # M above the tile
