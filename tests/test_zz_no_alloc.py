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
