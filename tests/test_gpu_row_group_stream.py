"""Parity of the row-group stream kernels -- MFMA4 (v_mfma_f32_4x4x4_16b,
path 10) and DOT2W (v_dot2_f32_bf16, path 11) -- with the CPU oracle, through
the C ABI.

Every compiled (tokens, row groups, stages in flight) instance is forced on a
weight whose equal row ranges fill all of its 4-row groups (a few ranges
short by a row), with K/8 = 129 chunks (eight whole 16-chunk stages and a
one-chunk tail), without a K split and with the atomic-swap exchange over two
and three K parts, on one and four waves (four waves over three-stage K parts
leave a wave with no stage).  Integer inputs make every fp32 partial sum
exact, so each output must equal the oracle bit for bit -- in whatever order
the MFMA blocks or chunk lanes, the waves and the K parts were added.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest

import oracle
import skinny_inputs as si
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# the compiled instances: (path, token tile, row groups, stages in flight)
ROW_GROUPS = (1, 2, 4, 7, 13, 14)
INSTANCES = ([(10, 4 * tg, rg, u) for u in (2, 3) for tg in (1, 2, 4) for rg in ROW_GROUPS]
             + [(10, 32, rg, u) for u in (2, 3) for rg in (1, 2, 4, 7)]
             + [(11, mt, rg, u) for u in (2, 3) for mt in (1, 2, 4) for rg in ROW_GROUPS]
             + [(11, 8, rg, u) for u in (2, 3) for rg in (1, 2, 4, 7)])
K_EXACT = 1032


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


def _cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def _filling_rows(rg, split):
    """N whose equal ranges (a whole multiple of CUs / split of them) hold
    4 RG rows, but for a few that hold one row less."""
    per_round = -(-_cus() // split)
    return per_round * 4 * rg - 3


def _dev(bits, dtype):
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


def _run_exact(sk, plan, x_bits, o, m, dtype, label):
    import torch
    out = gu.out_buffer(plan.n, plan.out_dtype)
    plan.run(_dev(x_bits[:m], dtype), out[:m])
    torch.cuda.synchronize()
    assert gu.sentinel_intact(out, m), f"{label}: rows >= M were written"
    got = gu.host_bits(out)[:m]
    want = o[:m].astype(np.float32).view(np.uint32) if plan.out_dtype == torch.float32 else oracle.round_bf16(o[:m])
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)[0]
        raise AssertionError(f"{label}: first mismatch at {tuple(bad)}: got {got[tuple(bad)]:#x} "
                             f"want {want[tuple(bad)]:#x} (exact {o[tuple(bad)]})")


@pytest.mark.parametrize("split", [1, 2, 3])
@pytest.mark.parametrize("rg", ROW_GROUPS)
def test_row_group_stream_every_instance_exact(sk, rg, split):
    import torch
    n, k = _filling_rows(rg, split), K_EXACT
    x_bits, w_bits = si.small_int_case(4000 + 10 * rg + split, 64, n, k)
    o, _ = oracle.gemm(x_bits, w_bits)
    assert np.all(np.abs(o) < 2 ** 24)
    w = _dev(w_bits, "bf16")
    for path, mt, rg_, u in INSTANCES:
        if rg_ != rg:
            continue
        for waves in (1, 4):
            t = sk.Tactic(path, mt, 4 * rg, waves, u, split)
            od = torch.bfloat16 if (mt + waves + u) % 2 else torch.float32
            _say(f"[rgs exact] N={n} K={k} {t} out={od}")
            plan = sk.Prepared(w, od, table=gu.forced_table(t))
            assert plan.tactic(t.mt) == t
            for m in sorted({1, max(1, t.mt - 3), t.mt}):
                for rep in range(2 if split > 1 else 1):   # the exchange nodes are left empty
                    _run_exact(sk, plan, x_bits, o, m, "bf16", f"{t} M={m} call {rep}")
            plan.close()


@pytest.mark.parametrize("split", [1, 2])
def test_row_group_stream_f16_every_instance_exact(sk, split):
    """The FP16 twins (v_mfma_f32_4x4x4_16b_f16, v_dot2_f32_f16) of every instance."""
    import torch
    for rg in ROW_GROUPS:
        n, k = _filling_rows(rg, split), K_EXACT
        x_bits, w_bits = si.small_int_case(4500 + 10 * rg + split, 64, n, k, dtype="f16")
        o, _ = oracle.gemm(x_bits, w_bits, dtype="f16")
        w = _dev(w_bits, "f16")
        for path, mt, rg_, u in INSTANCES:
            if rg_ != rg:
                continue
            t = sk.Tactic(path, mt, 4 * rg, 4, u, split)
            _say(f"[rgs f16 exact] N={n} {t}")
            plan = sk.Prepared(w, torch.float32, table=gu.forced_table(t))
            for m in sorted({max(1, t.mt - 3), t.mt}):
                _run_exact(sk, plan, x_bits, o, m, "f16", f"f16 {t} M={m}")
            plan.close()


def _tight(got, o, s, label):
    rep = oracle.check(got, o, s, "bf16")
    _say(f"  {label}: {rep}")
    assert rep.ok, f"{label}: {rep}"
    tight = 1e-4 * np.asarray(s) + 1e-6 + 2.0 ** -8 * np.abs(np.asarray(o))
    worst = float(np.max(np.abs(np.asarray(got) - np.asarray(o)) / tight))
    assert worst <= 1.0, f"{label}: error level above the fp32-accumulation expectation ({worst:.3f})"


@pytest.mark.parametrize("cid", [2, 3])
def test_row_group_stream_decode_weights_repeats_and_graph_replays(sk, cid):
    """The square [3584, 7168] and packed [6288, 7168] decode weights at full
    size with MFMA4 and DOT2W tactics with and without the swap exchange:
    within the bound against the whole oracle at the tile and at a ragged M,
    bitwise identical over repeats and over graph replays with eager work
    between them (the exchange nodes must be empty again after every call)."""
    import torch
    wl = si.WORKLOADS[cid]
    w_bits, x_bits = si.weight(cid, 0), si.activations(cid)
    t0 = time.time()
    o, s = oracle.gemm(x_bits, w_bits)
    _say(f"[rgs cfg{cid}] oracle {time.time() - t0:.1f}s")
    w, x = _dev(w_bits, "bf16"), _dev(x_bits, "bf16")
    A, D = sk.PATH_MFMA4, sk.PATH_DOT2W
    if cid == 3:     # 24-25 rows per CU; 49 with two K parts, 98 with four
        tactics = [sk.Tactic(A, 8, 28, 4, 3, 1), sk.Tactic(A, 16, 52, 2, 2, 2), sk.Tactic(A, 32, 28, 4, 2, 1),
                   sk.Tactic(A, 16, 28, 2, 3, 4), sk.Tactic(D, 4, 28, 4, 3, 1), sk.Tactic(D, 8, 28, 4, 2, 2)]
    else:            # 14 rows per CU; 28 with two K parts, 56 with four
        tactics = [sk.Tactic(A, 4, 16, 4, 3, 1), sk.Tactic(A, 16, 28, 4, 2, 2), sk.Tactic(A, 32, 28, 4, 3, 2),
                   sk.Tactic(A, 16, 56, 2, 2, 4), sk.Tactic(D, 2, 16, 4, 3, 1), sk.Tactic(D, 8, 28, 4, 2, 2)]
    for t in tactics:
        plan = sk.Prepared(w, torch.bfloat16, table=gu.forced_table(t))
        ms = (max(1, t.mt - 5), t.mt)
        ref = {}
        for m in ms:
            out = gu.out_buffer(wl.n, torch.bfloat16)
            plan.run(x[:m], out[:m])
            torch.cuda.synchronize()
            assert gu.sentinel_intact(out, m), f"{t} M={m}"
            ref[m] = gu.host_bits(out).copy()
            _tight(si.bf16_bits_to_f32(ref[m][:m]).astype(np.float64), o[:m], s[:m], f"cfg{cid} {t} M={m}")
            for _ in range(5):
                out2 = gu.out_buffer(wl.n, torch.bfloat16)
                plan.run(x[:m], out2[:m])
                torch.cuda.synchronize()
                assert np.array_equal(gu.host_bits(out2), ref[m]), f"{t} M={m}: repeat differs"
        outs = {m: gu.out_buffer(wl.n, torch.bfloat16) for m in ms}
        stream = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for m in ms:
                    plan.run(x[:m], outs[m][:m])
        for rep in range(10):
            for m in ms:
                outs[m][:m].fill_(0)          # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for m in ms:
                assert np.array_equal(gu.host_bits(outs[m]), ref[m]), (t, rep, m)
        del g
        plan.close()
