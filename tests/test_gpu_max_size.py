"""Weights at the library's size limit: N K just under 2^31 elements, 4.3 GB
of BF16.

  - wide, 65535 x 32768: row tiles ragged against every tile size;
  - long, 128 x 16773120: each row is 32 MiB, and the 64 rows of x reach the
    32-bit buffer offsets' limit (the same bound skinny_prepare_ex checks).

For every kernel family the candidate list offers at the shape, its
largest-tile, deepest-split tactic and its first unsplit one are forced and
run at their full token tile and at a ragged M.  Inputs are small integers
(the long weight's in {-1, 0, 1}), so every partial sum stays below 2^24 and
fp32 accumulation is exact in any order: sampled outputs must equal the
oracle bit for bit.  At full size every output row < M must hold finite
integers, and rows >= M keep their sentinel.  The weights come from
skinny_inputs' block-seeded integer generator, built and uploaded block by
block.
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

CASES = {
    "wide_65535x32768": (65535, 32768, (-3, -2, -1, 0, 1, 2, 3), 4096),
    "long_128x16773120": (128, 16773120, (-1, 0, 1), 64),
}


@pytest.fixture(scope="module")
def sk():
    import torch
    import skinny_bf16_decode_amd as lib
    lib.load_library()
    assert torch.cuda.is_available()
    return lib


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _pick(sk, n, k):
    """Per kernel family: the largest token tile with the deepest split, and
    the first unsplit candidate."""
    by_path = {}
    for t in sk.enumerate_tactics(n, k):
        by_path.setdefault(t.path, []).append(t)
    picks = []
    for path in sorted(by_path):
        ts = by_path[path]
        big = max(ts, key=lambda t: (t.mt, t.split, t.rows, t.waves))
        picks.append(big)
        first = next((t for t in ts if t.split == 1), None)
        if first is not None and repr(first) != repr(big):
            picks.append(first)
    return picks


@pytest.mark.parametrize("case", sorted(CASES))
def test_maximum_weight_size_exact(sk, case):
    import torch
    n, k, values, samples = CASES[case]
    assert n * k < 2 ** 31
    seed = 20261203 + n
    _say(f"[max size] {case}: generating and uploading {2 * n * k / 1e9:.2f} GB of weight")
    w_bits = np.empty((n, k), dtype=np.uint16)
    w_dev = torch.empty((n, k), dtype=torch.int16, device="cuda")
    for row0, bits in si.int_weight_blocks(seed, n, k, values):
        w_bits[row0:row0 + bits.shape[0]] = bits
        w_dev[row0:row0 + bits.shape[0]].copy_(torch.from_numpy(bits.view(np.int16)))
    w = w_dev.view(torch.bfloat16)
    x_bits = si.int_matrix(seed + 1, 64, k, values)
    x = gu.dev_bf16(x_bits)
    rng = np.random.default_rng(seed + 2)
    mi = rng.integers(0, 64, size=samples)
    ni = rng.integers(0, n, size=samples)
    _say(f"[max size] {case}: oracle at {samples} sampled outputs")
    want, _ = oracle.gemm_sampled(x_bits, w_bits, mi, ni)
    del w_bits
    paths = set()
    for t in _pick(sk, n, k):
        plan = sk.Prepared(w, torch.float32, table=gu.forced_table(t))
        for m in sorted({t.mt, t.mt // 2 + 1}):
            _say(f"[max size] {case}: {t} M={m}")
            out = gu.out_buffer(n, torch.float32)
            plan.run(x[:m], out[:m])
            torch.cuda.synchronize()
            assert gu.sentinel_intact(out, m), f"{case} {t} M={m}: rows >= M were written"
            got = out[:m].cpu().numpy()
            assert np.all(np.isfinite(got)) and np.array_equal(got, np.round(got)), \
                f"{case} {t} M={m}: an output is not a finite integer"
            sel = mi < m
            g = got[mi[sel], ni[sel]].astype(np.float64)
            bad = np.nonzero(g != want[sel])[0]
            assert bad.size == 0, (f"{case} {t} M={m}: {bad.size} of {sel.sum()} sampled outputs differ, "
                                   f"first ({mi[sel][bad[0]]}, {ni[sel][bad[0]]}): got {g[bad[0]]} "
                                   f"want {want[sel][bad[0]]}")
        plan.close()
        paths.add(t.path)
    _say(f"[max size] {case}: paths {sorted(paths)}")
    assert len(paths) >= 6
