"""The library from a C program on the GPU: tests/c_abi/run_from_c (built
by __graft_entry__.build() from run_from_c.c) uses only the HIP runtime's C
API and include/skinny.h -- prepare with tuning, run at every M = 1..64,
a captured and replayed graph, and the allocation-free entry point with a
K-split tactic -- and checks every output bit against exact integer sums."""
from __future__ import annotations

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "run_from_c")


def test_c_program_prepares_runs_and_replays():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run __graft_entry__.build() first")
    print("[c abi] running tests/c_abi/run_from_c", flush=True)
    run = subprocess.run([EXE], capture_output=True, text=True, timeout=240)
    print(run.stdout[-2000:], run.stderr[-2000:], flush=True)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "c run ok " in run.stdout
