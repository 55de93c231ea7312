"""The host-only C++ of the library (tactic legality and enumeration, the
table rule, the stored-table parser, the launch-constant division) built with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/host/check_host.cpp: enumeration at int-range extreme shapes and CU
counts, 200k tactics of arbitrary fields, and table-file lines that are
truncated, over-long, out of int range, binary or otherwise malformed.  No HIP
and no GPU: the kernel instance list is expanded into entries without kernels.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "skinny_bf16_decode_amd", "csrc")


def test_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = tmp_path / "check_host"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "check_host.cpp"),
           os.path.join(CSRC, "tactics.cpp"), os.path.join(CSRC, "tables.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe), str(tmp_path)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "host checks ok" in r.stdout, f"{r.stdout}\n{r.stderr}"
    assert "runtime error" not in r.stderr, r.stderr
