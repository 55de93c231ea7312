"""The CPU oracle against its pins, the checker, and the input generator.

Runs on the CPU only.  Planted mistakes go into copies of the oracle's C
source, compiled here; the real oracle is never modified.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import skinny_inputs as si
from tests import oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(oracle_lib, pin):
    pin(oracle_lib)


# Plausible mistakes, each a single textual change to oracle.c.  Every one
# must make at least one pin fail.
MUTATIONS = {
    "dropped_last_term": ("for (int k = 0; k < K; ++k) {\n                        double p",
                          "for (int k = 0; k < K - 1; ++k) {\n                        double p"),
    "dropped_first_term": ("for (int k = 0; k < K; ++k) {\n                        double p",
                           "for (int k = 1; k < K; ++k) {\n                        double p"),
    "sign_flip": ("acc += p;\n                        mag", "acc -= p;\n                        mag"),
    "transposed_weight": ("wrow[k] = to_double(w[(long)n * K + k], f16);",
                          "wrow[k] = to_double(w[(long)k * N + n], f16);"),
    "f16_exponent_bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "f16_subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "f16_read_as_bf16": ("return f16 ? f16_to_double(bits) : bf16_to_double(bits);",
                         "return bf16_to_double(bits);"),
    "f16_sampled_ignores_type": ("double p = to_double(xr[k], f16) * to_double(wr[k], f16);",
                                 "double p = to_double(xr[k], 0) * to_double(wr[k], f16);"),
    "x_row_stride": ("const double *xr = xd + (long)m * K;",
                     "const double *xr = xd + (long)m;"),
    "output_transposed": ("o[(long)m * N + n] = acc;", "o[(long)n * M + m] = acc;"),
    "abs_sum_signed": ("mag += fabs(p);\n                    }", "mag += p;\n                    }"),
    "round_ties_away": ("if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))",
                        "if (rem >= 0.5)"),
    "round_truncate": ("if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))",
                       "if (0)"),
    "round_nine_bits": ("int q_exp = e - 8;", "int q_exp = e - 9;"),
    "decode_wrong_shift": ("uint32_t u = (uint32_t)bits << 16;\n    float f;",
                           "uint32_t u = (uint32_t)bits << 15;\n    float f;"),
    "sampled_skips_last": ("for (int k = 0; k < K; ++k) {\n            double p",
                           "for (int k = 0; k + 1 < K; ++k) {\n            double p"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutant_dir, name):
    old, new = MUTATIONS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    path = os.path.join(mutant_dir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib_path = os.path.join(mutant_dir, f"lib{name}.so")
    oracle.build(src=path, out=lib_path)
    lib = oracle.load(lib_path)
    failed = pins.run_all(lib)
    assert failed, f"no pin caught the planted mistake {name}"


# ---------------------------------------------------------------------------
# Checker
# ---------------------------------------------------------------------------

def test_checker_accepts_rounded_oracle(oracle_lib):
    for cid in (1, 4):
        o, s = oracle.gemm(si.activations(cid), si.weight(cid), lib=oracle_lib)
        assert oracle.check(o.astype(np.float32), o, s, "f32").ok
        bf = oracle.round_bf16(o, lib=oracle_lib)
        assert oracle.check(oracle.decode_bf16(bf, lib=oracle_lib), o, s, "bf16").ok


def test_checker_rejects_nan_and_big_error(oracle_lib):
    o, s = oracle.gemm(si.activations(1), si.weight(1), lib=oracle_lib)
    g = o.copy()
    g[0, 3] = np.nan
    assert not oracle.check(g, o, s, "f32").ok
    g = o.copy()
    g[0, 7] += 2e-3 * s[0, 7] + 1e-5
    rep = oracle.check(g, o, s, "f32")
    assert not rep.ok and rep.first_bad[0] == (0, 7)


def test_exact_probe_catches_dropped_chunk(oracle_lib):
    """On integer inputs any correct fp32 kernel is exact; a kernel that
    skipped one 16-byte (8-element) chunk of K is not."""
    x, w = si.small_int_case(21, 8, 64, 1024)
    o, _ = oracle.gemm(x, w, lib=oracle_lib)
    assert np.all(np.abs(o) < 2 ** 24)       # every partial sum exact in fp32
    w_bad = w.copy()
    w_bad[:, 8 * 37: 8 * 38] = 0              # one chunk dropped from every row
    o_bad, _ = oracle.gemm(x, w_bad, lib=oracle_lib)
    assert not np.array_equal(o_bad.astype(np.float32), o.astype(np.float32))


def test_tie_probe_values(oracle_lib):
    """The tie probe's exact sums are 257, 259, ...; nearest-even BF16 is
    256, 260, 260, 264, ... and truncation would give 256, 258, 260, ..."""
    x, w = si.tie_case(128, 512, m=2)
    o, _ = oracle.gemm(x, w, lib=oracle_lib)
    want = 257.0 + 2.0 * (np.arange(128) % 64)
    assert np.array_equal(o, np.broadcast_to(want, (2, 128)))
    bf = oracle.decode_bf16(oracle.round_bf16(o, lib=oracle_lib), lib=oracle_lib)
    expect_rne = np.array([256, 260, 260, 264, 264, 268], dtype=np.float64)
    assert np.array_equal(bf[0, :6], expect_rne)


def test_k_probe_closed_form(oracle_lib):
    x, w, cols, scales = si.k_probe_case(4, 3, 600, 1536)
    o, _ = oracle.gemm(x, w, lib=oracle_lib)
    xf = si.bf16_bits_to_f32(x).astype(np.float64)
    want = xf[:, cols] * scales.astype(np.float64)[None, :]
    assert np.array_equal(o, want)
    # coverage of the residues the probe promises
    assert set((cols % 512).tolist()) == set(range(512))


# ---------------------------------------------------------------------------
# Generator
# ---------------------------------------------------------------------------

def test_generator_deterministic_and_bf16_rounding():
    a = si.weight(1)
    b = si.weight(1)
    assert si.fingerprint(a) == si.fingerprint(b)
    assert si.fingerprint(si.weight(1, 0)) != si.fingerprint(si.draw(si.seed_for(1, 1, 1), (256, 512), ("uniform",)))
    # RNE on bit patterns: 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.5, 3.0], dtype=np.float32)
    assert si.f32_to_bf16_bits(v).tolist() == [0x3F80, 0x3F82, 0xBFC0, 0x4040]


def test_generator_distributions():
    w = si.bf16_bits_to_f32(si.draw(99, (512, 512), ("normal", 0.02)))
    assert abs(float(w.std()) - 0.02) < 0.001
    u = si.bf16_bits_to_f32(si.draw(98, (512, 512), ("uniform",)))
    assert float(u.min()) >= -1.0 and float(u.max()) <= 1.0
    assert abs(float(u.mean())) < 0.01


def test_generator_fingerprints_match_golden():
    """Input determinism across machines: the stored SHA-256 of each
    workload's first weight copy and activation block (written by
    tests/golden/make_fingerprints.py, which uses the generator only)."""
    import json
    path = os.path.join(os.path.dirname(__file__), "golden", "input_fingerprints.json")
    with open(path) as f:
        golden = json.load(f)
    for cid in (1, 4):
        assert si.fingerprint(si.weight(cid)) == golden[str(cid)]["weight0"]
        assert si.fingerprint(si.activations(cid)) == golden[str(cid)]["x"]


def test_thread_count_changes_nothing_but_speed():
    """set_threads only changes how many threads later calls use: the
    product and the magnitude sums are identical with one thread and with
    all of them."""
    all_threads = oracle.threads()
    w_bits, x_bits = si.weight(4), si.activations(4)
    try:
        oracle.set_threads(1)
        assert oracle.threads() == 1
        o1, s1 = oracle.gemm(x_bits[:8], w_bits)
    finally:
        oracle.set_threads(all_threads)
    assert oracle.threads() == all_threads
    o, s = oracle.gemm(x_bits[:8], w_bits)
    assert np.array_equal(o, o1) and np.array_equal(s, s1)


def test_block_seeded_integer_weight():
    """skinny_inputs.int_weight_blocks (the maximum-size GPU tests' weight):
    blocks tile the rows in order, each block is seeded on its own so
    int_weight_rows draws any rows again alone, and every entry is one of
    the given integers, exact in BF16."""
    n, k, be = 20, 300, 1000                             # 3 rows per block: six whole blocks and a ragged one
    assert si.int_block_rows(k, be) == 3 and si.int_block_rows(k) == (1 << 27) // k
    blocks = list(si.int_weight_blocks(11, n, k, (-1, 0, 1), be))
    assert [r0 for r0, _ in blocks] == list(range(0, n, 3))
    full = np.concatenate([b for _, b in blocks])
    assert full.shape == (n, k)
    assert set(np.unique(si.bf16_bits_to_f32(full))) == {-1.0, 0.0, 1.0}
    rows = [19, 0, 2, 3, 18, 5, 5]
    assert np.array_equal(si.int_weight_rows(11, n, k, rows, (-1, 0, 1), be), full[rows])
    other = np.concatenate([b for _, b in si.int_weight_blocks(12, n, k, (-1, 0, 1), be)])
    assert not np.array_equal(full, other)
    assert not np.array_equal(full[:3], full[3:6])     # blocks are drawn independently
    x = si.int_matrix(3, 4, 64)
    assert set(np.unique(si.bf16_bits_to_f32(x))) <= set(range(-3, 4))
