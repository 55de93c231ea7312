"""Tune tactic tables on this GPU and append them to a table file.

    python -m skinny_bf16_decode_amd.tune --file tables.txt 6288x7168 3584x7168 [--in bf16|f16] [--out bf16|f32]

Each shape is prepared once with SKINNY_TABLE_CACHE naming the file. A shape
the file already holds for this chip (arch and CU count), input and output
type is loaded from it, not tuned. Any other shape is tuned on the current
GPU, which takes a few seconds, and its two tables (plain runs and runs with a
residual) are appended to the file. Later processes started with
SKINNY_TABLE_CACHE set to the same file then skip tuning. Start from a
fresh file to retune a shape the file already holds. The weight is random
(its values do not change the timings); the chosen kernel for a few token
counts is printed per shape.
"""
from __future__ import annotations

import argparse
import os
import sys
import time


def parse_shape(text: str) -> tuple:
    """'NxK' -> (N, K), with N >= 1, K >= 8 and K % 8 == 0 (the library's
    own shape rules, checked here before the GPU is touched)."""
    parts = text.lower().split("x")
    if len(parts) != 2 or not all(p.isdigit() for p in parts):
        raise ValueError(f"shape {text!r} is not NxK")
    n, k = int(parts[0]), int(parts[1])
    if n < 1 or k < 8 or k % 8:
        raise ValueError(f"shape {text!r}: N must be >= 1 and K a multiple of 8, at least 8")
    return n, k


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m skinny_bf16_decode_amd.tune", description=__doc__.split("\n")[0])
    ap.add_argument("--file", required=True, help="table file to load from and append to")
    ap.add_argument("--in", dest="in_dtype", choices=("bf16", "f16"), default="bf16", help="input type of W and x")
    ap.add_argument("--out", dest="out_dtype", choices=("bf16", "f32"), default="bf16", help="output type")
    ap.add_argument("shapes", nargs="+", help="weight shapes as NxK, e.g. 6288x7168")
    args = ap.parse_args(argv)
    try:
        shapes = [parse_shape(s) for s in args.shapes]
    except ValueError as e:
        ap.error(str(e))

    import torch
    import skinny_bf16_decode_amd as sk
    sk.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    in_dt = torch.float16 if args.in_dtype == "f16" else torch.bfloat16
    out_dt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    saved = os.environ.get("SKINNY_TABLE_CACHE")
    os.environ["SKINNY_TABLE_CACHE"] = os.path.abspath(args.file)
    try:
        for n, k in shapes:
            w = (torch.randn(n, k, device="cuda") * 0.02).to(in_dt)
            t0 = time.time()
            plan = sk.Prepared(w, out_dt)
            secs = time.time() - t0
            picks = "  ".join(f"M={m}: {plan.describe(m).split(' grid=')[0]}" for m in (1, 8, 16, 32, 64))
            print(f"{n}x{k} {args.in_dtype}->{args.out_dtype} ({secs:.1f} s): {picks}", flush=True)
            plan.close()
            del w
            torch.cuda.empty_cache()
    finally:
        if saved is None:
            os.environ.pop("SKINNY_TABLE_CACHE", None)
        else:
            os.environ["SKINNY_TABLE_CACHE"] = saved
    return 0


if __name__ == "__main__":
    sys.exit(main())
