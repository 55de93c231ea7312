"""Summaries of rocprofv3 output for the projection kernels.

    python -m skinny_bf16_decode_amd.profiling TRACE_DIR FETCH_CSV WRITE_CSV OUT_MD OUT_JSON \
        --command "..." --command "..."

Reads the kernel-trace statistics (``*_kernel_stats.csv``) and the per-dispatch
counter collections of a FETCH_SIZE run and a WRITE_SIZE run (KiB per
dispatch), and optionally of a MfmaUtil run and an SQ_INSTS_VALU_MFMA_MOPS_BF16
run (MFMA busy percent and MFMA operations per dispatch) and of one run of the
LDS and issue counters LDS_COUNTERS (LDS instructions, bank-conflict cycles,
waits for LDS issue and for anything as a share of wave time, vector-memory
reads, LDS data FIFO full cycles).  Counter values are scaled by the ratio of the known bytes of a
calibration kernel to what the counter reports for it: ``k_probe_read``
streams exactly 2*N*K bytes of one weight copy (FETCH_SIZE), and a 64 MiB
device-to-device copy writes exactly 64 MiB (WRITE_SIZE).  Writes a short
Markdown summary and a JSON record of HBM bytes per projection launch, keyed
by the SHA-256 of the kernel source so that a later kernel change voids it.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "csrc", "kernels.hip")


def kernel_source_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _short(name: str) -> str:
    return (name.replace("(skinny::KArgs)", "").replace("skinny::", "")
            .replace("void ", "").replace("unsigned int __vector(4) const*", "u32x4 const*"))


def load_counters(path):
    rows = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            rows[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return rows


# one --pmc pass: seven SQ counters (a pass may hold eight)
LDS_COUNTERS = ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY",
                "SQ_INSTS_VMEM_RD", "SQ_LDS_DATA_FIFO_FULL")


def load_counter_sets(path):
    """kernel -> counter -> per-dispatch values, from a run of several counters."""
    rows = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            rows[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return rows


def lds_table(path):
    """Markdown rows of the LDS and issue counters per kernel.  SQ_WAIT_INST_LDS,
    SQ_WAIT_ANY and SQ_WAVE_CYCLES are all wave quad-cycles, so their ratios
    are shares of wave time."""
    sets = load_counter_sets(path)
    out = ["| kernel | dispatches | LDS instructions | bank-conflict cycles per LDS instruction | "
           "waiting for LDS issue, % of wave time | waiting for anything, % of wave time | "
           "VMEM read instructions | LDS data FIFO full cycles |", "|---|---|---|---|---|---|---|---|"]
    for k in sorted(sets, key=_short):
        if not _ours(k):
            continue
        c = {n: statistics.mean(v) for n, v in sets[k].items()}
        lds, wave = c.get("SQ_INSTS_LDS", 0.0), c.get("SQ_WAVE_CYCLES", 0.0)
        conflict = c.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds if lds else float("nan")
        wait_lds = 100.0 * c.get("SQ_WAIT_INST_LDS", 0.0) / wave if wave else float("nan")
        wait_any = 100.0 * c.get("SQ_WAIT_ANY", 0.0) / wave if wave else float("nan")
        out.append(f"| `{_short(k)}` | {len(sets[k].get('SQ_INSTS_LDS', []))} | {lds:.3e} | {conflict:.3f} | "
                   f"{wait_lds:.1f} | {wait_any:.1f} | {c.get('SQ_INSTS_VMEM_RD', 0.0):.3e} | "
                   f"{c.get('SQ_LDS_DATA_FIFO_FULL', 0.0):.3e} |")
    return out


def load_stats(trace_dir):
    paths = glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))
    if not paths:
        raise FileNotFoundError(f"no kernel_stats.csv under {trace_dir}")
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def _ours(name: str) -> bool:
    return "k_dot2" in name or "k_mfma" in name or "k_rgs" in name


def summarize(trace_dir, fetch_csv, write_csv, weight_bytes, copy_bytes=64 << 20, fetch_scale=None):
    stats = load_stats(trace_dir)
    fetch = load_counters(fetch_csv)
    write = load_counters(write_csv)
    probe = [k for k in fetch if "k_probe_read" in k]
    copy = [k for k in write if "copyBuffer" in k or "copy" in k.lower()]
    if fetch_scale is None and probe:
        fetch_scale = weight_bytes / 1024.0 / statistics.mean(fetch[probe[0]])
    big_copy = [k for k in copy if max(write[k]) >= copy_bytes / 1024 * 0.5]
    write_scale = (copy_bytes / 1024.0 / max(write[big_copy[0]])) if big_copy else None
    kernels = {}
    for k in fetch:
        if _ours(k):
            f = statistics.mean(fetch[k]) * (fetch_scale or float("nan"))
            w = statistics.mean(write.get(k, [float("nan")])) * (write_scale or float("nan"))
            kernels[_short(k)] = {"fetch_kib": round(f, 1), "write_kib": round(w, 1),
                                  "dispatches": len(fetch[k])}
    return stats, kernels, fetch_scale, write_scale


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace_dir")
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("out_md")
    ap.add_argument("out_json")
    ap.add_argument("--weight-bytes", type=int, default=2 * 6288 * 7168)
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--title", default="skinny projection, 6288x7168 M sweep")
    ap.add_argument("--mfma-util", help="counter collection of a --pmc MfmaUtil run")
    ap.add_argument("--mfma-mops", help="counter collection of a --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 run")
    ap.add_argument("--lds", help="counter collection of a --pmc run of LDS_COUNTERS")
    ap.add_argument("--fetch-scale", type=float,
                    help="FETCH_SIZE scale factor taken from a larger weight's calibration, for a weight "
                         "that stays in L2 (its own plain read fetches next to nothing from HBM)")
    args = ap.parse_args()
    stats, kernels, fs, ws = summarize(args.trace_dir, args.fetch_csv, args.write_csv, args.weight_bytes,
                                       fetch_scale=args.fetch_scale)
    lines = [f"# {args.title}", "", "Commands (run from the repository root):", ""]
    lines += [f"    {c}" for c in args.command]
    lines += ["", "## Kernel trace statistics (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        n = _short(r["Name"])
        if _ours(n) or "k_probe" in n:
            lines.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    calib = (f"given, from a larger weight's k_probe_read calibration" if args.fetch_scale is not None
             else f"k_probe_read streams exactly {args.weight_bytes} B")
    lines += ["", "## HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
              f"FETCH_SIZE scale factor {fs:.4f} ({calib}); "
              f"WRITE_SIZE scale factor {ws:.4f} (64 MiB device copy).", "",
              "| kernel | dispatches | fetch KiB (scaled) | write KiB (scaled) |", "|---|---|---|---|"]
    for n, v in sorted(kernels.items()):
        lines.append(f"| `{n}` | {v['dispatches']} | {v['fetch_kib']:.1f} | {v['write_kib']:.1f} |")
    if args.mfma_util and args.mfma_mops:
        util, mops = load_counters(args.mfma_util), load_counters(args.mfma_mops)
        lines += ["", "## MFMA use (rocprofv3 --pmc MfmaUtil, then --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16)", "",
                  "MfmaUtil = 100 x sum of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs); "
                  "MFMA flops = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 (rows of a row group past N and "
                  "token columns past M are multiplied too).", "",
                  "| kernel | dispatches | MFMA busy % | MFMA flops per dispatch |", "|---|---|---|---|"]
        for k in sorted(util, key=_short):
            if _ours(k):
                lines.append(f"| `{_short(k)}` | {len(util[k])} | {statistics.mean(util[k]):.2f} | "
                             f"{statistics.mean(mops.get(k, [0.0])) * 512:.3e} |")
    if args.lds:
        lines += ["", "## LDS and issue (rocprofv3 --pmc " + " ".join(LDS_COUNTERS) + ")", "",
                  "Per dispatch, summed over the chip; the wait shares are wave quad-cycles over "
                  "SQ_WAVE_CYCLES.", ""]
        lines += lds_table(args.lds)
    os.makedirs(os.path.dirname(os.path.abspath(args.out_md)), exist_ok=True)
    with open(args.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    rec = {"kernel_source_sha256": kernel_source_sha(), "fetch_scale": fs, "write_scale": ws,
           "kernels": kernels}
    with open(args.out_json, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(args.out_md)


if __name__ == "__main__":
    main()
