#!/usr/bin/env python3
"""Benchmark of the skinny BF16 decode projection on one MI355X.

One step is one pass of the whole hot path over the packed Q/K/V/G/F_A/beta
projection weight [6288, 7168]: six calls out[M, N] = x[M, K] @ W^T with
M = 1, 2, 4, 8, 16, 32 (BF16 out), each call on the next of 4 distinct weight
copies (360 MB, past the 256 MiB Infinity Cache), each resolving its kernel
through the plan's per-M table.  Steps are replayed from captured hipGraphs
of 16 steps (96 launches), as a captured decode forward pass would hold many
projections in one graph; inputs are resident in HBM before the timed region
starts.

Prints one JSON line on stdout:
  value = weight-stream GB/s over the timed steps (6 * 2NK bytes per step / time)
  roofline = the projection launches: algorithmic bytes (W + x + out) per
             launch / average launch time (HIP events on the replay stream),
             against the 8 TB/s HBM peak
  cpu_baseline = the fp64 CPU oracle on one step of the same workload
Diagnostics (per-M times, the plain read ceiling over the same rotated
weights, the empty-launch floor, parity of the last outputs) go to the JSON's
extra fields and to stderr.

The per-M tactic table is the one this library's tuner measured on an MI355X
(256 CUs) when the committed profiles were taken, shipped in
skinny_bf16_decode_amd/tables/ the way the pages ship measured per-part
tables; it is loaded through a temporary copy of that file.  A GPU with
another CU count finds no matching line and is tuned on the spot, and so is
every run with --retune.  SKINNY_TABLE_CACHE, when set, takes precedence.

  python bench.py [--steps K] [--warmup W] [--extra] [--no-cpu] [--retune] [--workload 2|3|5]

--workload times the M sweep of another decode weight instead (2: the square
[3584, 7168], 5: the long-K [7168, 18432]), with its own metric line and
counter record; 3, the packed [6288, 7168], is the headline.
"""
from __future__ import annotations

import argparse
import json
import os
import shutil
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
SHIPPED_TABLES = os.path.join(ROOT, "skinny_bf16_decode_amd", "tables", "mi355x_tuned.txt")
WORKLOAD = 3
M_SWEEP = (1, 2, 4, 8, 16, 32)   # the headline step (packed 6288x7168)
STEPS_PER_GRAPH = 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(bits):
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).cuda()


def bf16_values(t):
    import torch
    import skinny_inputs as si
    return si.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def capture(fn, stream):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            fn()
    return g


def time_graph(g, stream, reps):
    """Seconds for `reps` replays of g on `stream` (replays go to the current
    stream, so the events and the replays share `stream`)."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3


class Setup:
    """Weights, activations, outputs and plans of one workload."""

    def __init__(self, cid, copies=None, out_dtype="bf16"):
        import torch
        import skinny_inputs as si
        import skinny_bf16_decode_amd as sk
        self.wl = si.WORKLOADS[cid]
        self.cid = cid
        self.od = out_dtype
        self.copies = copies or self.wl.copies
        self.w_bits = [si.weight(cid, c) for c in range(self.copies)]
        self.x_bits = si.activations(cid)
        if self.x_bits.shape[0] < 64:
            self.x_bits = np.ascontiguousarray(np.resize(self.x_bits, (64, self.wl.k)))
        self.w = [dev_bf16(b) for b in self.w_bits]
        self.x = dev_bf16(self.x_bits)
        self.out_dtype = torch.float32 if out_dtype == "f32" else torch.bfloat16
        self.out = torch.zeros((self.copies, 64, self.wl.n), dtype=self.out_dtype, device="cuda")
        t0 = time.time()
        self.plans = [sk.Prepared(w, self.out_dtype) for w in self.w]
        self.prepare_s = time.time() - t0

    def run(self, call_index, m):
        c = call_index % self.copies
        self.plans[c].run(self.x[:m], self.out[c, :m])
        return c

    def per_m(self, stream, m, reps=10, min_s=5e-3):
        """µs per call at token count m, from a graph of 16 * copies calls
        replayed `reps` times -- or, for a graph that short replays finish in
        under `min_s` (the small weights), as many times as fill `min_s`, after
        a warm-up of a quarter of that, so that the timing does not catch the
        clocks between states."""
        calls = 16 * self.copies
        g = capture(lambda: [self.run(i, m) for i in range(calls)], stream)
        time_graph(g, stream, 1)
        dt = time_graph(g, stream, reps)
        if dt < min_s:
            reps = int(reps * min_s / max(dt, 1e-9)) + 1
            time_graph(g, stream, reps // 4 + 1)
            dt = time_graph(g, stream, reps)
        return 1e6 * dt / (reps * calls)


def algorithmic_bytes(n, k, m, out_bytes=2):
    return 2 * n * k + 2 * m * k + out_bytes * m * n


def read_ceiling(setup, stream, reps=10):
    import torch
    import skinny_bf16_decode_amd as sk
    sink = torch.zeros(sk.probe_read_blocks(), dtype=torch.float32, device="cuda")
    nbytes = setup.wl.weight_bytes
    calls = 16 * setup.copies

    def body():
        for i in range(calls):
            sk.probe_read(setup.w[i % setup.copies].data_ptr(), nbytes, sink.data_ptr())
    g = capture(body, stream)
    time_graph(g, stream, 1)
    dt = time_graph(g, stream, reps)
    us = 1e6 * dt / (reps * calls)
    return us, nbytes / us / 1e3


def empty_floor(stream, reps=20):
    import skinny_bf16_decode_amd as sk
    g = capture(lambda: [sk.probe_empty() for _ in range(64)], stream)
    time_graph(g, stream, 1)
    dt = time_graph(g, stream, reps)
    return 1e6 * dt / (reps * 64)


def cpu_baseline(setup):
    """The oracle on one step of the workload (its timed token counts on one
    weight copy), repeated until about 10 s of CPU time (at least 3 steps);
    GB/s of weight processed."""
    sweep = tuple(setup.wl.m_values)
    import oracle
    x = setup.x_bits
    w = setup.w_bits[0]
    reps, t_total = 0, 0.0
    while reps < 3 or (t_total < 10.0 and reps < 1000):
        t0 = time.perf_counter()
        for m in sweep:
            oracle.gemm(x[:m], w)
        t_total += time.perf_counter() - t0
        reps += 1
    step_s = t_total / reps
    gbps = len(sweep) * setup.wl.weight_bytes / step_s / 1e9
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"one full step ({len(sweep)} calls, M={list(sweep)}, one "
                      f"[{setup.wl.n},{setup.wl.k}] weight copy), {reps} rep(s), "
                      f"{step_s:.2f} s per step"}


def traffic_record_path(wl, od="bf16"):
    """The committed HBM traffic record of a workload's M sweep (BF16 output,
    or fp32 output with a _f32 suffix)."""
    suffix = "_f32" if od == "f32" else ""
    return os.path.join(ROOT, "profiles", f"skinny_projection_{wl.name}_msweep{suffix}.traffic.json")


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "skinny_projection_packed_qkvg_6288x7168_msweep.traffic.json")


def kernel_name(t):
    """The kernel instance a BF16 tactic launches, spelled as rocprofv3 lists it."""
    T, w = t.mt // 16, t.waves
    if t.path in (0, 8):                     # DOT2, DOT2R
        args = (t.mt, t.rows, t.unroll)
        name = "k_dot2"
    elif t.path == 1:                        # MFMA
        args, name = (T, t.rows // 16, t.unroll), "k_mfma"
    elif t.path == 12:                       # MFMAT: the 16-token MFMA kernel over token groups
        args, name = (1, t.rows // 16, t.unroll), "k_mfma"
    elif t.path == 3:                        # MFMAX: unroll picks the grid, not the kernel
        args, name = (T, w), "k_mfmax"
    elif t.path == 9:                        # MFMAW: row groups, waves, stage chunks, stages in flight
        sc, depth = (16 if t.unroll in (2, 4) else 8), (2 if t.unroll <= 2 else 1)
        args, name = (T, t.rows // 16, w, sc, depth), "k_mfmaw"
    elif t.path == 10:                       # MFMA4: token groups and row groups of 4, stages in flight
        args, name = ("true", t.mt // 4, t.rows // 4, t.unroll), "k_rgs"
    elif t.path == 11:                       # DOT2W: tokens, row groups of 4, stages in flight
        args, name = ("false", t.mt, t.rows // 4, t.unroll), "k_rgs"
    else:
        return None
    return f"{name}<{', '.join(str(a) for a in args)}, false>"


def counted_traffic(setup):
    """HBM bytes per launch over the step, from the committed rocprofv3 counter
    record -- only if it was taken on this exact kernel source and covers every
    kernel the step uses; otherwise None."""
    sweep = tuple(setup.wl.m_values)
    import json as _json
    from skinny_bf16_decode_amd import profiling
    record = traffic_record_path(setup.wl, setup.od)
    if not os.path.exists(record):
        return None
    with open(record) as f:
        rec = _json.load(f)
    if rec.get("kernel_source_sha256") != profiling.kernel_source_sha():
        return None
    total = 0.0
    for m in sweep:
        name = kernel_name(setup.plans[0].tactic(m))
        k = rec["kernels"].get(name) if name else None
        if k is None:
            return None
        total += (k["fetch_kib"] + k["write_kib"]) * 1024.0
    return total / len(sweep)


def parity_of_last(setup, last_copy, m, samples=4096):
    import oracle
    rng = np.random.default_rng(2024)
    mi = rng.integers(0, m, size=samples)
    ni = rng.integers(0, setup.wl.n, size=samples)
    o, s = oracle.gemm_sampled(setup.x_bits, setup.w_bits[last_copy], mi, ni)
    if setup.od == "f32":
        got = setup.out[last_copy].cpu().numpy().astype(np.float64)[mi, ni]
    else:
        got = bf16_values(setup.out[last_copy])[mi, ni]
    rep = oracle.check(got, o, s, setup.od)
    return rep


def use_tables(retune, cus, wl, od="bf16"):
    """Point SKINNY_TABLE_CACHE at a temporary copy of the shipped tables
    (unless the caller set it, or asked to retune); say where the timed
    shape's table comes from."""
    global _OWN_TABLE_COPY
    if os.environ.get("SKINNY_TABLE_CACHE") and not _OWN_TABLE_COPY:
        return f"SKINNY_TABLE_CACHE={os.environ['SKINNY_TABLE_CACHE']}"
    if retune:
        return "tuned on this GPU (--retune)"
    if not _OWN_TABLE_COPY:
        fd, path = tempfile.mkstemp(prefix="skinny_tables_", suffix=".txt")
        os.close(fd)
        shutil.copyfile(SHIPPED_TABLES, path)
        os.environ["SKINNY_TABLE_CACHE"] = path
        _OWN_TABLE_COPY = path
    with open(SHIPPED_TABLES) as f:
        key = ["skinny-table", "v2", "gfx950", str(cus), str(wl.n), str(wl.k), "bf16", od]
        if any(line.split()[:8] == key for line in f):
            return f"shipped ({os.path.relpath(SHIPPED_TABLES, ROOT)}, {cus} CUs)"
    return f"tuned on this GPU (no shipped table for {cus} CUs)"


_OWN_TABLE_COPY = None
SECOND_MIN_STEPS, SECOND_MIN_WARMUP = 200, 32   # the 3584x7168 sweep beside the headline


def time_workload(setup, stream, steps, warmup, per_m_reps):
    """Time `steps` steps of the workload's M sweep (graphs of STEPS_PER_GRAPH
    steps, HIP events on `stream`), check the last call's output, and take
    the per-M times, the read ceiling and the empty-launch floor."""
    import torch
    wl = setup.wl
    sweep = tuple(wl.m_values)
    for m in sweep:
        log(f"  {wl.name} M={m:2d}: {setup.plans[0].describe(m)}")
    # Graphs of one step and of STEPS_PER_GRAPH consecutive steps, one per
    # starting copy offset: a captured decode forward pass holds many
    # projections in one graph, so the time between graph launches is spread
    # over 16 steps rather than paid by every step.  Each step is the same
    # calls either way; `steps` steps are exactly that many steps.
    calls = len(sweep)
    offsets = sorted({(calls * s) % setup.copies for s in range(setup.copies)})
    graphs, big = {}, {}
    for off in offsets:
        graphs[off] = capture(lambda off=off: [setup.run(off + j, m) for j, m in enumerate(sweep)], stream)
        big[off] = capture(lambda off=off: [setup.run(off + j, sweep[j % calls])
                                            for j in range(calls * STEPS_PER_GRAPH)], stream)

    def replay_steps(first, count):
        i = first
        while i < first + count:
            off = (calls * i) % setup.copies
            if first + count - i >= STEPS_PER_GRAPH:
                big[off].replay()
                i += STEPS_PER_GRAPH
            else:
                graphs[off].replay()
                i += 1

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):        # replays, and the events, on `stream`
        replay_steps(0, warmup)
        torch.cuda.synchronize()
        e0.record(stream)
        t0 = time.perf_counter()
        replay_steps(warmup, steps)
        e1.record(stream)
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    elapsed = e0.elapsed_time(e1) / 1e3
    ms_per_step = 1e3 * elapsed / steps
    value = calls * wl.weight_bytes * steps / elapsed / 1e9
    us_per_launch = 1e6 * elapsed / (calls * steps)
    log(f"{wl.name}: timed {steps} steps: {ms_per_step * 1e3:.2f} us/step, {us_per_launch:.2f} us/call, "
        f"{value:.1f} GB/s weight stream ({100 * value / PEAK_GBPS:.1f}% of 8 TB/s); host wall {wall:.3f}s")
    # the last call of the last step
    last_copy = (calls * (warmup + steps) - 1) % setup.copies
    rep = parity_of_last(setup, last_copy, sweep[-1])
    log(f"parity of the last call (M={sweep[-1]}, copy {last_copy}): {rep}")
    if not rep.ok:
        print(f"parity failure ({wl.name}): {rep}", file=sys.stderr)
        sys.exit(3)
    per_m = {}
    for m in sweep:
        us = setup.per_m(stream, m, reps=per_m_reps)
        gb = wl.weight_bytes / us / 1e3
        per_m[str(m)] = {"us_per_call": round(us, 3), "weight_gbps": round(gb, 1),
                         "pct_peak": round(100 * gb / PEAK_GBPS, 1)}
        log(f"  {wl.name} M={m:2d}: {us:7.2f} us/call  {gb:7.1f} GB/s  {100 * gb / PEAK_GBPS:5.1f}%")
    ceil_us, ceil_gb = read_ceiling(setup, stream)
    floor_us = empty_floor(stream)
    log(f"{wl.name}: read ceiling (plain nt stream of the same rotated weights): {ceil_us:.2f} us, "
        f"{ceil_gb:.1f} GB/s; empty-launch floor {floor_us:.2f} us")
    return {"value": value, "ms_per_step": ms_per_step, "us_per_launch": us_per_launch, "per_m": per_m,
            "read_ceiling_gbps": ceil_gb, "read_ceiling_us": ceil_us, "empty_launch_us": floor_us}


def summary(setup, res, table_source):
    """The JSON fields of one timed workload: per-M times, the step's
    roofline (algorithmic bytes per launch / average launch time against the
    8 TB/s peak, and the counted HBM traffic per launch when the committed
    record matches this kernel source), read ceiling and launch floor."""
    wl = setup.wl
    sweep = tuple(wl.m_values)
    out_bytes = 4 if setup.od == "f32" else 2
    algo = sum(algorithmic_bytes(wl.n, wl.k, m, out_bytes) for m in sweep) / len(sweep)
    achieved = algo / res["us_per_launch"] / 1e3
    traffic = counted_traffic(setup)
    if traffic is not None:
        traffic = round(traffic)
        log(f"{wl.name}: counted HBM traffic per launch: {traffic} B (algorithmic {round(algo)} B)")
    return {
        "workload": f"{wl.name} [{wl.n}, {wl.k}], M in {list(sweep)}, {setup.copies} rotated weight copies",
        "us_per_call": round(res["us_per_launch"], 3),
        "pct_of_peak": round(100 * res["value"] / PEAK_GBPS, 1),
        "weight_gbps": round(res["value"], 1),
        "per_m": res["per_m"],
        "read_ceiling_gbps": round(res["read_ceiling_gbps"], 1),
        "read_ceiling_us": round(res["read_ceiling_us"], 3),
        "empty_launch_us": round(res["empty_launch_us"], 3),
        "parity_last_call": "ok",
        "tactic_table": table_source,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "skinny projection launches of the step (the per-M table's kernels)",
                     "bytes_per_launch": round(algo), "us_per_launch": round(res["us_per_launch"], 3)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--extra", action="store_true", help="also time the other workloads (stderr)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--per-m-reps", type=int, default=10, help="graph replays per token count")
    ap.add_argument("--calibrate", action="store_true",
                    help="also launch a plain read of one weight copy and a 64 MiB device copy, "
                         "whose known byte counts scale the HBM traffic counters")
    ap.add_argument("--retune", action="store_true",
                    help="tune the tactic tables on this GPU instead of loading the shipped ones")
    ap.add_argument("--workload", type=int, default=WORKLOAD, choices=(1, 2, 3, 4, 5),
                    help="the weight whose M sweep is timed (3, the packed 6288x7168, is the headline)")
    ap.add_argument("--out-dtype", choices=("bf16", "f32"), default="bf16",
                    help="output type of the timed sweep (the headline is BF16)")
    ap.add_argument("--no-second", action="store_true",
                    help="skip the square 3584x7168 sweep reported beside the headline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the projection would shard W by rows, one shard per GPU, with no exchange "
              "inside the GEMM); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import skinny_bf16_decode_amd as sk
    sk.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count} "
        f"torch={torch.__version__} hip={torch.version.hip}")
    import skinny_inputs as si
    sweep = tuple(si.WORKLOADS[args.workload].m_values)
    table_source = use_tables(args.retune, props.multi_processor_count, si.WORKLOADS[args.workload],
                              args.out_dtype)
    log(f"tactic table: {table_source}")

    setup = Setup(args.workload, out_dtype=args.out_dtype)
    wl = setup.wl
    log(f"workload {wl.name}: prepare {setup.prepare_s:.2f}s")
    stream = torch.cuda.Stream()
    res = time_workload(setup, stream, args.steps, args.warmup, args.per_m_reps)
    if args.calibrate:
        calibration_kernels(setup, stream)
    if args.extra:
        extra_workloads(stream)
        oracle_small_workloads()
    # the other target weight: the square [3584, 7168] sweep from its shipped
    # table, reported beside the headline (not part of `value`)
    other = None
    if args.workload == WORKLOAD and not args.no_second:
        table_source2 = use_tables(args.retune, props.multi_processor_count, si.WORKLOADS[2])
        log(f"tactic table (square weight): {table_source2}")
        setup2 = Setup(2)
        # its own step count: a handful of steps of a 64 µs step mostly
        # measures the first replays of freshly captured graphs
        steps2, warmup2 = max(args.steps, SECOND_MIN_STEPS), max(args.warmup, SECOND_MIN_WARMUP)
        res2 = time_workload(setup2, stream, steps2, warmup2, args.per_m_reps)
        other = summary(setup2, res2, table_source2)
        other.update({"steps": steps2, "warmup": warmup2})
        del setup2
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(setup)
        log(f"cpu baseline: {cpu}")

    line = {
        "metric": ("µs/call and weight-stream HBM GB/s (% of peak), 6288x7168 at M=1..32"
                   if args.workload == WORKLOAD else
                   f"µs/call and weight-stream HBM GB/s (% of peak), {wl.n}x{wl.k} at M={sweep[0]}..{sweep[-1]}"),
        "value": round(res["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: out[M,N] = x[M,K] @ W[N,K]^T, N={wl.n}, K={wl.k}, "
                               f"one step = M in {list(sweep)}, BF16 in, "
                               f"{'fp32' if args.out_dtype == 'f32' else 'BF16'} out, fp32 accumulate, "
                               f"{setup.copies} rotated weight copies, hipGraph replay",
                   "N": wl.n, "K": wl.k, "m_values": list(sweep), "weight_copies": setup.copies},
    }
    main_summary = summary(setup, res, table_source)
    line.update({k: v for k, v in main_summary.items() if k not in ("workload",)})
    line["cpu_baseline"] = cpu
    if other is not None:
        line["square_3584x7168"] = other
    print(json.dumps(line), flush=True)


def calibration_kernels(setup, stream):
    """Kernels of known traffic for scaling rocprofv3's FETCH_SIZE/WRITE_SIZE:
    k_probe_read reads exactly 2NK bytes of one weight copy; torch's copy
    reads and writes 64 MiB."""
    import torch
    import skinny_bf16_decode_amd as sk
    sink = torch.zeros(sk.probe_read_blocks(), dtype=torch.float32, device="cuda")
    src = torch.ones(16 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        sk.probe_read(setup.w[1 % setup.copies].data_ptr(), setup.wl.weight_bytes, sink.data_ptr())
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration: probe_read of {setup.wl.weight_bytes} B, device copy of {src.numel() * 4} B")


def kda_overlap(stream):
    """The KDA decode projection (packed [6288, 7168] QKVG on the main stream,
    F_A/beta then F_B [1536, 128] on an auxiliary stream) against the same
    three products on one stream, each from a graph of 16 projections over 4
    rotated packed-weight copies."""
    import torch
    import skinny_inputs as si
    from skinny_bf16_decode_amd.kda import KdaProjection
    copies = 4
    f_b = dev_bf16(si.weight(4))
    packed = [dev_bf16(si.weight(3, c)) for c in range(copies)]
    x = dev_bf16(si.activations(3))
    projs = [KdaProjection(w, f_b) for w in packed]
    aux = torch.cuda.Stream()
    events = [(torch.cuda.Event(), torch.cuda.Event()) for _ in range(16 * copies)]
    for m in (1, 4, 8, 16, 32):
        outs = [p.outputs(m) for p in projs]

        def overlapped():
            for i in range(16 * copies):
                projs[i % copies].run(x[:m], outs[i % copies], aux, events[i])

        def serial():
            for i in range(16 * copies):
                projs[i % copies].run_serial(x[:m], outs[i % copies])

        pouts = [p.packed_outputs(m) for p in projs]

        def packed():
            for i in range(16 * copies):
                projs[i % copies].run_packed(x[:m], *pouts[i % copies])

        res = {}
        for name, fn in (("serial", serial), ("overlapped", overlapped), ("packed", packed)):
            g = capture(fn, stream)
            time_graph(g, stream, 1)
            res[name] = 1e6 * time_graph(g, stream, 10) / (10 * 16 * copies)
        log(f"[kda projection] M={m:2d}: three products on one stream {res['serial']:7.2f} us, "
            f"F_A/beta->F_B on a second stream {res['overlapped']:7.2f} us, "
            f"one packed product then F_B {res['packed']:7.2f} us per projection")
    for p in projs:
        p.close()


def extra_workloads(stream):
    import skinny_inputs as si
    kda_overlap(stream)
    for cid, od in ((2, "bf16"), (4, "f32"), (4, "bf16"), (5, "bf16"), (1, "f32")):
        s = Setup(cid, out_dtype=od)
        for m in s.wl.m_values:
            us = s.per_m(stream, m)
            gb = s.wl.weight_bytes / us / 1e3
            log(f"[{s.wl.name} {od}] M={m:2d}: {us:7.2f} us/call {gb:7.1f} GB/s "
                f"{100 * gb / PEAK_GBPS:5.1f}% | {s.plans[0].describe(m)}")
        del s
        import torch
        torch.cuda.empty_cache()


def oracle_small_workloads():
    """The CPU oracle on the tiny and short-K workloads at each timed M, with
    all of the host's threads and with one (min of 3 runs after 5 untimed
    ones): baselines only, printed next to the GPU lines."""
    import oracle
    import skinny_inputs as si
    all_threads = oracle.threads()
    for cid in (1, 4):
        wl = si.WORKLOADS[cid]
        w_bits, x_bits = si.weight(cid), si.activations(cid)
        for m in wl.m_values:
            res = []
            for t in (all_threads, 1):
                oracle.set_threads(t)
                for _ in range(5):             # untimed: the first calls after a team change start threads
                    oracle.gemm(x_bits[:m], w_bits)
                best = None
                for _ in range(3):
                    t0 = time.perf_counter()
                    oracle.gemm(x_bits[:m], w_bits)
                    dt = time.perf_counter() - t0
                    best = dt if best is None else min(best, dt)
                res.append(f"{t} thread(s) {best * 1e3:8.3f} ms/call {wl.weight_bytes / best / 1e9:7.3f} GB/s")
            log(f"[oracle {wl.name}] M={m:2d}: " + ", ".join(res))
    oracle.set_threads(all_threads)


if __name__ == "__main__":
    main()
