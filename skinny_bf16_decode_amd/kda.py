"""The TP8 KDA decode projection with its two branches on two streams.

run_kda_projection_overlap on the page "vllm.models.kimi_k3.nvidia.
low_latency_gemm" runs, for hidden states [M, 7168], the QKVG projection of
the packed Q/K/V/G/F_A/beta/pad weight [6288, 7168] on the main stream and
"the F_A/beta then F_B branch" on an auxiliary stream, forked and joined
with two events.  The page does not print the row split of the packed
weight.  F_B's weight is [1536, 128], so F_A has 128 output rows; the reading
taken here is Q, K, V and G of 1536 rows each (rows 0..6143), F_A (rows
6144..6271), beta (rows 6272..6283, one per head of 128 dims) and 4 pad rows,
which adds up to 6288.  A contiguous row range of a packed [N, K] weight is
itself a packed [N', K] weight, so each branch is a plan on a row range.

The F_A/beta output is written with a row pitch of 144 elements (a multiple
of 8), so its first 128 columns -- F_A -- are a pitched [M, 128] view that F_B
reads directly as its x.  Every product runs in this package's kernels; torch
supplies the device memory, the streams and the events.

run_packed is a third schedule: one product over all 6288 packed rows (the
weight is packed so that one GEMM can serve every branch), then F_B reading
the F_A columns of that output as a pitched view (row pitch 6288).  Measured
on MI355X it is the fastest of the three: the two-stream fork mostly adds
the cost of the fork and join and takes CUs from the large product.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import Prepared

QKVG_ROWS = 4 * 1536
F_A_ROWS = 128
BETA_ROWS = 12
FAB_PITCH = 144       # >= F_A_ROWS + BETA_ROWS, a multiple of 8


@dataclass
class KdaOutputs:
    qkvg: object      # [M, 6144]
    fab: object       # [M, 140] view (row pitch 144): F_A then beta
    f_b: object       # [M, 1536]


class KdaProjection:
    """Plans for the three products of the KDA decode projection."""

    def __init__(self, packed_weight, f_b_weight, out_dtype=None, tables=None):
        import torch
        out_dtype = out_dtype or torch.bfloat16
        n, k = packed_weight.shape
        if n < QKVG_ROWS + F_A_ROWS + BETA_ROWS:
            raise ValueError(f"packed weight has {n} rows, fewer than Q/K/V/G + F_A + beta")
        if tuple(f_b_weight.shape) != (f_b_weight.shape[0], F_A_ROWS):
            raise ValueError(f"F_B weight must be [N, {F_A_ROWS}]")
        if out_dtype != torch.bfloat16:
            raise ValueError("F_B reads F_A's output as its input, so the outputs are BF16")
        tables = tables or {}
        self.k = k
        self.qkvg = Prepared(packed_weight[:QKVG_ROWS], out_dtype, table=tables.get("qkvg"))
        self.fab = Prepared(packed_weight[QKVG_ROWS:QKVG_ROWS + F_A_ROWS + BETA_ROWS], out_dtype,
                            table=tables.get("fab"))
        self.f_b = Prepared(f_b_weight, out_dtype, table=tables.get("f_b"))
        self.packed = Prepared(packed_weight, out_dtype, table=tables.get("packed"))
        self.out_dtype = out_dtype

    def outputs(self, m: int, device="cuda") -> KdaOutputs:
        import torch
        fab = torch.empty((m, FAB_PITCH), dtype=self.out_dtype, device=device)
        return KdaOutputs(torch.empty((m, QKVG_ROWS), dtype=self.out_dtype, device=device),
                          fab[:, :F_A_ROWS + BETA_ROWS],
                          torch.empty((m, self.f_b.n), dtype=self.out_dtype, device=device))

    def _aux_branch(self, x, out: KdaOutputs, stream):
        self.fab.run(x, out.fab, stream=stream)
        self.f_b.run(out.fab[:, :F_A_ROWS], out.f_b, stream=stream)

    def run(self, x, out: KdaOutputs, aux_stream, events):
        """Fork onto aux_stream after events[0], join back after events[1]."""
        import torch
        main = torch.cuda.current_stream()
        start, done = events
        start.record(main)
        aux_stream.wait_event(start)
        self.qkvg.run(x, out.qkvg, stream=main)
        self._aux_branch(x, out, aux_stream)
        done.record(aux_stream)
        main.wait_event(done)
        return out

    def run_serial(self, x, out: KdaOutputs):
        """The same three products one after another on the current stream."""
        import torch
        main = torch.cuda.current_stream()
        self.qkvg.run(x, out.qkvg, stream=main)
        self._aux_branch(x, out, main)
        return out

    def packed_outputs(self, m: int, device="cuda"):
        """([M, 6288] packed output, [M, 1536] F_B output) for run_packed."""
        import torch
        return (torch.empty((m, self.packed.n), dtype=self.out_dtype, device=device),
                torch.empty((m, self.f_b.n), dtype=self.out_dtype, device=device))

    def run_packed(self, x, packed_out, f_b_out):
        """One product over all packed rows, then F_B on its F_A columns."""
        import torch
        main = torch.cuda.current_stream()
        self.packed.run(x, packed_out, stream=main)
        self.f_b.run(packed_out[:, QKVG_ROWS:QKVG_ROWS + F_A_ROWS], f_b_out, stream=main)
        return packed_out, f_b_out

    def close(self):
        for p in (self.qkvg, self.fab, self.f_b, self.packed):
            p.close()
