"""Helpers for the GPU tests: moving BF16 bit arrays to and from the device,
running a plan, and the forced-tactic tables.  No arithmetic of the method."""
from __future__ import annotations

import numpy as np

import skinny_inputs as si

SENTINEL_BF16 = 0x7FBF        # a NaN pattern no correct kernel writes
SENTINEL_F32 = 0x7FBFBFBF

# Used for the token counts above a forced tactic's tile.
FALLBACK = (1, 64, 16, 1, 1, 1)   # mfma, mt=64, rows=16, waves=1, unroll=1, split=1


def torch():
    import torch as t
    return t


def dev_bf16(bits: np.ndarray):
    t = torch()
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return t.from_numpy(a).view(t.bfloat16).cuda()


def host_bits(tensor) -> np.ndarray:
    t = torch()
    if tensor.dtype == t.bfloat16:
        return tensor.view(t.int16).cpu().numpy().view(np.uint16)
    return tensor.view(t.int32).cpu().numpy().view(np.uint32)


def values(tensor) -> np.ndarray:
    """Decoded float64 values of a BF16 or fp32 device tensor."""
    t = torch()
    if tensor.dtype == t.bfloat16:
        return si.bf16_bits_to_f32(host_bits(tensor)).astype(np.float64)
    return tensor.cpu().numpy().astype(np.float64)


def out_buffer(n: int, out_dtype, rows: int = 64):
    """A [rows, n] output buffer prefilled with a sentinel bit pattern."""
    t = torch()
    if out_dtype == t.bfloat16:
        return t.full((rows, n), SENTINEL_BF16, dtype=t.int16, device="cuda").view(t.bfloat16)
    return t.full((rows, n), SENTINEL_F32, dtype=t.int32, device="cuda").view(t.float32)


def sentinel_intact(buf, m: int) -> bool:
    t = torch()
    bits = host_bits(buf)
    want = SENTINEL_BF16 if buf.dtype == t.bfloat16 else SENTINEL_F32
    return bool(np.all(bits[m:] == want))


def forced_table(tactic):
    """64-entry table: `tactic` for M <= its tile, a fixed MFMA tactic above."""
    import skinny_bf16_decode_amd as sk
    fb = sk.Tactic(*FALLBACK)
    return [tactic if m <= tactic.mt else fb for m in range(1, 65)]
