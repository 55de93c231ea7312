"""Python binding of libskinny.so, the MI355X skinny BF16 decode projection.

    out[M, N] = x[M, K] @ W[N, K]^T,   M = 1..64

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/skinny.h).  PyTorch supplies device memory
and streams.  There is no fallback: if the library is missing or the device is
not gfx950, calls raise.

    plan = Prepared(W)                 # W: torch.bfloat16 [N, K] on cuda
    plan.run(x, out)                   # x: bf16 [M, K]; out: bf16/f32 [M, N]

Errors follow the pages' wrappers: bad arguments raise ValueError (as
PreparedWarpSplitK / PreparedProjection do), HIP failures RuntimeError, and an
unsupported token count raises UnsupportedTokens (the pages' selectors return
None so the caller falls back).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskinny.so")

MAX_M = 64
OUT_BF16 = 0
OUT_F32 = 1
IN_BF16 = 0
IN_F16 = 1
PATH_DOT2 = 0
PATH_MFMA = 1
PATH_MFMAX = 3
PATH_DOT2R = 8
PATH_MFMAW = 9
PATH_MFMA4 = 10
PATH_DOT2W = 11
PATH_MFMAT = 12
PATH_NAMES = {0: "dot2", 1: "mfma", 2: "dot2x", 3: "mfmax", 4: "mfmad", 5: "mfmas", 6: "mfmar", 7: "mfmak",
              8: "dot2r", 9: "mfmaw", 10: "mfma4", 11: "dot2w", 12: "mfmat"}

STATUS = {
    0: "SKINNY_OK",
    1: "SKINNY_ERR_INVALID_ARG",
    2: "SKINNY_ERR_SHAPE",
    3: "SKINNY_ERR_ALIGN",
    4: "SKINNY_ERR_UNSUPPORTED_M",
    5: "SKINNY_ERR_DEVICE",
    6: "SKINNY_ERR_NOMEM",
    7: "SKINNY_ERR_HIP",
}


class SkinnyError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class UnsupportedTokens(ValueError):
    """M outside 1..64: the caller should fall back to another GEMM."""


class Tactic(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("mt", ctypes.c_int), ("rows", ctypes.c_int),
                ("waves", ctypes.c_int), ("unroll", ctypes.c_int), ("split", ctypes.c_int)]

    def astuple(self):
        return (self.path, self.mt, self.rows, self.waves, self.unroll, self.split)

    def __repr__(self):
        p = PATH_NAMES.get(self.path, str(self.path))
        return (f"Tactic({p}, mt={self.mt}, rows={self.rows}, waves={self.waves}, "
                f"unroll={self.unroll}, split={self.split})")

    def __eq__(self, other):
        return isinstance(other, Tactic) and self.astuple() == other.astuple()

    def __hash__(self):
        return hash(self.astuple())


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libskinny.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m skinny_bf16_decode_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    planp = ctypes.c_void_p
    tp = ctypes.POINTER(Tactic)
    sig = {
        "skinny_prepare": (i, [vp, i, i, i, ctypes.POINTER(planp)]),
        "skinny_prepare_tactics": (i, [vp, i, i, i, tp, ctypes.POINTER(planp)]),
        "skinny_prepare_ex": (i, [vp, i, i, i, i, i, ctypes.POINTER(planp)]),
        "skinny_prepare_tactics_ex": (i, [vp, i, i, i, i, i, tp, ctypes.POINTER(planp)]),
        "skinny_run": (i, [planp, vp, vp, i, vp]),
        "skinny_run_ex": (i, [planp, vp, i, vp, i, vp, i, i, vp]),
        "skinny_supports": (i, [planp, i]),
        "skinny_plan_tactic": (i, [planp, i, tp]),
        "skinny_describe": (i, [planp, i, ctypes.c_char_p, sz]),
        "skinny_destroy": (None, [planp]),
        "skinny_status_string": (ctypes.c_char_p, [i]),
        "skinny_last_error": (ctypes.c_char_p, []),
        "skinny_tactic_check": (i, [tp, i, i]),
        "skinny_enumerate_tactics": (i, [i, i, tp, i]),
        "skinny_enumerate_tactics_ex": (i, [i, i, i, tp, i]),
        "skinny_select_table": (i, [tp, ctypes.POINTER(ctypes.c_double), i, tp]),
        "skinny_run_static": (i, [vp, i, i, i, i, i, tp, vp, i, vp, i, vp, i, i, vp]),
        "skinny_probe_read": (i, [vp, sz, vp, vp]),
        "skinny_probe_read_blocks": (i, []),
        "skinny_probe_empty": (i, [vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().skinny_last_error().decode()


def _raise(status: int):
    if status == 0:
        return
    msg = last_error()
    if status == 4:
        raise UnsupportedTokens(msg)
    if status in (1, 2, 3):
        raise ValueError(f"{STATUS[status]}: {msg}")
    raise SkinnyError(status, msg)


def tactic_check(t: Tactic, n: int, k: int) -> None:
    _raise(load_library().skinny_tactic_check(ctypes.byref(t), n, k))


def enumerate_tactics(n: int, k: int, cus: int = 256) -> list:
    """The candidates the tuner times for an [n, k] weight on a device with `cus` CUs."""
    lib = load_library()
    count = lib.skinny_enumerate_tactics_ex(n, k, cus, None, 0)
    if count < 0:
        raise ValueError(f"bad shape N={n} K={k} or CU count {cus}")
    buf = (Tactic * count)()
    lib.skinny_enumerate_tactics_ex(n, k, cus, buf, count)
    return [Tactic(*t.astuple()) for t in buf]


def select_table(cands, times_us) -> list:
    """The per-M table rule: fastest candidate whose token tile covers M."""
    lib = load_library()
    n = len(cands)
    arr = (Tactic * max(n, 1))(*[Tactic(*c.astuple()) for c in cands])
    tm = (ctypes.c_double * max(n, 1))(*times_us)
    out = (Tactic * MAX_M)()
    _raise(lib.skinny_select_table(arr, tm, n, out))
    return [Tactic(*t.astuple()) for t in out]


def _stream_handle(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream))


def probe_read(buf_ptr: int, nbytes: int, sink_ptr: int, stream=None) -> None:
    """Measurement only: stream nbytes from buf with 16-byte nontemporal loads."""
    _raise(load_library().skinny_probe_read(ctypes.c_void_p(buf_ptr), nbytes,
                                            ctypes.c_void_p(sink_ptr), _stream_handle(stream)))


def probe_read_blocks() -> int:
    return load_library().skinny_probe_read_blocks()


def probe_empty(stream=None) -> None:
    """Measurement only: one empty launch."""
    _raise(load_library().skinny_probe_empty(_stream_handle(stream)))


STATIC_SCRATCH_BYTES = 4 << 20   # SKINNY_STATIC_SCRATCH_BYTES


def run_static(weight, tactic: Tactic, x, out, stream=None, residual=None, out_dtype=None):
    """out[:M] = x @ weight^T (+ residual[:M]) with one given tactic and no
    plan: skinny_run_static, which allocates nothing (its split-K exchange
    uses a device array the library holds per GPU).  Tensors as for
    Prepared.run; out's dtype (BF16 or fp32) selects the output type."""
    import torch
    lib = load_library()
    out_dtype = out.dtype if out_dtype is None else out_dtype
    od = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    idt = IN_F16 if weight.dtype == torch.float16 else IN_BF16
    n, k = weight.shape
    m = x.shape[0]
    ldx = x.stride(0) if m > 1 else k
    ldo = out.stride(0) if out.shape[0] > 1 else n
    ldr = (residual.stride(0) if residual.shape[0] > 1 else n) if residual is not None else 0
    _raise(lib.skinny_run_static(ctypes.c_void_p(weight.data_ptr()), n, k, weight.stride(0), idt, od,
                                 ctypes.byref(Tactic(*tactic.astuple())), ctypes.c_void_p(x.data_ptr()), ldx,
                                 ctypes.c_void_p(residual.data_ptr()) if residual is not None else None, ldr,
                                 ctypes.c_void_p(out.data_ptr()), ldo, m, _stream_handle(stream)))
    return out


class Prepared:
    """A prepared weight: tactic table, split-K workspace, warmed kernels.

    The plan keeps W's device pointer (not a copy); the tensor is held here so
    it stays allocated.  ``weight`` is BF16 or FP16 [N, K] with unit column
    stride and a row pitch that is a multiple of 8 elements (16 bytes); x must
    then have the same type.  ``table`` forces a per-M tactic list (64
    entries) instead of tuning on the device.
    """

    def __init__(self, weight, out_dtype=None, table=None):
        import torch
        lib = load_library()
        if out_dtype is None:
            out_dtype = torch.bfloat16
        if weight.dim() != 2 or weight.dtype not in (torch.bfloat16, torch.float16) or not weight.is_cuda:
            raise ValueError("weight must be a 2-D torch.bfloat16 or torch.float16 tensor on a GPU")
        if weight.stride(1) != 1 or weight.stride(0) < weight.shape[1]:
            raise ValueError("weight rows must have unit stride and a pitch >= K")
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError(f"unsupported output dtype {out_dtype}")
        self.weight = weight
        self.n, self.k = weight.shape
        self.in_dtype = weight.dtype
        self.out_dtype = out_dtype
        od = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
        idt = IN_F16 if weight.dtype == torch.float16 else IN_BF16
        ldw = weight.stride(0)
        self._plan = ctypes.c_void_p()
        with torch.cuda.device(weight.device):
            if table is None:
                st = lib.skinny_prepare_ex(weight.data_ptr(), self.n, self.k, ldw, idt, od,
                                           ctypes.byref(self._plan))
            else:
                if len(table) != MAX_M:
                    raise ValueError("table needs one tactic per M = 1..64")
                arr = (Tactic * MAX_M)(*[Tactic(*t.astuple()) for t in table])
                st = lib.skinny_prepare_tactics_ex(weight.data_ptr(), self.n, self.k, ldw, idt, od, arr,
                                                   ctypes.byref(self._plan))
        _raise(st)

    def supports(self, tokens: int) -> bool:
        return bool(load_library().skinny_supports(self._plan, tokens))

    def tactic(self, tokens: int, residual: bool = False) -> Tactic:
        """The tactic run for `tokens` tokens, with or without a residual."""
        t = Tactic()
        _raise(load_library().skinny_plan_tactic_ex(self._plan, tokens, int(bool(residual)), ctypes.byref(t)))
        return t

    def describe(self, tokens: int) -> str:
        buf = ctypes.create_string_buffer(256)
        _raise(load_library().skinny_describe(self._plan, tokens, buf, 256))
        return buf.value.decode()

    def run(self, x, out, stream=None, residual=None):
        """out[:M] = x @ W^T (+ residual[:M]) with M = x.shape[0], on the current
        (or given) stream.  x, out and residual may be row-pitched views with
        unit column stride; residual has out's dtype and may be out itself."""
        import torch
        if x.dim() != 2 or x.shape[1] != self.k or x.dtype != self.in_dtype:
            raise ValueError(f"x must be {self.in_dtype} [M, {self.k}], got {tuple(x.shape)} {x.dtype}")
        m = x.shape[0]
        if out.dim() != 2 or out.shape[1] != self.n or out.shape[0] < m or out.dtype != self.out_dtype:
            raise ValueError(f"out must be {self.out_dtype} [>= {m}, {self.n}]")
        for name, t in (("x", x), ("out", out)) + ((("residual", residual),) if residual is not None else ()):
            if t.stride(1) != 1 and t.shape[1] > 1:
                raise ValueError(f"{name} rows must have unit stride")
            if t.device != self.weight.device:
                raise ValueError(f"{name} and the weight must be on the same device")
        if residual is not None and (residual.dim() != 2 or residual.shape[1] != self.n or
                                     residual.shape[0] < m or residual.dtype != self.out_dtype):
            raise ValueError(f"residual must be {self.out_dtype} [>= {m}, {self.n}]")
        ldx = x.stride(0) if m > 1 else self.k
        ldo = out.stride(0) if out.shape[0] > 1 else self.n
        if residual is None:
            self.run_ptr(x.data_ptr(), out.data_ptr(), m, stream, ldx=ldx, ldo=ldo)
        else:
            ldr = residual.stride(0) if residual.shape[0] > 1 else self.n
            self.run_ptr(x.data_ptr(), out.data_ptr(), m, stream, ldx=ldx, ldo=ldo,
                         res_ptr=residual.data_ptr(), ldr=ldr)
        return out

    def run_ptr(self, x_ptr: int, out_ptr: int, m: int, stream=None, ldx=None, ldo=None, res_ptr=None,
                ldr=None):
        """Raw-pointer form of run (used inside graph capture loops)."""
        lib = load_library()
        if ldx is None and ldo is None and res_ptr is None:
            _raise(lib.skinny_run(self._plan, ctypes.c_void_p(x_ptr), ctypes.c_void_p(out_ptr), m,
                                  _stream_handle(stream)))
            return
        _raise(lib.skinny_run_ex(self._plan, ctypes.c_void_p(x_ptr), self.k if ldx is None else ldx,
                                 ctypes.c_void_p(res_ptr) if res_ptr else None,
                                 (self.n if ldr is None else ldr) if res_ptr else 0,
                                 ctypes.c_void_p(out_ptr), self.n if ldo is None else ldo, m,
                                 _stream_handle(stream)))

    def close(self):
        if self._plan:
            load_library().skinny_destroy(self._plan)
            self._plan = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
