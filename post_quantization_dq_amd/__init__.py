"""Python binding of the DualQuant dual-scale solver library (libdq.so, gfx950).

The functions named like the C entry points (``dq_solve``, ``dq_quantize_weights``,
``dq_rescale_quantize_acts``, ``dq_rescale_quantize_acts_noalloc``,
``dq_rescale_quantize_acts_multi``, ``dq_quantized_linear``,
``dq_dequantize``,
``dq_workspace_bytes``, ``dq_quantize_workspace_bytes``, ``dq_quantize_multi_workspace_bytes``,
``dq_status_string``, ``dq_debug_round``) only marshal
arguments: torch tensors supply device memory and the current HIP stream; every step of
the computation runs in the library's HIP kernels.  ``solve``, ``quantize_weights``,
``rescale_quantize_acts``, ``rescale_quantize_acts_multi`` and ``dequantize`` are conveniences that allocate the outputs
with torch and call those entry points.

There is no fallback: importing the package fails if ``libdq.so`` has not been built
(``python -m post_quantization_dq_amd.build``).
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from pathlib import Path

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libdq.so"
if not _LIB_PATH.exists():
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m post_quantization_dq_amd.build`")
_lib = C.CDLL(str(_LIB_PATH))

FMT = {"INT4": 0, "MXINT4": 1, "MXFP4": 2, "NVFP4": 3, "INT8": 4, "MXINT8": 5,
       "MXFP8_E4M3": 6, "MXFP8_E5M2": 7, "MXFP6_E2M3": 8, "MXFP6_E3M2": 9}
DEFAULT_GROUP = {"INT4": 128, "MXINT4": 32, "MXFP4": 32, "NVFP4": 16, "INT8": 128, "MXINT8": 32,
                 "MXFP8_E4M3": 32, "MXFP8_E5M2": 32, "MXFP6_E2M3": 32, "MXFP6_E3M2": 32}
CODE_BITS = {"INT4": 4, "MXINT4": 4, "MXFP4": 4, "NVFP4": 4, "INT8": 8, "MXINT8": 8,
             "MXFP8_E4M3": 8, "MXFP8_E5M2": 8, "MXFP6_E2M3": 6, "MXFP6_E3M2": 6}
DT = {torch.float32: 0, torch.bfloat16: 1}
FLAGS = {1: "nonfinite", 2: "zero_row", 4: "zero_col", 8: "nv_block_underflow", 16: "nv_tensor_underflow"}
ROUND_FN = {"e2m1": 0, "e4m3": 1, "bf16": 2, "int4": 3, "proj_mx": 4, "proj_e4m3": 5, "proj_bf16": 6}


class dq_quant_spec(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("group", C.c_int32)]


DQ_STEP_ROW, DQ_STEP_COL = 1, 2   # dq_solve_opts.scale_steps bits (0 = both)
DQ_MAX_MULTI = 8                   # outputs of one dq_rescale_quantize_acts_multi call


class dq_solve_opts(C.Structure):
    _fields_ = [("iters", C.c_int32), ("tol_relchg", C.c_float), ("scale_steps", C.c_int32)]


class dq_report(C.Structure):
    _fields_ = [("iters_run", C.c_int32), ("rejected_steps", C.c_int32), ("flags", C.c_uint32),
                ("sweeps", C.c_int32)]


class dq_problem(C.Structure):
    _fields_ = [("W", C.c_void_p), ("w_dtype", C.c_int32), ("reserved", C.c_int32),
                ("rows", C.c_int64), ("cols", C.c_int64), ("ld", C.c_int64),
                ("r_init", C.c_void_p), ("c_init", C.c_void_p), ("r", C.c_void_p),
                ("c", C.c_void_p), ("codes", C.c_void_p), ("block_scales", C.c_void_p),
                ("tensor_scale", C.c_void_p), ("nmse_hist", C.c_void_p),
                ("relchg_hist", C.c_void_p), ("r_trace", C.c_void_p), ("c_trace", C.c_void_p),
                ("report", C.c_void_p)]


_vp, _i32, _i64, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_lib.dq_status_string.argtypes = [C.c_int]
_lib.dq_status_string.restype = C.c_char_p
_lib.dq_workspace_bytes.argtypes = [C.POINTER(dq_problem), _i32, dq_quant_spec, C.POINTER(dq_solve_opts)]
_lib.dq_workspace_bytes.restype = _sz
_lib.dq_solve.argtypes = [C.POINTER(dq_problem), _i32, dq_quant_spec, C.POINTER(dq_solve_opts), _vp, _sz, _vp]
_lib.dq_solve.restype = C.c_int
_lib.dq_solve_timed.argtypes = [C.POINTER(dq_problem), _i32, dq_quant_spec, C.POINTER(dq_solve_opts), _vp,
                                _sz, _vp, C.POINTER(C.c_float), _i32, C.POINTER(C.c_int32)]
_lib.dq_solve_timed.restype = C.c_int
_lib.dq_solve_timed_enqueue.argtypes = [C.POINTER(dq_problem), _i32, dq_quant_spec, C.POINTER(dq_solve_opts),
                                        _vp, _sz, _vp, _i32]
_lib.dq_solve_timed_enqueue.restype = C.c_int
_lib.dq_solve_timed_read.argtypes = [C.POINTER(C.c_float), _i32, C.POINTER(C.c_int32)]
_lib.dq_solve_timed_read.restype = C.c_int
_lib.dq_quantize_workspace_bytes.argtypes = [_i64, _i64, dq_quant_spec]
_lib.dq_quantize_workspace_bytes.restype = _sz
_lib.dq_quantize_weights.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _vp, dq_quant_spec, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dq_quantize_weights.restype = C.c_int
_lib.dq_rescale_quantize_acts.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, dq_quant_spec, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dq_rescale_quantize_acts.restype = C.c_int
_lib.dq_rescale_quantize_acts_noalloc.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, dq_quant_spec, _vp, _vp, _vp, _vp]
_lib.dq_rescale_quantize_acts_noalloc.restype = C.c_int
_lib.dq_quantize_multi_workspace_bytes.argtypes = [_i64, _i64, _i32, dq_quant_spec]
_lib.dq_quantize_multi_workspace_bytes.restype = _sz
_lib.dq_rescale_quantize_acts_multi.argtypes = [_vp, _i32, _i64, _i64, _i64, _i32, _vp, dq_quant_spec,
                                                _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dq_rescale_quantize_acts_multi.restype = C.c_int
_lib.dq_quantized_linear.argtypes = [dq_quant_spec, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _i64,
                                     _vp, _vp, _i32, _i64, _vp]
_lib.dq_quantized_linear.restype = C.c_int
_lib.dq_quantized_linear_ws.argtypes = [dq_quant_spec, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _i64,
                                        _vp, _vp, _i32, _i64, _vp, _sz, _vp]
_lib.dq_quantized_linear_ws.restype = C.c_int
_lib.dq_quantized_linear_workspace_bytes.argtypes = [dq_quant_spec, _i64, _i64, _i64]
_lib.dq_quantized_linear_workspace_bytes.restype = _sz
_lib.dq_recode_mxint4_to_mxfp6.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _vp]
_lib.dq_recode_mxint4_to_mxfp6.restype = C.c_int
_lib.dq_dequantize.argtypes = [dq_quant_spec, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]
_lib.dq_dequantize.restype = C.c_int
_lib.dq_debug_round.argtypes = [_i32, _vp, _vp, _i64, _vp]
_lib.dq_debug_round.restype = C.c_int

EXPORTED = ("dq_workspace_bytes", "dq_solve", "dq_solve_timed", "dq_solve_timed_enqueue",
            "dq_solve_timed_read", "dq_quantize_workspace_bytes",
            "dq_quantize_weights",
            "dq_rescale_quantize_acts", "dq_rescale_quantize_acts_noalloc",
            "dq_quantize_multi_workspace_bytes",
            "dq_rescale_quantize_acts_multi", "dq_quantized_linear", "dq_quantized_linear_ws",
            "dq_quantized_linear_workspace_bytes", "dq_recode_mxint4_to_mxfp6",
            "dq_dequantize",
            "dq_status_string", "dq_debug_round")


class DQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {dq_status_string(status)} ({status})")


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise DQError(rc, what)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream if isinstance(stream, int) else stream.cuda_stream


def spec_of(fmt: str, group: int | None = None) -> dq_quant_spec:
    return dq_quant_spec(FMT[fmt], int(group or 0))


def scale_dtype(fmt: str) -> torch.dtype:
    return torch.int16 if fmt in ("INT4", "INT8") else torch.uint8


# ------------------------------------------------------------------ C-ABI mirrors
def dq_status_string(status: int) -> str:
    return _lib.dq_status_string(int(status)).decode()


@dataclass
class Problem:
    """One matrix of a solve; every tensor lives on the GPU."""
    W: torch.Tensor
    r: torch.Tensor
    c: torch.Tensor
    codes: torch.Tensor
    block_scales: torch.Tensor
    tensor_scale: torch.Tensor | None = None
    r_init: torch.Tensor | None = None
    c_init: torch.Tensor | None = None
    nmse_hist: torch.Tensor | None = None
    relchg_hist: torch.Tensor | None = None
    r_trace: torch.Tensor | None = None
    c_trace: torch.Tensor | None = None
    report: torch.Tensor | None = None   # int32 [4] on the device: a dq_report

    def to_c(self) -> dq_problem:
        W = self.W
        rows, cols = (W.shape[0], W.shape[1]) if W.dim() == 2 else (0, 0)
        return dq_problem(
            W=_ptr(W), w_dtype=DT.get(W.dtype, -1), reserved=0, rows=rows, cols=cols,
            ld=W.stride(0) if W.dim() == 2 and W.numel() else cols,
            r_init=_ptr(self.r_init), c_init=_ptr(self.c_init), r=_ptr(self.r), c=_ptr(self.c),
            codes=_ptr(self.codes), block_scales=_ptr(self.block_scales),
            tensor_scale=_ptr(self.tensor_scale), nmse_hist=_ptr(self.nmse_hist),
            relchg_hist=_ptr(self.relchg_hist), r_trace=_ptr(self.r_trace), c_trace=_ptr(self.c_trace),
            report=_ptr(self.report))


def _problem_array(problems):
    arr = (dq_problem * len(problems))()
    for k, p in enumerate(problems):
        arr[k] = p.to_c()
    return arr


def dq_workspace_bytes(problems, spec: dq_quant_spec, opts: dq_solve_opts) -> int:
    arr = _problem_array(problems)
    return int(_lib.dq_workspace_bytes(arr, len(problems), spec, C.byref(opts)))


def dq_solve(problems, spec: dq_quant_spec, opts: dq_solve_opts, workspace: torch.Tensor,
             stream=None) -> None:
    """Enqueues the solve on the stream and returns; each problem's `report` tensor holds its
    dq_report once the stream's work has completed."""
    arr = _problem_array(problems)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.dq_solve(arr, len(problems), spec, C.byref(opts), _ptr(workspace), nbytes,
                         _stream(stream)), "dq_solve")


def dq_solve_timed(problems, spec: dq_quant_spec, opts: dq_solve_opts, workspace: torch.Tensor,
                   capacity: int, stream=None) -> list[tuple[float, float, float]]:
    """The diagnostic variant: (row pass, column pass, finalize) durations in ms per queued
    sweep, read after the library synchronises the stream."""
    arr = _problem_array(problems)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    buf = (C.c_float * (3 * max(1, capacity)))()
    n = C.c_int32(0)
    _check(_lib.dq_solve_timed(arr, len(problems), spec, C.byref(opts), _ptr(workspace), nbytes,
                               _stream(stream), buf, int(capacity), C.byref(n)), "dq_solve_timed")
    return [tuple(float(buf[3 * k + q]) for q in range(3)) for k in range(n.value)]


def dq_solve_timed_enqueue(problems, spec: dq_quant_spec, opts: dq_solve_opts,
                           workspace: torch.Tensor, timed_sweeps: int, stream=None) -> None:
    """dq_solve with event pairs on the first `timed_sweeps` queued sweeps; returns without
    waiting.  Read the durations with dq_solve_timed_read once the stream has run them."""
    arr = _problem_array(problems)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.dq_solve_timed_enqueue(arr, len(problems), spec, C.byref(opts), _ptr(workspace),
                                       nbytes, _stream(stream), int(timed_sweeps)),
           "dq_solve_timed_enqueue")


def dq_solve_timed_read(capacity: int) -> list[tuple[float, float, float]]:
    """(row pass, column pass, finalize) durations in ms per timed sweep of the last timed
    solve enqueued on the current device; the caller has waited for its stream."""
    buf = (C.c_float * (3 * max(1, capacity)))()
    n = C.c_int32(0)
    _check(_lib.dq_solve_timed_read(buf, int(capacity), C.byref(n)), "dq_solve_timed_read")
    return [tuple(float(buf[3 * k + q]) for q in range(3)) for k in range(n.value)]


def read_report(problem: Problem) -> dq_report:
    """The problem's dq_report, copied from the device (waits for the solve)."""
    a = problem.report.cpu().numpy()
    return dq_report(int(a[0]), int(a[1]), int(a[2]) & 0xFFFFFFFF, int(a[3]))


def dq_quantize_workspace_bytes(rows: int, cols: int, spec: dq_quant_spec) -> int:
    return int(_lib.dq_quantize_workspace_bytes(rows, cols, spec))


def dq_quantize_weights(W, r, c, spec, codes, block_scales, tensor_scale, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.dq_quantize_weights(_ptr(W), DT.get(W.dtype, -1), W.shape[0], W.shape[1],
                                    W.stride(0) if W.numel() else W.shape[1], _ptr(r), _ptr(c),
                                    spec, _ptr(codes), _ptr(block_scales), _ptr(tensor_scale),
                                    _ptr(workspace), nbytes, _stream(stream)),
           "dq_quantize_weights")


def dq_rescale_quantize_acts(X, c, spec, codes, block_scales, tensor_scale, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.dq_rescale_quantize_acts(_ptr(X), DT.get(X.dtype, -1), X.shape[0], X.shape[1],
                                         X.stride(0) if X.numel() else X.shape[1], _ptr(c), spec,
                                         _ptr(codes), _ptr(block_scales), _ptr(tensor_scale),
                                         _ptr(workspace), nbytes, _stream(stream)),
           "dq_rescale_quantize_acts")


def dq_rescale_quantize_acts_noalloc(X, c, spec, codes, block_scales, tensor_scale, stream=None):
    """The no-workspace variant: the library's fixed per-GPU scratch array stands in for the
    workspace, and nothing is allocated."""
    _check(_lib.dq_rescale_quantize_acts_noalloc(_ptr(X), DT.get(X.dtype, -1), X.shape[0], X.shape[1],
                                                 X.stride(0) if X.numel() else X.shape[1], _ptr(c),
                                                 spec, _ptr(codes), _ptr(block_scales),
                                                 _ptr(tensor_scale), _stream(stream)),
           "dq_rescale_quantize_acts_noalloc")


def dq_quantize_multi_workspace_bytes(rows: int, cols: int, count: int, spec: dq_quant_spec) -> int:
    return int(_lib.dq_quantize_multi_workspace_bytes(rows, cols, count, spec))


def _ptr_array(ts) -> C.Array:
    return (C.c_void_p * len(ts))(*[_ptr(t) for t in ts])


def dq_rescale_quantize_acts_multi(X, cs, spec, codes, block_scales, tensor_scales, workspace,
                                   stream=None):
    """`cs`, `codes`, `block_scales`, `tensor_scales`: one entry per output (c entries may be
    None); they are handed to the library as host arrays of device pointers."""
    n = len(codes)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    c_arr = _ptr_array(cs) if cs is not None else None
    _check(_lib.dq_rescale_quantize_acts_multi(
        _ptr(X), DT.get(X.dtype, -1), X.shape[0], X.shape[1],
        X.stride(0) if X.numel() else X.shape[1], n, c_arr, spec, _ptr_array(codes),
        _ptr_array(block_scales), _ptr_array(tensor_scales), _ptr(workspace), nbytes,
        _stream(stream)), "dq_rescale_quantize_acts_multi")


def dq_quantized_linear(spec, a_codes, a_scales, a_tensor_scale, M, b_codes, b_scales,
                        b_tensor_scale, N, K, r, y, stream=None):
    """y: a 2-D fp32 or bf16 tensor [M][>= N] (row pitch y.stride(0)); the tensor scales are
    [1] fp32 device tensors (NVFP4) or None."""
    _check(_lib.dq_quantized_linear(spec, _ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale), M,
                                    _ptr(b_codes), _ptr(b_scales), _ptr(b_tensor_scale), N, K,
                                    _ptr(r), _ptr(y), DT.get(y.dtype, -1),
                                    y.stride(0) if y.numel() else N, _stream(stream)),
           "dq_quantized_linear")


def dq_quantized_linear_ws(spec, a_codes, a_scales, a_tensor_scale, M, b_codes, b_scales,
                           b_tensor_scale, N, K, r, y, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.dq_quantized_linear_ws(spec, _ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale), M,
                                       _ptr(b_codes), _ptr(b_scales), _ptr(b_tensor_scale), N, K,
                                       _ptr(r), _ptr(y), DT.get(y.dtype, -1),
                                       y.stride(0) if y.numel() else N, _ptr(workspace), nbytes,
                                       _stream(stream)),
           "dq_quantized_linear_ws")


def dq_quantized_linear_workspace_bytes(spec, M, N, K) -> int:
    return int(_lib.dq_quantized_linear_workspace_bytes(spec, M, N, K))


def dq_recode_mxint4_to_mxfp6(codes, block_scales, rows, cols, out_codes, out_scales, stream=None):
    _check(_lib.dq_recode_mxint4_to_mxfp6(_ptr(codes), _ptr(block_scales), rows, cols, _ptr(out_codes),
                                          _ptr(out_scales), _stream(stream)), "dq_recode_mxint4_to_mxfp6")


def dq_dequantize(spec, codes, block_scales, tensor_scale, rows, cols, r, c, out, stream=None):
    _check(_lib.dq_dequantize(spec, _ptr(codes), _ptr(block_scales), _ptr(tensor_scale), rows,
                              cols, _ptr(r), _ptr(c), _ptr(out), _stream(stream)), "dq_dequantize")


def dq_debug_round(fn: str, x: torch.Tensor, out: torch.Tensor, stream=None):
    _check(_lib.dq_debug_round(ROUND_FN[fn], _ptr(x), _ptr(out), x.numel(), _stream(stream)),
           "dq_debug_round")


# ------------------------------------------------------------------ conveniences
def _outputs(rows: int, cols: int, fmt: str, group: int, device):
    codes = torch.empty(rows * cols * CODE_BITS[fmt] // 8, dtype=torch.uint8, device=device)
    scales = torch.empty(rows * cols // group, dtype=scale_dtype(fmt), device=device)
    ts = torch.zeros(1, dtype=torch.float32, device=device)
    return codes, scales, ts


def make_problem(W: torch.Tensor, fmt: str, iters: int, group: int | None = None,
                 r_init=None, c_init=None, trace: bool = False) -> Problem:
    group = group or DEFAULT_GROUP[fmt]
    rows, cols = W.shape
    dev = W.device
    codes, scales, ts = _outputs(rows, cols, fmt, group, dev)
    return Problem(
        W=W, r=torch.empty(rows, dtype=torch.float32, device=dev),
        c=torch.empty(cols, dtype=torch.float32, device=dev), codes=codes, block_scales=scales,
        tensor_scale=ts, r_init=r_init, c_init=c_init,
        nmse_hist=torch.zeros(iters + 1, dtype=torch.float64, device=dev),
        relchg_hist=torch.zeros(iters + 1, dtype=torch.float64, device=dev),
        r_trace=torch.full((max(iters, 1), rows), float("nan"), device=dev) if trace else None,
        c_trace=torch.full((max(iters, 1), cols), float("nan"), device=dev) if trace else None,
        report=torch.zeros(4, dtype=torch.int32, device=dev))


def solve_many(problems, fmt: str, iters: int, group: int | None = None, tol: float = 0.0,
               stream=None, workspace: torch.Tensor | None = None, pass_ms: list | None = None,
               steps: int = 0, read_reports: bool = True, timed_sweeps: int = 0):
    """Solve a batch of problems.  `workspace` may be passed in to reuse one allocation.
    When `pass_ms` is a list, the diagnostic dq_solve_timed runs instead and appends one
    (row pass, column pass, finalize) tuple of event-timed durations in ms per sweep that did
    work.  With timed_sweeps > 0 the solve is enqueued with those events attached to its
    first `timed_sweeps` queued sweeps but nothing waits for it; timed_passes() reads them
    afterwards.  `steps` selects the scale steps
    (DQ_STEP_ROW | DQ_STEP_COL; 0 = both).  Returns the reports read back from the device
    (a synchronisation), or None with read_reports=False (the solve is then only
    enqueued)."""
    spec = spec_of(fmt, group)
    opts = dq_solve_opts(int(iters), float(tol), int(steps))
    nbytes = dq_workspace_bytes(problems, spec, opts)
    if nbytes == 0:
        raise DQError(-7, "dq_workspace_bytes")
    ws = workspace
    if ws is None or ws.numel() * ws.element_size() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=problems[0].W.device)
    if pass_ms is not None:
        per = dq_solve_timed(problems, spec, opts, ws, 2 * int(iters) + 2, stream)
        ran = max(read_report(p).sweeps for p in problems)
        pass_ms.extend(per[:ran])
    elif timed_sweeps > 0:
        dq_solve_timed_enqueue(problems, spec, opts, ws, int(timed_sweeps), stream)
    else:
        dq_solve(problems, spec, opts, ws, stream)
    if not read_reports:
        return None
    return [read_report(p) for p in problems]


def timed_passes(problems, iters: int) -> list[tuple[float, float, float]]:
    """The per-sweep pass durations of the last timed solve_many(timed_sweeps=...) on the
    current device, for the timed sweeps that did work; call after waiting for the solve's
    stream."""
    per = dq_solve_timed_read(2 * int(iters) + 2)
    ran = max(read_report(p).sweeps for p in problems)
    return per[:ran]


def solve(W: torch.Tensor, fmt: str, iters: int, group: int | None = None, r_init=None,
          c_init=None, tol: float = 0.0, trace: bool = False, stream=None, steps: int = 0) -> dict:
    """Run the solve on one matrix; returns the output tensors and the report.  With
    trace=True, r_trace / c_trace hold every iteration's unprojected closed forms."""
    p = make_problem(W, fmt, iters, group, r_init, c_init, trace)
    rep = solve_many([p], fmt, iters, group, tol, stream, steps=steps)[0]
    k = rep.iters_run
    return dict(r=p.r, c=p.c, codes=p.codes, scales=p.block_scales, tscale=p.tensor_scale,
                nmse=p.nmse_hist[:k + 1], relchg=p.relchg_hist[:k + 1],
                r_trace=None if p.r_trace is None else p.r_trace[:iters],
                c_trace=None if p.c_trace is None else p.c_trace[:iters],
                iters_run=rep.iters_run, rejected=rep.rejected_steps, flags=rep.flags,
                sweeps=rep.sweeps)


def quantize_weights(W: torch.Tensor, r=None, c=None, fmt: str = "NVFP4", group: int | None = None,
                     stream=None):
    group = group or DEFAULT_GROUP[fmt]
    spec = spec_of(fmt, group)
    codes, scales, ts = _outputs(W.shape[0], W.shape[1], fmt, group, W.device)
    nb = dq_quantize_workspace_bytes(W.shape[0], W.shape[1], spec)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=W.device)
    dq_quantize_weights(W, r, c, spec, codes, scales, ts, ws, stream)
    return codes, scales, ts


def rescale_quantize_acts(X: torch.Tensor, c=None, fmt: str = "NVFP4", group: int | None = None,
                          stream=None):
    group = group or DEFAULT_GROUP[fmt]
    spec = spec_of(fmt, group)
    codes, scales, ts = _outputs(X.shape[0], X.shape[1], fmt, group, X.device)
    nb = dq_quantize_workspace_bytes(X.shape[0], X.shape[1], spec)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=X.device)
    dq_rescale_quantize_acts(X, c, spec, codes, scales, ts, ws, stream)
    return codes, scales, ts


def rescale_quantize_acts_multi(X: torch.Tensor, cs, fmt: str = "NVFP4", group: int | None = None,
                                stream=None):
    """One activation matrix, several column-scale vectors (None = no beta): returns a list
    of (codes, scales, tensor scale), one per entry of `cs`, each equal to
    rescale_quantize_acts(X, cs[k], ...)."""
    group = group or DEFAULT_GROUP[fmt]
    spec = spec_of(fmt, group)
    outs = [_outputs(X.shape[0], X.shape[1], fmt, group, X.device) for _ in cs]
    nb = dq_quantize_multi_workspace_bytes(X.shape[0], X.shape[1], len(cs), spec)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=X.device)
    dq_rescale_quantize_acts_multi(X, list(cs), spec, [o[0] for o in outs], [o[1] for o in outs],
                                   [o[2] for o in outs], ws, stream)
    return outs


def recode_mxint4_to_mxfp6(codes, scales, rows: int, cols: int, stream=None):
    """MXINT4 codes and scales -> the equal-valued MXFP6 E2M3 codes and scales."""
    out_c = torch.empty(rows * cols * 3 // 4, dtype=torch.uint8, device=codes.device)
    out_s = torch.empty(rows * cols // 32, dtype=torch.uint8, device=codes.device)
    dq_recode_mxint4_to_mxfp6(codes, scales, rows, cols, out_c, out_s, stream)
    return out_c, out_s


def quantized_linear(a_codes, a_scales, b_codes, b_scales, M: int, N: int, K: int, fmt: str,
                     r=None, out_dtype=torch.float32, stream=None, a_tensor_scale=None,
                     b_tensor_scale=None, group: int | None = None, split: bool = True) -> torch.Tensor:
    """Y [M][N] = deq(A) deq(B)^T diag(r) from activation codes A [M][K] and weight codes
    B [N][K] of an MX format, NVFP4 (which also takes the two [1] fp32 tensor scales) or
    INT4 (bf16 scales per `group` = 64 or 128 elements).  MXINT4 operands are re-encoded as
    MXFP6 E2M3 first (exact; for weights this can be done once and kept).  With `split`, an
    INT4 layer with few output tiles splits K over a workspace allocated here."""
    if fmt == "MXINT4":
        a_codes, a_scales = recode_mxint4_to_mxfp6(a_codes, a_scales, M, K, stream)
        b_codes, b_scales = recode_mxint4_to_mxfp6(b_codes, b_scales, N, K, stream)
        fmt = "MXFP6_E2M3"
    y = torch.empty(M, N, dtype=out_dtype, device=a_codes.device)
    spec = spec_of(fmt, group)
    nb = dq_quantized_linear_workspace_bytes(spec, M, N, K) if split else 0
    ws = torch.empty(nb, dtype=torch.uint8, device=a_codes.device) if nb else None
    dq_quantized_linear_ws(spec, a_codes, a_scales, a_tensor_scale, M, b_codes, b_scales,
                           b_tensor_scale, N, K, r, y, ws, stream)
    return y


def dequantize(codes, scales, tscale, rows: int, cols: int, fmt: str, group: int | None = None,
               r=None, c=None, stream=None) -> torch.Tensor:
    out = torch.empty(rows, cols, dtype=torch.float32, device=codes.device)
    dq_dequantize(spec_of(fmt, group), codes, scales, tscale, rows, cols, r, c, out, stream)
    return out
