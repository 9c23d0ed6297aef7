"""CPU oracle for the DualQuant dual-scale BCD solver (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (``post_quantization_dq_amd``) never
imports, links or runs it, and the two share no code: this wraps ``dq_oracle.cpp``,
a plain C++ implementation built with g++, through ctypes.

Parity status of each function is recorded in its docstring; the pins live in
``tests/test_oracle_*.py``.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "dq_oracle.cpp"
_LIB_PATH = _HERE / "_build" / "libdq_oracle.so"

FMT = {"INT4": 0, "MXINT4": 1, "MXFP4": 2, "NVFP4": 3, "INT8": 4, "MXINT8": 5,
       "MXFP8_E4M3": 6, "MXFP8_E5M2": 7, "MXFP6_E2M3": 8, "MXFP6_E3M2": 9}
DEFAULT_GROUP = {"INT4": 128, "MXINT4": 32, "MXFP4": 32, "NVFP4": 16, "INT8": 128, "MXINT8": 32,
                 "MXFP8_E4M3": 32, "MXFP8_E5M2": 32, "MXFP6_E2M3": 32, "MXFP6_E3M2": 32}
CODE_BITS = {"INT4": 4, "MXINT4": 4, "MXFP4": 4, "NVFP4": 4, "INT8": 8, "MXINT8": 8,
             "MXFP8_E4M3": 8, "MXFP8_E5M2": 8, "MXFP6_E2M3": 6, "MXFP6_E3M2": 6}


def code_bytes(rows: int, cols: int, fmt: str) -> int:
    """Bytes of packed element codes: two per byte for the 4-bit formats, one for 8-bit."""
    return rows * cols * CODE_BITS[fmt] // 8


def build(force: bool = True) -> Path:
    """Compile the oracle with g++ (no fast-math, no FMA contraction)."""
    if _LIB_PATH.exists() and not force:
        return _LIB_PATH
    _LIB_PATH.parent.mkdir(parents=True, exist_ok=True)
    tmp = _LIB_PATH.with_suffix(".so.tmp")
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", str(_SRC), "-o", str(tmp)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            build(force=False)
        L = C.CDLL(str(_LIB_PATH))
        p = C.c_void_p
        i64 = C.c_int64
        L.o_set_threads.argtypes = [C.c_int]
        L.o_get_threads.restype = C.c_int
        for name in ("o_e2m1_encode", "o_e4m3_encode"):
            getattr(L, name).argtypes = [p, p, i64]
        for name in ("o_e2m1_decode", "o_e4m3_decode", "o_bf16_round"):
            getattr(L, name).argtypes = [p, p, i64]
        L.o_int_round.argtypes = [p, p, i64, C.c_int]
        L.o_mini_encode.argtypes = [C.c_int, p, p, i64]
        L.o_mini_encode.restype = C.c_int
        L.o_mini_decode.argtypes = [C.c_int, p, p, i64]
        L.o_mini_decode.restype = C.c_int
        L.o_project.argtypes = [C.c_int, p, p, i64]
        L.o_fq.argtypes = [C.c_int, C.c_int, p, i64, i64, p, p, p, p, p]
        L.o_fq.restype = C.c_int
        L.o_quantize_weights.argtypes = [p, C.c_int, i64, i64, i64, p, p, C.c_int, C.c_int,
                                         p, p, p, p]
        L.o_quantize_weights.restype = C.c_int
        L.o_dequantize.argtypes = [C.c_int, C.c_int, p, p, C.c_float, i64, i64, p]
        L.o_dequantize.restype = C.c_int
        L.o_solve.argtypes = [p, C.c_int, i64, i64, i64, C.c_int, C.c_int, C.c_int, C.c_float,
                              p, p, p, p, p, p, p, p, p, p, p, p, p, p, C.c_int, p, p,
                              C.c_float]
        L.o_solve.restype = C.c_int
        L.o_rescale_quantize_acts.argtypes = [p, i64, i64, i64, p, C.c_int, C.c_int, p, p, p, p]
        L.o_rescale_quantize_acts.restype = C.c_int
        L.o_quantized_linear.argtypes = [C.c_int, C.c_int, p, p, C.c_float, i64, p, p, C.c_float,
                                         i64, i64, p, p]
        L.o_quantized_linear.restype = C.c_int
        L.o_quantized_linear_entries.argtypes = [C.c_int, C.c_int, p, p, C.c_float, i64, p, p,
                                                 C.c_float, i64, i64, p, p, p, i64, p, p]
        L.o_quantized_linear_entries.restype = C.c_int
        L.o_act_sqnr.argtypes = [p, i64, i64, i64, p, C.c_int, C.c_int, p, p, C.c_float]
        L.o_act_sqnr.restype = C.c_double
        _lib = L
    return _lib


def set_threads(n: int | None = None) -> int:
    n = n or os.cpu_count() or 1
    lib().o_set_threads(int(n))
    return int(n)


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def _w_dtype(W: np.ndarray) -> int:
    if W.dtype == np.float32:
        return 0
    if W.dtype == np.uint16:
        return 1
    raise TypeError("W must be float32 or uint16 (bf16 bit patterns)")


def _scale_dtype(fmt: str):
    return np.uint16 if fmt in ("INT4", "INT8") else np.uint8


# ------------------------------------------------------------------ scalar rounding
def e2m1_encode(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().o_e2m1_encode(_ptr(x), _ptr(out), x.size)
    return out


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    code = np.ascontiguousarray(code, dtype=np.uint8)
    out = np.empty(code.shape, dtype=np.float32)
    lib().o_e2m1_decode(_ptr(code), _ptr(out), code.size)
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest non-negative E4M3FN code (0..126), ties to even, saturating at 448."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().o_e4m3_encode(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    code = np.ascontiguousarray(code, dtype=np.uint8)
    out = np.empty(code.shape, dtype=np.float32)
    lib().o_e4m3_decode(_ptr(code), _ptr(out), code.size)
    return out


def mini_encode(fmt: str, x: np.ndarray) -> np.ndarray:
    """Code (sign bit above the magnitude bits) of the nearest element of an MX FP8/FP6
    type, ties to even, saturating."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _check(lib().o_mini_encode(FMT[fmt], _ptr(x), _ptr(out), x.size), "mini_encode")
    return out


def mini_decode(fmt: str, code: np.ndarray) -> np.ndarray:
    """Values of MX FP8/FP6 element codes (NaN for the non-finite codes)."""
    code = np.ascontiguousarray(code, dtype=np.uint8)
    out = np.empty(code.shape, dtype=np.float32)
    _check(lib().o_mini_decode(FMT[fmt], _ptr(code), _ptr(out), code.size), "mini_decode")
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().o_bf16_round(_ptr(x), _ptr(out), x.size)
    return out


def int_round(x: np.ndarray, qmax: int = 7) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.int8)
    lib().o_int_round(_ptr(x), _ptr(out), x.size, qmax)
    return out


def project(fmt: str, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().o_project(FMT[fmt], _ptr(x), _ptr(out), x.size)
    return out


# ------------------------------------------------------------------ quantisers
def fq(V: np.ndarray, fmt: str, group: int | None = None):
    """FQ_f on an already-normalised fp32 matrix -> (codes, scales, tscale, qhat, flags)."""
    group = group or DEFAULT_GROUP[fmt]
    V = np.ascontiguousarray(V, dtype=np.float32)
    rows, cols = V.shape
    codes = np.zeros(code_bytes(rows, cols, fmt), dtype=np.uint8)
    scales = np.zeros(rows * cols // group, dtype=_scale_dtype(fmt))
    ts = np.zeros(1, dtype=np.float32)
    qhat = np.zeros((rows, cols), dtype=np.float32)
    flags = np.zeros(1, dtype=np.uint32)
    _check(lib().o_fq(FMT[fmt], group, _ptr(V), rows, cols, _ptr(codes), _ptr(scales),
                      _ptr(ts), _ptr(qhat), _ptr(flags)), "fq")
    return codes, scales, float(ts[0]), qhat, int(flags[0])


def quantize_weights(W: np.ndarray, r, c, fmt: str, group: int | None = None):
    """FQ_f(W ./ (r c^T)) -> (codes, scales, tscale, qhat)."""
    group = group or DEFAULT_GROUP[fmt]
    W = np.ascontiguousarray(W)
    rows, cols = W.shape
    r = None if r is None else np.ascontiguousarray(r, dtype=np.float32)
    c = None if c is None else np.ascontiguousarray(c, dtype=np.float32)
    codes = np.zeros(code_bytes(rows, cols, fmt), dtype=np.uint8)
    scales = np.zeros(rows * cols // group, dtype=_scale_dtype(fmt))
    ts = np.zeros(1, dtype=np.float32)
    qhat = np.zeros((rows, cols), dtype=np.float32)
    _check(lib().o_quantize_weights(_ptr(W), _w_dtype(W), rows, cols, cols, _ptr(r), _ptr(c),
                                    FMT[fmt], group, _ptr(codes), _ptr(scales), _ptr(ts),
                                    _ptr(qhat)), "quantize_weights")
    return codes, scales, float(ts[0]), qhat


def dequantize(codes, scales, tscale: float, fmt: str, rows: int, cols: int,
               group: int | None = None) -> np.ndarray:
    group = group or DEFAULT_GROUP[fmt]
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=_scale_dtype(fmt))
    out = np.zeros((rows, cols), dtype=np.float32)
    _check(lib().o_dequantize(FMT[fmt], group, _ptr(codes), _ptr(scales), float(tscale), rows,
                              cols, _ptr(out)), "dequantize")
    return out


def solve(W: np.ndarray, fmt: str, iters: int, group: int | None = None, r_init=None,
          c_init=None, tol: float = 0.0, steps: int = 3, q_init=None) -> dict:
    """The BCD solve; returns r, c, codes, scales, tscale, nmse, relchg, rejected,
    iters_run, r_trace / c_trace (every iteration's unprojected closed forms, NaN where
    D = 0 or the step is frozen; r_pre / c_pre are the last rows) and flags.  `steps`
    selects the scale steps that run: 1 = row scales only, 2 = column scales only, 3 = both
    (the ablation of the news summary: only one of the two scale sets turned on).
    `q_init` = (codes, scales, tscale) of a kept Qhat resumes a solve from the state
    (r_init, c_init, that Qhat) instead of starting from FQ(W ./ r c^T)."""
    group = group or DEFAULT_GROUP[fmt]
    W = np.ascontiguousarray(W)
    rows, cols = W.shape
    ri = None if r_init is None else np.ascontiguousarray(r_init, dtype=np.float32)
    ci = None if c_init is None else np.ascontiguousarray(c_init, dtype=np.float32)
    r = np.zeros(rows, dtype=np.float32)
    c = np.zeros(cols, dtype=np.float32)
    codes = np.zeros(code_bytes(rows, cols, fmt), dtype=np.uint8)
    scales = np.zeros(rows * cols // group, dtype=_scale_dtype(fmt))
    ts = np.zeros(1, dtype=np.float32)
    nmse = np.zeros(iters + 1, dtype=np.float64)
    relchg = np.zeros(iters + 1, dtype=np.float64)
    rej = np.zeros(1, dtype=np.int32)
    run = np.zeros(1, dtype=np.int32)
    r_tr = np.full((max(iters, 1), rows), np.nan, dtype=np.float32)
    c_tr = np.full((max(iters, 1), cols), np.nan, dtype=np.float32)
    flags = np.zeros(1, dtype=np.uint32)
    qc = qs = None
    qt = 0.0
    if q_init is not None:
        qc = np.ascontiguousarray(q_init[0], dtype=np.uint8)
        qs = np.ascontiguousarray(q_init[1], dtype=_scale_dtype(fmt))
        qt = float(q_init[2])
        assert qc.size == codes.size and qs.size == scales.size
    _check(lib().o_solve(_ptr(W), _w_dtype(W), rows, cols, cols, FMT[fmt], group, iters,
                         float(tol), _ptr(ri), _ptr(ci), _ptr(r), _ptr(c), _ptr(codes),
                         _ptr(scales), _ptr(ts), _ptr(nmse), _ptr(relchg), _ptr(rej), _ptr(run),
                         _ptr(r_tr), _ptr(c_tr), _ptr(flags), int(steps), _ptr(qc), _ptr(qs),
                         qt), "solve")
    k = int(run[0])
    return dict(r=r, c=c, codes=codes, scales=scales, tscale=float(ts[0]), nmse=nmse[:k + 1],
                relchg=relchg[:k + 1], rejected=int(rej[0]), iters_run=k, r_trace=r_tr[:iters],
                c_trace=c_tr[:iters], r_pre=r_tr[iters - 1] if iters else r_tr[0],
                c_pre=c_tr[iters - 1] if iters else c_tr[0], flags=int(flags[0]))


def rescale_quantize_acts(X: np.ndarray, c, fmt: str, group: int | None = None):
    """FQ_f(X * c) per token row -> (codes, scales, tscale, dequantised rescaled values)."""
    group = group or DEFAULT_GROUP[fmt]
    X = np.ascontiguousarray(X, dtype=np.uint16)
    tokens, cols = X.shape
    c = None if c is None else np.ascontiguousarray(c, dtype=np.float32)
    codes = np.zeros(code_bytes(tokens, cols, fmt), dtype=np.uint8)
    scales = np.zeros(tokens * cols // group, dtype=_scale_dtype(fmt))
    ts = np.zeros(1, dtype=np.float32)
    xq = np.zeros((tokens, cols), dtype=np.float32)
    _check(lib().o_rescale_quantize_acts(_ptr(X), tokens, cols, cols, _ptr(c), FMT[fmt], group,
                                         _ptr(codes), _ptr(scales), _ptr(ts), _ptr(xq)),
           "rescale_quantize_acts")
    return codes, scales, float(ts[0]), xq


def act_sqnr(X: np.ndarray, c, codes, scales, tscale: float, fmt: str,
             group: int | None = None) -> float:
    """Activation-domain SQNR (dB) of xhat = deq(codes) / c against X."""
    group = group or DEFAULT_GROUP[fmt]
    X = np.ascontiguousarray(X, dtype=np.uint16)
    tokens, cols = X.shape
    c = None if c is None else np.ascontiguousarray(c, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=_scale_dtype(fmt))
    return float(lib().o_act_sqnr(_ptr(X), tokens, cols, cols, _ptr(c), FMT[fmt], group,
                                  _ptr(codes), _ptr(scales), float(tscale)))


# ------------------------------------------------------------------ quantised linear layer
def quantized_linear(a_codes, a_scales, M: int, b_codes, b_scales, N: int, K: int, fmt: str,
                     r=None, group: int | None = None, a_ts: float = 1.0,
                     b_ts: float = 1.0) -> np.ndarray:
    """Y = deq(A) . deq(B)^T . diag(r) in fp64 ([M][N]); A, B in the format's code layout;
    a_ts, b_ts are the NVFP4 tensor scales (ignored by the other formats)."""
    group = group or DEFAULT_GROUP[fmt]
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    b_codes = np.ascontiguousarray(b_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales, dtype=_scale_dtype(fmt))
    b_scales = np.ascontiguousarray(b_scales, dtype=_scale_dtype(fmt))
    r = None if r is None else np.ascontiguousarray(r, dtype=np.float32)
    Y = np.zeros((M, N), dtype=np.float64)
    _check(lib().o_quantized_linear(FMT[fmt], group, _ptr(a_codes), _ptr(a_scales), a_ts, M,
                                    _ptr(b_codes), _ptr(b_scales), b_ts, N, K, _ptr(r), _ptr(Y)),
           "quantized_linear")
    return Y


def quantized_linear_entries(a_codes, a_scales, M: int, b_codes, b_scales, N: int, K: int,
                             fmt: str, mi, ni, r=None, group: int | None = None,
                             a_ts: float = 1.0, b_ts: float = 1.0):
    """Entries (mi[i], ni[i]) of quantized_linear and the sums of |products| (fp64)."""
    group = group or DEFAULT_GROUP[fmt]
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    b_codes = np.ascontiguousarray(b_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales, dtype=_scale_dtype(fmt))
    b_scales = np.ascontiguousarray(b_scales, dtype=_scale_dtype(fmt))
    r = None if r is None else np.ascontiguousarray(r, dtype=np.float32)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    y = np.zeros(mi.size, dtype=np.float64)
    ay = np.zeros(mi.size, dtype=np.float64)
    _check(lib().o_quantized_linear_entries(FMT[fmt], group, _ptr(a_codes), _ptr(a_scales), a_ts,
                                            M, _ptr(b_codes), _ptr(b_scales), b_ts, N, K, _ptr(r),
                                            _ptr(mi),
                                            _ptr(ni), mi.size, _ptr(y), _ptr(ay)),
           "quantized_linear_entries")
    return y, ay
