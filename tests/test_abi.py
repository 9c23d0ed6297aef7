"""C-ABI checks that need no GPU: the library loads, exports every entry point the header
declares, and rejects bad arguments synchronously (before any HIP call)."""

import ctypes as C
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def dq():
    import post_quantization_dq_amd as dq

    return dq


def _declared():
    text = (ROOT / "include" / "dq.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(dq):
    names = _declared()
    assert set(names) == set(dq.EXPORTED)
    lib = C.CDLL(str(ROOT / "post_quantization_dq_amd" / "libdq.so"))
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(dq):
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert dq.dq_status_string(s) and dq.dq_status_string(s) != "unknown status"


def _problem(dq, rows=64, cols=256, ld=None, dtype=1, W=0x10000, codes=0x20000):
    kw = dict(W=W, w_dtype=dtype, reserved=0, rows=rows, cols=cols,
              ld=ld if ld is not None else cols, r_init=None, c_init=None, r=0x30000,
              c=0x40000, codes=codes, block_scales=0x50000, tensor_scale=0x60000,
              nmse_hist=None, relchg_hist=None, r_trace=None, c_trace=None, report=None)
    # ctypes keeps an unknown keyword as a plain attribute: name every field exactly
    assert set(kw) == {f[0] for f in dq.dq_problem._fields_}
    return dq.dq_problem(**kw)


def _solve_rc(dq, probs, fmt=3, group=0, iters=4, ws=0x70000, wsb=1 << 40):
    arr = (dq.dq_problem * len(probs))(*probs)
    opts = dq.dq_solve_opts(iters, 0.0, 0)
    return dq._lib.dq_solve(arr, len(probs), dq.dq_quant_spec(fmt, group), C.byref(opts), ws, wsb, None)


def test_solve_argument_errors(dq):
    ok = _problem(dq)
    assert _solve_rc(dq, [ok], fmt=10) == -4                        # unknown format
    assert _solve_rc(dq, [ok], fmt=8, group=16) == -4               # MX blocks are 32 elements
    assert _solve_rc(dq, [ok], fmt=0, group=32) == -4               # INT4 needs 64 or 128
    assert _solve_rc(dq, [_problem(dq, cols=200)]) == -2            # not a whole number of blocks
    assert _solve_rc(dq, [_problem(dq, cols=65664)]) == -2          # wider than 65536
    assert _solve_rc(dq, [_problem(dq, ld=100)]) == -2              # ld < cols
    assert _solve_rc(dq, [_problem(dq, W=0x10004)]) == -3           # misaligned W
    assert _solve_rc(dq, [_problem(dq, ld=260)]) == -3              # row pitch not 16-byte multiple
    assert _solve_rc(dq, [_problem(dq, W=0)]) == -1                 # null W
    assert _solve_rc(dq, [_problem(dq, dtype=5)]) == -4             # unknown dtype
    assert _solve_rc(dq, [ok], iters=-1) == -7
    assert _solve_rc(dq, [ok], ws=0) == -5                          # no workspace
    assert _solve_rc(dq, [ok], wsb=16) == -5                        # workspace too small
    arr = (dq.dq_problem * 1)(ok)
    assert dq._lib.dq_solve(arr, 0, dq.dq_quant_spec(3, 0), C.byref(dq.dq_solve_opts(1, 0.0, 0)), 0x70000, 1 << 40, None) == -7


def test_timed_solve_argument_errors(dq):
    """The diagnostic timed solves check their own arguments, then the solve's, before any
    HIP call."""
    L = dq._lib
    ok, bad = _problem(dq), _problem(dq, cols=200)
    spec, opts = dq.dq_quant_spec(3, 0), C.byref(dq.dq_solve_opts(4, 0.0, 0))
    arr, barr = (dq.dq_problem * 1)(ok), (dq.dq_problem * 1)(bad)
    buf, n = (C.c_float * 30)(), C.c_int32(5)
    for k in (0, -3):   # nothing to time
        assert L.dq_solve_timed_enqueue(arr, 1, spec, opts, 0x70000, 1 << 40, None, k) == -7
    assert L.dq_solve_timed_enqueue(barr, 1, spec, opts, 0x70000, 1 << 40, None, 8) == -2
    assert L.dq_solve_timed_enqueue(arr, 1, spec, opts, 0, 0, None, 8) == -5
    assert L.dq_solve_timed_read(None, 10, C.byref(n)) == -1
    assert L.dq_solve_timed_read(buf, 10, None) == -1
    assert L.dq_solve_timed_read(buf, -1, C.byref(n)) == -7
    assert L.dq_solve_timed(arr, 1, spec, opts, 0x70000, 1 << 40, None, None, 10, C.byref(n)) == -1
    assert L.dq_solve_timed(arr, 1, spec, opts, 0x70000, 1 << 40, None, buf, -1, C.byref(n)) == -7
    assert L.dq_solve_timed(barr, 1, spec, opts, 0x70000, 1 << 40, None, buf, 10, C.byref(n)) == -2


def test_workspace_bytes_accounting(dq):
    ok = _problem(dq, rows=4096, cols=14336)
    arr = (dq.dq_problem * 1)(ok)
    nb = dq._lib.dq_workspace_bytes(arr, 1, dq.dq_quant_spec(3, 0), C.byref(dq.dq_solve_opts(16, 0.0, 0)))
    # at least the second code/scale buffer, scales, column partials for one strip per CU
    assert nb >= 4096 * 14336 // 2 + 4096 * 14336 // 16
    assert nb < 4096 * 14336 * 2   # below the size of W itself
    bad = (dq.dq_problem * 1)(_problem(dq, cols=200))
    assert dq._lib.dq_workspace_bytes(bad, 1, dq.dq_quant_spec(3, 0), C.byref(dq.dq_solve_opts(16, 0.0, 0))) == 0


def test_quantize_argument_errors(dq):
    L = dq._lib
    sp = dq.dq_quant_spec(3, 0)
    assert L.dq_quantize_weights(0x10000, 1, 8, 200, 200, None, None, sp, 0x20000, 0x30000, 0x40000, 0x50000, 4096, None) == -2
    assert L.dq_quantize_weights(0x10000, 1, 8, 256, 256, None, None, sp, 0x20000, 0x30000, 0x40000, 0, 0, None) == -5
    assert L.dq_quantize_weights(0x10000, 1, 8, 256, 256, None, None, dq.dq_quant_spec(10, 0), 0x20000, 0x30000, 0x40000, 0x50000, 4096, None) == -4
    assert L.dq_rescale_quantize_acts(0x10000, 1, 8, 256, 256, None, sp, 0, 0x30000, 0x40000, 0x50000, 4096, None) == -1
    assert L.dq_rescale_quantize_acts(0x10002, 1, 8, 256, 256, None, sp, 0x20000, 0x30000, 0x40000, 0x50000, 4096, None) == -3
    assert L.dq_quantize_weights(0x10000, 1, 0, 256, 256, None, None, sp, 0, 0, 0, 0, 0, None) == 0   # empty
    assert L.dq_dequantize(dq.dq_quant_spec(2, 0), 0x10000, 0x20000, None, 4, 48, None, None, 0x30000, None) == -2
    assert L.dq_debug_round(99, 0x10000, 0x20000, 4, None) == -7


def test_quantize_multi_argument_errors(dq):
    L = dq._lib
    sp = dq.dq_quant_spec(3, 0)
    ptrs = (C.c_void_p * 8)(*([0x20000] * 8))
    for n in (0, 9, -1):
        assert L.dq_rescale_quantize_acts_multi(0x10000, 1, 8, 256, 256, n, None, sp, ptrs, ptrs, ptrs, 0x50000, 1 << 20, None) == -7
        assert L.dq_quantize_multi_workspace_bytes(8, 256, n, sp) == 0
    assert L.dq_quantize_multi_workspace_bytes(8, 256, 3, sp) == 3 * L.dq_quantize_workspace_bytes(8, 256, sp)
    assert L.dq_quantize_multi_workspace_bytes(8, 256, 3, dq.dq_quant_spec(1, 0)) == 0
    assert L.dq_rescale_quantize_acts_multi(0x10000, 1, 8, 200, 200, 3, None, sp, ptrs, ptrs, ptrs, 0x50000, 1 << 20, None) == -2
    assert L.dq_rescale_quantize_acts_multi(0x10000, 1, 8, 256, 256, 3, None, sp, None, ptrs, ptrs, 0x50000, 1 << 20, None) == -1
    holes = (C.c_void_p * 3)(0x20000, None, 0x20000)
    assert L.dq_rescale_quantize_acts_multi(0x10000, 1, 8, 256, 256, 3, None, sp, holes, ptrs, ptrs, 0x50000, 1 << 20, None) == -1
    assert L.dq_rescale_quantize_acts_multi(0x10000, 1, 8, 256, 256, 3, None, sp, ptrs, ptrs, holes, 0x50000, 1 << 20, None) == -1
    odd = (C.c_void_p * 3)(0x20000, 0x20008, 0x20000)
    assert L.dq_rescale_quantize_acts_multi(0x10000, 1, 8, 256, 256, 3, None, sp, odd, ptrs, ptrs, 0x50000, 1 << 20, None) == -3
    assert L.dq_rescale_quantize_acts_multi(0x10000, 1, 8, 256, 256, 3, None, sp, ptrs, ptrs, ptrs, 0x50000, 16, None) == -5
    assert L.dq_rescale_quantize_acts_multi(0x10000, 1, 8, 256, 256, 3, None, sp, ptrs, ptrs, ptrs, 0, 0, None) == -5
    # tensor scales are not needed outside NVFP4
    assert L.dq_rescale_quantize_acts_multi(0x10000, 1, 0, 256, 256, 3, None, dq.dq_quant_spec(1, 0), ptrs, ptrs, None, None, 0, None) == 0


def test_quantized_linear_argument_errors(dq):
    L = dq._lib
    mx = dq.dq_quant_spec(2, 0)
    nv = dq.dq_quant_spec(3, 0)

    def call(spec, ac=0x10000, asc=0x20000, ats=None, M=64, bc=0x30000, bsc=0x40000, bts=None,
             N=64, K=256, r=None, y=0x50000, dt=0, ldy=64):
        return L.dq_quantized_linear(spec, ac, asc, ats, M, bc, bsc, bts, N, K, r, y, dt, ldy, None)

    assert call(dq.dq_quant_spec(1, 0)) == -4            # MXINT4 (recode it first)
    assert call(dq.dq_quant_spec(4, 64)) == -4           # INT8 has no layer
    assert call(dq.dq_quant_spec(0, 32)) == -4           # INT4 groups are 64 or 128
    assert call(dq.dq_quant_spec(0, 64), K=96) == -2     # K not a multiple of the group
    assert call(dq.dq_quant_spec(0, 128), K=192) == -2
    assert call(dq.dq_quant_spec(0, 64), asc=0x20001) == -3   # bf16 scales at an odd address
    assert call(dq.dq_quant_spec(0, 64), bsc=0x40001) == -3
    assert call(mx, dt=5) == -4                          # output dtype
    assert call(mx, ldy=63) == -2                        # ldy < N
    assert call(mx, K=100) == -2                         # K not a multiple of 32
    assert call(nv, K=48, ats=0x60000, bts=0x60000) == -2
    assert call(mx, ac=0x10008) == -3                    # codes not 16-byte aligned
    assert call(mx, y=0x50002) == -3                     # fp32 output misaligned
    assert call(mx, ac=None) == -1
    assert call(mx, y=None) == -1
    assert call(nv) == -1                                # NVFP4 needs both tensor scales
    assert call(nv, ats=0x60000) == -1
    assert call(nv, bts=0x60000) == -1
    assert call(mx, ac=None, asc=None, M=0, bc=None, bsc=None, y=None) == 0   # M = 0


def test_linear_workspace_sizes(dq):
    """Host-side split plan of the INT4 layer: few output tiles split K, many do not, other
    formats never; the size is splits x M x N (rounded to 4) fp32 values."""
    i4 = dq.dq_quant_spec(0, 64)
    nb = dq.dq_quantized_linear_workspace_bytes(i4, 82, 4096, 4096)
    assert nb > 0 and nb % (82 * 4096 * 4) == 0
    assert dq.dq_quantized_linear_workspace_bytes(i4, 2048, 4096, 4096) == 0
    assert dq.dq_quantized_linear_workspace_bytes(dq.dq_quant_spec(2, 0), 82, 4096, 4096) == 0
    assert dq.dq_quantized_linear_workspace_bytes(i4, 82, 4096, 64) == 0     # one stage of K
    assert dq.dq_quantized_linear_workspace_bytes(i4, 0, 4096, 4096) == 0
    for M, N, K in [(1, 1024, 4096), (16, 4096, 14336), (82, 1024, 4096), (82, 14336, 4096),
                    (130, 1024, 4096), (5, 300, 640)]:
        nb2 = dq.dq_quantized_linear_workspace_bytes(i4, M, N, K)
        assert 0 < nb2 <= K * (N + 3), (M, N, K)   # within twice the weight codes
    L = dq._lib
    # a workspace smaller than needed is refused before anything is launched
    assert L.dq_quantized_linear_ws(i4, 0x10000, 0x20000, None, 82, 0x30000, 0x40000, None, 4096,
                                    4096, None, 0x50000, 0, 4096, 0x60000, nb - 16, None) == -5


def test_recode_argument_errors(dq):
    L = dq._lib
    assert L.dq_recode_mxint4_to_mxfp6(0x10000, 0x20000, 4, 48, 0x30000, 0x40000, None) == -2
    assert L.dq_recode_mxint4_to_mxfp6(None, 0x20000, 4, 64, 0x30000, 0x40000, None) == -1
    assert L.dq_recode_mxint4_to_mxfp6(0x10008, 0x20000, 4, 64, 0x30000, 0x40000, None) == -3
    assert L.dq_recode_mxint4_to_mxfp6(0x10000, 0x20000, 4, 64, 0x30004, 0x40000, None) == -3
    assert L.dq_recode_mxint4_to_mxfp6(None, None, 0, 64, None, None, None) == 0


def test_header_is_plain_c(tmp_path):
    """The header compiles as strict C99 (no C++ or HIP types in the ABI), and a C program
    links against the library and calls it (status strings only: no device needed)."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    src = tmp_path / "abi.c"
    src.write_text('#include <string.h>\n#include "dq.h"\n'
                   'int main(void) {\n'
                   '  const char* s = dq_status_string(DQ_ERR_WORKSPACE);\n'
                   '  return (s && strstr(s, "workspace")) ? 0 : 1;\n}\n')
    lib = ROOT / "post_quantization_dq_amd"
    exe = tmp_path / "abi"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    f"-I{ROOT / 'include'}", str(src), f"-L{lib}", "-ldq",
                    f"-Wl,-rpath,{lib}", "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0
