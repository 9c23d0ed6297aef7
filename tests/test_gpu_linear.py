"""dq_quantized_linear against the oracle's fp64 product of the dequantised codes.

Tolerances follow the arithmetic of the matrix cores:
  * E2M1 and E2M3 operands: each instruction's 128 products and their sum are exact, so
    only the fp32 accumulation over the K/128 instructions and the r multiply round:
    |y - ref| <= (K/128 + 2) 2^-24 sum_k |a_k b_k| |r_n|;
  * E4M3, E5M2 and E3M2 operands: the cores keep fewer bits in their internal sum (measured
    on random codes: up to 2.3e-4 of sum |a b| per instruction), bound 2^-11 sum |a b| |r|;
  * bf16 output adds its rounding to 8 significant bits, at most 2^-8 |y|.
Inputs are uniformly random finite codes (every grid value, both signs) with block scales
spread over 2^-7 .. 2^7, so every code and the scale handling are exercised.
"""

import numpy as np
import pytest
import torch

import post_quantization_dq_amd as dq
import synth
from gpu_util import BITS, DEV, pack_codes, random_codes, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["MXFP4", "MXFP6_E2M3", "MXFP6_E3M2", "MXFP8_E4M3", "MXFP8_E5M2"]
EXACT = {"MXFP4", "MXFP6_E2M3"}


def _inputs(fmt, M, N, K, seed):
    rng = np.random.default_rng(seed)
    ae, be = random_codes(rng, fmt, M, K), random_codes(rng, fmt, N, K)
    asc = rng.integers(120, 135, M * K // 32).astype(np.uint8)
    bsc = rng.integers(120, 135, N * K // 32).astype(np.uint8)
    r = np.exp2(rng.uniform(-2, 2, N)).astype(np.float32)
    return pack_codes(ae, BITS[fmt]), asc, pack_codes(be, BITS[fmt]), bsc, r


def _tol(fmt, K, absy, y, out_dtype):
    t = ((K // 128 + 3) * 2.0 ** -24 if fmt in EXACT else 2.0 ** -11) * absy
    if out_dtype == torch.bfloat16:
        t = t + 2.0 ** -8 * (np.abs(y) + t)
    return t + 1e-37


def _run(a, asc, b, bsc, M, N, K, fmt, r, out_dtype):
    y = dq.quantized_linear(torch.from_numpy(a).to(DEV), torch.from_numpy(asc).to(DEV),
                            torch.from_numpy(b).to(DEV), torch.from_numpy(bsc).to(DEV), M, N, K, fmt,
                            r=None if r is None else to_dev(r), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(100, 70, 384), (1, 16, 32), (130, 257, 4160), (256, 256, 1024)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_random_codes(oracle_lib, fmt, shape, out_dtype):
    M, N, K = shape
    a, asc, b, bsc, r = _inputs(fmt, M, N, K, M + N + K)
    for rr in (r, None):
        y = _run(a, asc, b, bsc, M, N, K, fmt, rr, out_dtype)
        ref = oracle_lib.quantized_linear(a, asc, M, b, bsc, N, K, fmt, r=rr)
        mi, ni = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        _, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, fmt, mi.ravel(),
                                                      ni.ravel(), r=rr)
        absy = absy.reshape(M, N)
        err = np.abs(y - ref)
        tol = _tol(fmt, K, absy, ref, out_dtype)
        assert np.all(err <= tol), (fmt, shape, float((err / (absy + 1e-300)).max()))


@pytest.mark.parametrize("fmt", ["MXFP4", "MXFP8_E4M3"])
def test_full_size_sampled(oracle_lib, fmt):
    """The benchmark shape (2048 tokens x 4096 outputs x 4096 inputs): 512 sampled entries."""
    M, N, K = 2048, 4096, 4096
    print(f"[linear] {fmt} {M}x{N}x{K}", flush=True)
    a, asc, b, bsc, r = _inputs(fmt, M, N, K, 7)
    y = _run(a, asc, b, bsc, M, N, K, fmt, r, torch.float32)
    rng = np.random.default_rng(8)
    mi, ni = rng.integers(0, M, 512), rng.integers(0, N, 512)
    mi[:4], ni[:4] = [0, M - 1, 0, M - 1], [0, 0, N - 1, N - 1]
    ref, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, fmt, mi, ni, r=r)
    got = y[mi, ni]
    assert np.all(np.abs(got - ref) <= _tol(fmt, K, absy, ref, torch.float32))


def test_empty_and_zero_k(oracle_lib):
    y = dq.quantized_linear(torch.empty(0, dtype=torch.uint8, device=DEV),
                            torch.empty(0, dtype=torch.uint8, device=DEV),
                            torch.empty(0, dtype=torch.uint8, device=DEV),
                            torch.empty(0, dtype=torch.uint8, device=DEV), 5, 7, 0, "MXFP4")
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    y0 = dq.quantized_linear(torch.zeros(16, dtype=torch.uint8, device=DEV),
                             torch.zeros(1, dtype=torch.uint8, device=DEV),
                             torch.zeros(16, dtype=torch.uint8, device=DEV),
                             torch.zeros(1, dtype=torch.uint8, device=DEV), 0, 1, 32, "MXFP4")
    torch.cuda.synchronize()
    assert y0.shape == (0, 1)


@pytest.mark.parametrize("name", ["q4096x4096_mxfp4", "k1024x4096_mxint4"])
def test_layer_from_solved_weights(oracle_lib, name):
    """End to end on a 512 x 4096 slice of a weight: solve (its format, T = 4), quantise 256
    tokens of activations with the solved column scales, run the layer.  The output matches
    the oracle's product of the same codes and approximates X W^T."""
    W, _, fmt, g, _ = synth.workload(name)
    W = np.ascontiguousarray(W[:512])
    X = synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(256, 4096), 3)
    res = dq.solve(to_dev(W), fmt, 4)
    codes_x, scales_x, _ = dq.rescale_quantize_acts(to_dev(X), res["c"], fmt)
    y = dq.quantized_linear(codes_x, scales_x, res["codes"], res["scales"], 256, 512, 4096, fmt,
                            r=res["r"])
    torch.cuda.synchronize()
    yc = y.cpu().numpy().astype(np.float64)
    args = (codes_x.cpu().numpy(), scales_x.cpu().numpy(), 256, res["codes"].cpu().numpy(),
            res["scales"].cpu().numpy(), 512, 4096, fmt)
    ref = oracle_lib.quantized_linear(*args, r=res["r"].cpu().numpy())
    mi, ni = np.meshgrid(np.arange(256), np.arange(512), indexing="ij")
    _, absy = oracle_lib.quantized_linear_entries(*args, mi.ravel(), ni.ravel(), r=res["r"].cpu().numpy())
    assert np.all(np.abs(yc - ref) <= _tol("MXFP4", 4096, absy.reshape(256, 512), ref, torch.float32))
    Xf = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Wf = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = Xf @ Wf.T
    rel = np.linalg.norm(yc - exact) / np.linalg.norm(exact)
    print(f"[linear] W4A4 {fmt} layer relative error vs bf16 product: {rel:.4f}", flush=True)
    assert rel < 0.5


@pytest.mark.parametrize("fmt", ["MXFP4", "MXFP8_E4M3", "MXFP8_E5M2"])
def test_direct_and_staged_kernels_agree(oracle_lib, fmt):
    """The direct-to-LDS kernel (4-byte aligned scale arrays, K a multiple of the stage)
    and the register-staged kernel (the same scales at an odd address) multiply the same
    codes in the same order: bitwise equal outputs, both within the oracle bound."""
    M, N, K = 160, 200, 1024
    a, asc, b, bsc, r = _inputs(fmt, M, N, K, 11)
    dev = lambda x: torch.from_numpy(x).to(DEV)
    A, B = dev(a), dev(b)
    sa_al, sb_al = dev(asc), dev(bsc)
    pad_a = torch.zeros(asc.size + 16, dtype=torch.uint8, device=DEV)
    pad_b = torch.zeros(bsc.size + 16, dtype=torch.uint8, device=DEV)
    pad_a[1:1 + asc.size] = sa_al
    pad_b[1:1 + bsc.size] = sb_al
    sa_odd, sb_odd = pad_a[1:1 + asc.size], pad_b[1:1 + bsc.size]
    assert sa_odd.data_ptr() % 4 != 0 and sa_al.data_ptr() % 4 == 0
    y1 = dq.quantized_linear(A, sa_al, B, sb_al, M, N, K, fmt, r=to_dev(r))
    y2 = dq.quantized_linear(A, sa_odd, B, sb_odd, M, N, K, fmt, r=to_dev(r))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ref = oracle_lib.quantized_linear(a, asc, M, b, bsc, N, K, fmt, r=r)
    mi, ni = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    _, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, fmt, mi.ravel(), ni.ravel(), r=r)
    err = np.abs(y1.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= _tol(fmt, K, absy.reshape(M, N), ref, torch.float32))


def _mxint4_inputs(rng, rows, cols):
    q = rng.integers(-7, 8, rows * cols)
    codes = pack_codes((q & 0xF).astype(np.uint8), 4)
    scales = rng.integers(0, 255, rows * cols // 32).astype(np.uint8)
    scales[:8] = [0, 1, 2, 3, 127, 200, 254, 0]
    return codes, scales


def test_recode_mxint4_is_exact(oracle_lib):
    """MXINT4 -> MXFP6 E2M3 re-encoding keeps every dequantised value, including the blocks
    whose scale is 2^-127 or 2^-126 (their elements become q/4 and q/2)."""
    rng = np.random.default_rng(12)
    rows, cols = 37, 1024
    codes, scales = _mxint4_inputs(rng, rows, cols)
    oc, os_ = dq.recode_mxint4_to_mxfp6(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                                        rows, cols)
    torch.cuda.synchronize()
    want = oracle_lib.dequantize(codes, scales, 0.0, "MXINT4", rows, cols)
    got = oracle_lib.dequantize(oc.cpu().numpy(), os_.cpu().numpy(), 0.0, "MXFP6_E2M3", rows, cols)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("shape", [(100, 70, 384), (256, 256, 1024)])
def test_mxint4_linear(oracle_lib, shape):
    M, N, K = shape
    rng = np.random.default_rng(M + K)
    a, asc = _mxint4_inputs(rng, M, K)
    b, bsc = _mxint4_inputs(rng, N, K)
    asc = np.clip(asc, 118, 136).astype(np.uint8)
    bsc = np.clip(bsc, 118, 136).astype(np.uint8)
    r = np.exp2(rng.uniform(-2, 2, N)).astype(np.float32)
    y = _run(a, asc, b, bsc, M, N, K, "MXINT4", r, torch.float32)
    ref = oracle_lib.quantized_linear(a, asc, M, b, bsc, N, K, "MXINT4", r=r)
    mi, ni = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    _, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, "MXINT4", mi.ravel(), ni.ravel(), r=r)
    assert np.all(np.abs(y - ref) <= _tol("MXFP6_E2M3", K, absy.reshape(M, N), ref, torch.float32))


# ---- NVFP4 on the f16 matrix cores.  Every element e2m1 * e4m3 is exact in fp16, so the
# products are exact and only fp32 sums round: the instructions' internal sums of 32 and the
# accumulation over K/32 of them (bound (K/32 + 2) 2^-24 + 2^-21 of sum |a b|, the last
# term leaving room for an internal sum kept in fewer bits), then the tensor-scale product,
# its multiply and the r multiply (3 more roundings of the result).

def _nv_inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = pack_codes(rng.integers(0, 16, M * K).astype(np.uint8), 4)
    b = pack_codes(rng.integers(0, 16, N * K).astype(np.uint8), 4)
    # E4M3 block scales over every finite non-negative code: zero, subnormals, up to 448
    asc = rng.integers(0, 0x7F, M * K // 16).astype(np.uint8)
    bsc = rng.integers(0, 0x7F, N * K // 16).astype(np.uint8)
    asc[:2], bsc[:2] = [1, 0x7E], [0x7E, 0]
    r = np.exp2(rng.uniform(-2, 2, N)).astype(np.float32)
    ats, bts = np.float32(rng.uniform(1e-3, 4.0)), np.float32(rng.uniform(1e-3, 4.0))
    return a, asc, b, bsc, r, ats, bts


def _nv_tol(K, absy, y, out_dtype):
    t = ((K // 32 + 5) * 2.0 ** -24 + 2.0 ** -21) * absy
    if out_dtype == torch.bfloat16:
        t = t + 2.0 ** -8 * (np.abs(y) + t)
    return t + 1e-37


def _nv_run(a, asc, b, bsc, M, N, K, r, ats, bts, out_dtype):
    dev = lambda x: torch.from_numpy(x).to(DEV)
    y = dq.quantized_linear(dev(a), dev(asc), dev(b), dev(bsc), M, N, K, "NVFP4",
                            r=None if r is None else to_dev(r), out_dtype=out_dtype,
                            a_tensor_scale=to_dev(np.array([ats])),
                            b_tensor_scale=to_dev(np.array([bts])))
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("shape", [(100, 70, 384), (1, 16, 32), (130, 257, 4128), (256, 256, 1024)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_nvfp4_random_codes(oracle_lib, shape, out_dtype):
    """Ragged M and N tiles; K = 32 and 4128 leave the last stage half empty."""
    M, N, K = shape
    print(f"[linear] NVFP4 {M}x{N}x{K} {out_dtype}", flush=True)
    a, asc, b, bsc, r, ats, bts = _nv_inputs(M, N, K, M + N + K)
    for rr in (r, None):
        y = _nv_run(a, asc, b, bsc, M, N, K, rr, ats, bts, out_dtype)
        ref = oracle_lib.quantized_linear(a, asc, M, b, bsc, N, K, "NVFP4", r=rr, a_ts=ats, b_ts=bts)
        mi, ni = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        _, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, "NVFP4", mi.ravel(),
                                                      ni.ravel(), r=rr, a_ts=ats, b_ts=bts)
        absy = absy.reshape(M, N)
        err = np.abs(y - ref)
        print(f"[linear] NVFP4 max err / sum|ab| = {float((err / (absy + 1e-300)).max()):.3g}", flush=True)
        assert np.all(err <= _nv_tol(K, absy, ref, out_dtype))


def test_nvfp4_full_size_sampled(oracle_lib):
    """2048 tokens x 4096 outputs x 14336 inputs (the down projection): 256 sampled entries."""
    M, N, K = 2048, 4096, 14336
    print(f"[linear] NVFP4 {M}x{N}x{K}", flush=True)
    a, asc, b, bsc, r, ats, bts = _nv_inputs(M, N, K, 9)
    y = _nv_run(a, asc, b, bsc, M, N, K, r, ats, bts, torch.float32)
    rng = np.random.default_rng(10)
    mi, ni = rng.integers(0, M, 256), rng.integers(0, N, 256)
    mi[:4], ni[:4] = [0, M - 1, 0, M - 1], [0, 0, N - 1, N - 1]
    ref, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, "NVFP4", mi, ni, r=r,
                                                    a_ts=ats, b_ts=bts)
    assert np.all(np.abs(y[mi, ni] - ref) <= _nv_tol(K, absy, ref, torch.float32))


def test_nvfp4_layer_from_solved_weights(oracle_lib):
    """512 x 4096 slice of the q projection solved in NVFP4 (T = 4), 256 tokens quantised
    with its column scales; the layer uses both tensor scales."""
    W, _, _, _, _ = synth.workload("q4096x4096_mxfp4")
    W = np.ascontiguousarray(W[:512])
    X = synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(256, 4096), 3)
    res = dq.solve(to_dev(W), "NVFP4", 4)
    cx, sx, tx = dq.rescale_quantize_acts(to_dev(X), res["c"], "NVFP4")
    y = dq.quantized_linear(cx, sx, res["codes"], res["scales"], 256, 512, 4096, "NVFP4",
                            r=res["r"], a_tensor_scale=tx, b_tensor_scale=res["tscale"])
    torch.cuda.synchronize()
    yc = y.cpu().numpy().astype(np.float64)
    ats, bts = float(tx.cpu()[0]), float(res["tscale"].cpu()[0])
    args = (cx.cpu().numpy(), sx.cpu().numpy(), 256, res["codes"].cpu().numpy(),
            res["scales"].cpu().numpy(), 512, 4096, "NVFP4")
    rr = res["r"].cpu().numpy()
    ref = oracle_lib.quantized_linear(*args, r=rr, a_ts=ats, b_ts=bts)
    mi, ni = np.meshgrid(np.arange(256), np.arange(512), indexing="ij")
    _, absy = oracle_lib.quantized_linear_entries(*args, mi.ravel(), ni.ravel(), r=rr, a_ts=ats, b_ts=bts)
    assert np.all(np.abs(yc - ref) <= _nv_tol(4096, absy.reshape(256, 512), ref, torch.float32))
    Xf = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Wf = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = Xf @ Wf.T
    rel = np.linalg.norm(yc - exact) / np.linalg.norm(exact)
    print(f"[linear] W4A4 NVFP4 layer relative error vs bf16 product: {rel:.4f}", flush=True)
    assert rel < 0.5


@pytest.mark.parametrize("fmt", ["MXFP4", "MXFP6_E2M3", "NVFP4", "INT4"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_output_row_pitch(oracle_lib, fmt, out_dtype):
    """Y written into a wider buffer (ldy = N + 37): the columns past N keep their contents,
    the first N equal the contiguous call bitwise (direct-to-LDS, register-staged and NVFP4
    kernels)."""
    M, N, K = 130, 100, 512
    group = None
    if fmt == "NVFP4":
        a, asc, b, bsc, r, ats, bts = _nv_inputs(M, N, K, 21)
        ts = dict(a_tensor_scale=to_dev(np.array([ats])), b_tensor_scale=to_dev(np.array([bts])))
    elif fmt == "INT4":
        group = 64
        a, asc, b, bsc, r = _i4_inputs(M, N, K, group, 21)
        asc, bsc = asc.view(np.int16), bsc.view(np.int16)
        ts = dict(a_tensor_scale=None, b_tensor_scale=None)
    else:
        a, asc, b, bsc, r = _inputs(fmt, M, N, K, 21)
        ts = dict(a_tensor_scale=None, b_tensor_scale=None)
    dev = lambda x: torch.from_numpy(x).to(DEV)
    A, As, B, Bs, R = dev(a), dev(asc), dev(b), dev(bsc), to_dev(r)
    y0 = dq.quantized_linear(A, As, B, Bs, M, N, K, fmt, r=R, out_dtype=out_dtype, group=group, **ts)
    wide = torch.full((M, N + 37), -7.0, dtype=out_dtype, device=DEV)
    view = wide[:, :N]
    assert view.stride(0) == N + 37
    dq.dq_quantized_linear(dq.spec_of(fmt, group), A, As, ts["a_tensor_scale"], M, B, Bs,
                           ts["b_tensor_scale"], N, K, R, view)
    torch.cuda.synchronize()
    assert torch.equal(view, y0)
    assert torch.all(wide[:, N:] == -7.0)


def test_nvfp4_both_kernels(oracle_lib):
    """K = 1024 with 4-byte-aligned scales takes the kernel that dequantises in registers;
    the same scales at an odd address take the one that dequantises into LDS.  They sum K
    in different orders, so each is checked against the oracle (not bitwise against the
    other)."""
    M, N, K = 160, 200, 1024
    a, asc, b, bsc, r, ats, bts = _nv_inputs(M, N, K, 41)
    dev = lambda x: torch.from_numpy(x).to(DEV)
    A, B = dev(a), dev(b)
    pad_a = torch.zeros(asc.size + 16, dtype=torch.uint8, device=DEV)
    pad_b = torch.zeros(bsc.size + 16, dtype=torch.uint8, device=DEV)
    pad_a[1:1 + asc.size] = dev(asc)
    pad_b[1:1 + bsc.size] = dev(bsc)
    ts = dict(a_tensor_scale=to_dev(np.array([ats])), b_tensor_scale=to_dev(np.array([bts])))
    ref = oracle_lib.quantized_linear(a, asc, M, b, bsc, N, K, "NVFP4", r=r, a_ts=ats, b_ts=bts)
    mi, ni = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    _, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, "NVFP4", mi.ravel(),
                                                  ni.ravel(), r=r, a_ts=ats, b_ts=bts)
    tol = _nv_tol(K, absy.reshape(M, N), ref, torch.float32)
    for sa, sb in ((dev(asc), dev(bsc)), (pad_a[1:1 + asc.size], pad_b[1:1 + bsc.size])):
        y = dq.quantized_linear(A, sa, B, sb, M, N, K, "NVFP4", r=to_dev(r), **ts)
        torch.cuda.synchronize()
        assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - ref) <= tol)


@pytest.mark.parametrize("fmt", ["MXFP4", "NVFP4"])
def test_output_offsets_beyond_2_31(oracle_lib, fmt):
    """A 32768 x 65552 bf16 output (element offsets past 2^31; N not a multiple of the tile)
    with K = 256: entries sampled across it, including the last rows and columns, against
    the oracle."""
    M, N, K = 32768, 65552, 256
    print(f"[linear] {fmt} {M}x{N}x{K} (4.3 GB output)", flush=True)
    rng = np.random.default_rng(51)
    if fmt == "NVFP4":
        a, asc, b, bsc, r, ats, bts = _nv_inputs(M, N, K, 51)
        ts = dict(a_tensor_scale=to_dev(np.array([ats])), b_tensor_scale=to_dev(np.array([bts])))
        kw = dict(a_ts=ats, b_ts=bts)
    else:
        a, asc, b, bsc, r = _inputs(fmt, M, N, K, 51)
        ts, kw = {}, {}
    dev = lambda x: torch.from_numpy(x).to(DEV)
    y = dq.quantized_linear(dev(a), dev(asc), dev(b), dev(bsc), M, N, K, fmt, r=to_dev(r),
                            out_dtype=torch.bfloat16, **ts)
    mi, ni = rng.integers(0, M, 400), rng.integers(0, N, 400)
    mi[:6], ni[:6] = [M - 1, M - 1, M - 1, 0, M // 2, M - 2], [N - 1, 0, N - 17, N - 1, N - 1, N - 2]
    assert int(mi.max()) * N + int(ni.max()) > 2 ** 31
    got = y[torch.from_numpy(mi).to(DEV), torch.from_numpy(ni).to(DEV)].float().cpu().numpy().astype(np.float64)
    del y
    torch.cuda.synchronize()
    ref, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, fmt, mi, ni, r=r, **kw)
    tol = (_nv_tol if fmt == "NVFP4" else (lambda K_, ab, yy, od: _tol(fmt, K_, ab, yy, od)))(K, absy, ref, torch.bfloat16)
    assert np.all(np.abs(got - ref) <= tol)


# ---- INT4 (bf16 scale per group of 64 or 128) on the int8 matrix cores.  Each group's
# integer dot product is exact in int32; per group the kernel rounds once converting
# P * sa * sb into fp32 (the int32 and the bf16 scale product are exact) and once adding it
# to the fp32 sum, then the r multiply rounds: |y - ref| <= (K/g + 3) 2^-24 sum |a b| |r|.

def _i4_inputs(M, N, K, g, seed):
    rng = np.random.default_rng(seed)
    a = pack_codes(rng.integers(0, 16, M * K).astype(np.uint8), 4)     # nibble 8 = -8 included
    b = pack_codes(rng.integers(0, 16, N * K).astype(np.uint8), 4)
    bf = lambda x: (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    asc = bf(np.exp2(rng.uniform(-8, 8, M * K // g)) * rng.uniform(1, 2, M * K // g))
    bsc = bf(np.exp2(rng.uniform(-8, 8, N * K // g)) * rng.uniform(1, 2, N * K // g))
    r = np.exp2(rng.uniform(-2, 2, N)).astype(np.float32)
    return a, asc, b, bsc, r


def _i4_splits(M, N, K, g):
    """K splits the library takes for this shape (from its workspace size: splits x M x N
    rounded to 4 fp32 values)."""
    nb = dq.dq_quantized_linear_workspace_bytes(dq.spec_of("INT4", g), M, N, K)
    return nb // (M * ((N + 3) // 4 * 4) * 4) if nb else 1


def _i4_tol(K, g, absy, y, out_dtype, splits=1):
    t = (K // g + splits + 3) * 2.0 ** -24 * absy
    if out_dtype == torch.bfloat16:
        t = t + 2.0 ** -8 * (np.abs(y) + t)
    return t + 1e-37


def _i4_run(a, asc, b, bsc, M, N, K, g, r, out_dtype):
    dev = lambda x: torch.from_numpy(x).to(DEV)
    y = dq.quantized_linear(dev(a), dev(asc.view(np.int16)), dev(b), dev(bsc.view(np.int16)),
                            M, N, K, "INT4", r=None if r is None else to_dev(r),
                            out_dtype=out_dtype, group=g)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("shape", [(100, 70, 384), (1, 16, 128), (130, 257, 4224), (256, 256, 1024),
                                   (3, 5, 64)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_int4_random_codes(oracle_lib, g, shape, out_dtype):
    """Ragged M and N tiles; K = 384 and 4224 end in a half stage, K = 64 (groups of 64
    only) in a quarter stage."""
    M, N, K = shape
    if K % g:
        pytest.skip("K is not a multiple of the group")
    print(f"[linear] INT4 g{g} {M}x{N}x{K} {out_dtype}", flush=True)
    a, asc, b, bsc, r = _i4_inputs(M, N, K, g, M + N + K + g)
    for rr in (r, None):
        y = _i4_run(a, asc, b, bsc, M, N, K, g, rr, out_dtype)
        ref = oracle_lib.quantized_linear(a, asc, M, b, bsc, N, K, "INT4", r=rr, group=g)
        mi, ni = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        _, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, "INT4", mi.ravel(),
                                                      ni.ravel(), r=rr, group=g)
        absy = absy.reshape(M, N)
        err = np.abs(y - ref)
        print(f"[linear] INT4 max err / sum|ab| = {float((err / (absy + 1e-300)).max()):.3g}", flush=True)
        assert np.all(err <= _i4_tol(K, g, absy, ref, out_dtype, _i4_splits(M, N, K, g)))


def test_int4_exact_small_integers(oracle_lib):
    """Scales 1.0 and K = 256: every output is an integer below 2^24, so the layer is exact."""
    M, N, K = 64, 48, 256
    rng = np.random.default_rng(21)
    a = pack_codes(rng.integers(0, 16, M * K).astype(np.uint8), 4)
    b = pack_codes(rng.integers(0, 16, N * K).astype(np.uint8), 4)
    asc = np.full(M * K // 64, 0x3F80, np.uint16)
    bsc = np.full(N * K // 64, 0x3F80, np.uint16)
    y = _i4_run(a, asc, b, bsc, M, N, K, 64, None, torch.float32)
    ref = oracle_lib.quantized_linear(a, asc, M, b, bsc, N, K, "INT4", group=64)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("K", [4096, 14336])
def test_int4_full_size_sampled(oracle_lib, K):
    """2048 tokens x 4096 outputs x K inputs (the q/o and the down projection), groups of
    64: 384 sampled entries, the four corners among them."""
    M, N, g = 2048, 4096, 64
    print(f"[linear] INT4 g64 {M}x{N}x{K}", flush=True)
    a, asc, b, bsc, r = _i4_inputs(M, N, K, g, K)
    y = _i4_run(a, asc, b, bsc, M, N, K, g, r, torch.float32)
    rng = np.random.default_rng(K + 1)
    mi, ni = rng.integers(0, M, 384), rng.integers(0, N, 384)
    mi[:4], ni[:4] = [0, M - 1, 0, M - 1], [0, 0, N - 1, N - 1]
    ref, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, "INT4", mi, ni, r=r,
                                                    group=g)
    assert np.all(np.abs(y[mi, ni] - ref) <= _i4_tol(K, g, absy, ref, torch.float32))


def test_int4_layer_from_solved_weights(oracle_lib):
    """W4A4 with INT4 groups of 64 end to end on a 512 x 4096 slice of a weight: solve
    (T = 4), quantise 256 tokens with the solved column scales, run the layer; the output
    matches the oracle's product of the same codes and approximates X W^T."""
    W, _, _, _, _ = synth.workload("q4096x4096_mxfp4")
    W = np.ascontiguousarray(W[:512])
    X = synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(256, 4096), 3)
    res = dq.solve(to_dev(W), "INT4", 4, group=64)
    codes_x, scales_x, _ = dq.rescale_quantize_acts(to_dev(X), res["c"], "INT4", group=64)
    y = dq.quantized_linear(codes_x, scales_x, res["codes"], res["scales"], 256, 512, 4096, "INT4",
                            r=res["r"], group=64)
    torch.cuda.synchronize()
    yc = y.cpu().numpy().astype(np.float64)
    u16 = lambda t: t.cpu().numpy().view(np.uint16)
    args = (codes_x.cpu().numpy(), u16(scales_x), 256, res["codes"].cpu().numpy(),
            u16(res["scales"]), 512, 4096, "INT4")
    rn = res["r"].cpu().numpy()
    ref = oracle_lib.quantized_linear(*args, r=rn, group=64)
    mi, ni = np.meshgrid(np.arange(256), np.arange(512), indexing="ij")
    _, absy = oracle_lib.quantized_linear_entries(*args, mi.ravel(), ni.ravel(), r=rn, group=64)
    assert np.all(np.abs(yc - ref) <= _i4_tol(4096, 64, absy.reshape(256, 512), ref, torch.float32))
    Xf = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Wf = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = Xf @ Wf.T
    rel = np.linalg.norm(yc - exact) / np.linalg.norm(exact)
    print(f"[linear] W4A4 INT4 g64 layer relative error vs bf16 product: {rel:.4f}", flush=True)
    assert rel < 0.5


def test_int4_argument_errors():
    """Host-side checks, before any launch: K not a multiple of the group, odd scale address."""
    z = lambda n, dt=torch.uint8: torch.zeros(n, dtype=dt, device=DEV)
    with pytest.raises(RuntimeError):
        dq.quantized_linear(z(48), z(2, torch.int16), z(48), z(2, torch.int16), 1, 1, 96, "INT4",
                            group=64)
    buf = z(64)
    with pytest.raises(RuntimeError):
        dq.quantized_linear(z(32), buf[1:5], z(32), z(2, torch.int16), 1, 1, 64, "INT4", group=64)


@pytest.mark.parametrize("shape", [(82, 4096, 4096), (1, 1024, 4096), (16, 4096, 14336), (40, 14336, 4096),
                                   (5, 300, 640), (130, 1024, 4096)])
def test_int4_split_k_few_tokens(oracle_lib, shape):
    """Few tokens (the listing page's Table 11 forwards of 82 tokens, and decoding): the
    layer splits K over a workspace (32-row tiles up to 96 tokens, 128-row tiles beyond).  Sampled entries (all of them for the small case)
    against the oracle within the split bound; two calls bitwise equal; the unsplit kernel
    on the same codes within the same bound."""
    M, N, K = shape
    g = 64
    ks = _i4_splits(M, N, K, g)
    print(f"[linear] INT4 split K {M}x{N}x{K}: {ks} splits", flush=True)
    assert ks > 1
    a, asc, b, bsc, r = _i4_inputs(M, N, K, g, M * 7 + N + K)
    dev = lambda x: torch.from_numpy(x).to(DEV)
    A, As, B, Bs, R = dev(a), dev(asc.view(np.int16)), dev(b), dev(bsc.view(np.int16)), to_dev(r)
    y1 = dq.quantized_linear(A, As, B, Bs, M, N, K, "INT4", r=R, group=g)
    y2 = dq.quantized_linear(A, As, B, Bs, M, N, K, "INT4", r=R, group=g)
    y0 = dq.quantized_linear(A, As, B, Bs, M, N, K, "INT4", r=R, group=g, split=False)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    rng = np.random.default_rng(M + N)
    if M * N <= 4096:
        mi, ni = [x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij")]
    else:
        mi, ni = rng.integers(0, M, 384), rng.integers(0, N, 384)
        mi[:4], ni[:4] = [0, M - 1, 0, M - 1], [0, 0, N - 1, N - 1]
    ref, absy = oracle_lib.quantized_linear_entries(a, asc, M, b, bsc, N, K, "INT4", mi, ni, r=r, group=g)
    for y, splits in ((y1, ks), (y0, 1)):
        got = y.cpu().numpy().astype(np.float64)[mi, ni]
        assert np.all(np.abs(got - ref) <= _i4_tol(K, g, absy, ref, torch.float32, splits)), splits


@pytest.mark.parametrize("g", [64, 128])
def test_int4_small_tile_bitwise(g):
    """Up to 96 tokens the INT4 layer tiles the activations 32 rows at a time, beyond that
    128; each output element is the same sum in the same order either way, so the first rows
    of a 200-token product equal the 1-, 40- and 96-token products of those rows bit for bit
    (unsplit, fp32 and bf16 out)."""
    Mb, N, K = 200, 300, 1024
    a, asc, b, bsc, r = _i4_inputs(Mb, N, K, g, 77 + g)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    B, Bs, R = dev(b), dev(bsc.view(np.int16)), to_dev(r)
    for out in (torch.float32, torch.bfloat16):
        yb = dq.quantized_linear(dev(a), dev(asc.view(np.int16)), B, Bs, Mb, N, K, "INT4", r=R,
                                 out_dtype=out, group=g, split=False)
        for M in (1, 40, 96):
            print(f"[linear] INT4 g{g} 32-row tiles, {M} of {Mb} rows, {out}", flush=True)
            A = dev(a.reshape(Mb, K // 2)[:M])
            As = dev(asc.view(np.int16).reshape(Mb, K // g)[:M])
            ys = dq.quantized_linear(A, As, B, Bs, M, N, K, "INT4", r=R, out_dtype=out, group=g,
                                     split=False)
            torch.cuda.synchronize()
            assert torch.equal(ys, yb[:M]), (M, out)


def test_int4_split_workspace_reused():
    """One workspace kept across calls of different shapes and output types (as a forward
    keeps it), filled with what earlier calls left: every call equals the same call on a
    fresh workspace bit for bit."""
    g = 64
    shapes = [(82, 4096, 4096), (16, 4096, 14336), (5, 300, 640), (82, 14336, 4096), (82, 4096, 4096)]
    spec = dq.spec_of("INT4", g)
    nb = max(dq.dq_quantized_linear_workspace_bytes(spec, M, N, K) for M, N, K in shapes)
    ws = torch.full((nb,), 0x7F, dtype=torch.uint8, device=DEV)
    for k, (M, N, K) in enumerate(shapes):
        out = torch.bfloat16 if k % 2 else torch.float32
        print(f"[linear] INT4 split K reused workspace {M}x{N}x{K} {out}", flush=True)
        a, asc, b, bsc, r = _i4_inputs(M, N, K, g, 1000 + k)
        dev = lambda x: torch.from_numpy(x).to(DEV)
        A, As, B, Bs, R = dev(a), dev(asc.view(np.int16)), dev(b), dev(bsc.view(np.int16)), to_dev(r)
        y = torch.empty(M, N, dtype=out, device=DEV)
        dq.dq_quantized_linear_ws(spec, A, As, None, M, B, Bs, None, N, K, R, y, ws)
        ref = dq.quantized_linear(A, As, B, Bs, M, N, K, "INT4", r=R, out_dtype=out, group=g)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), (M, N, K)


def test_int4_split_workspace_errors():
    """A workspace smaller than the shape needs, or misaligned, is refused before any work."""
    M, N, K, g = 8, 256, 4096, 64
    spec = dq.spec_of("INT4", g)
    nb = dq.dq_quantized_linear_workspace_bytes(spec, M, N, K)
    assert nb > 0
    z = lambda n, dt=torch.uint8: torch.zeros(n, dtype=dt, device=DEV)
    a, asc, b, bsc = z(M * K // 2), z(M * K // g, torch.int16), z(N * K // 2), z(N * K // g, torch.int16)
    y = torch.empty(M, N, device=DEV)
    with pytest.raises(RuntimeError):
        dq.dq_quantized_linear_ws(spec, a, asc, None, M, b, bsc, None, N, K, None, y, z(nb - 16))
    buf = z(nb + 64)
    with pytest.raises(RuntimeError):
        dq.dq_quantized_linear_ws(spec, a, asc, None, M, b, bsc, None, N, K, None, y, buf[4:4 + nb])
