"""dq_quantize_weights / dq_rescale_quantize_acts / dq_dequantize against the oracle:
codes, block scales and tensor scale bit-exact given identical scales."""

import numpy as np
import pytest
import torch

import post_quantization_dq_amd as dq
import synth
from gpu_util import ALL_FORMATS, DEV, GROUPS, scales_np, to_dev

pytestmark = pytest.mark.gpu

# (3, 16384): one pass of 1024 chunks; (3, 18944) and (2, 65536): several passes, the
# first ragged
SHAPES = [(64, 256), (37, 512), (3, 16384), (1, 128), (130, 14336), (3, 18944), (2, 65536)]


def _w(rows, cols, dtype, seed):
    spec = synth.MatrixSpec(rows, cols, "student_t", 0.02, nu=3, outliers=max(1, cols // 100),
                            outlier_scale=25.0, dtype=dtype, stream=40 + seed)
    return synth.matrix(spec, seed)


@pytest.mark.parametrize("fmt", ALL_FORMATS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_weights_bit_exact(oracle_lib, fmt, dtype, shape):
    rows, cols = shape
    if cols % GROUPS[fmt]:
        pytest.skip("shape not a whole number of blocks")
    W = _w(rows, cols, dtype, 1)
    rng = np.random.default_rng(rows * 7 + cols)
    for with_scales in (False, True):
        r = c = None
        if with_scales:
            r = oracle_lib.project(fmt, np.exp2(rng.uniform(-2, 2, rows)).astype(np.float32))
            c = oracle_lib.project(fmt, np.exp2(rng.uniform(-2, 2, cols)).astype(np.float32))
        codes, scales, ts, _ = oracle_lib.quantize_weights(W, r, c, fmt)
        gc, gs, gt = dq.quantize_weights(to_dev(W), None if r is None else to_dev(r),
                                         None if c is None else to_dev(c), fmt)
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), codes)
        assert np.array_equal(scales_np(gs, fmt), scales)
        if fmt == "NVFP4":
            assert gt.item() == np.float32(ts)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_weights_int4_group64_bit_exact(oracle_lib, dtype, shape):
    """INT4 with 64-element groups (the listing page's INT4 setting, Tables 1, 6, 10-12)."""
    rows, cols = shape
    W = _w(rows, cols, dtype, 2)
    rng = np.random.default_rng(rows * 11 + cols)
    for with_scales in (False, True):
        r = c = None
        if with_scales:
            r = oracle_lib.project("INT4", np.exp2(rng.uniform(-2, 2, rows)).astype(np.float32))
            c = oracle_lib.project("INT4", np.exp2(rng.uniform(-2, 2, cols)).astype(np.float32))
        codes, scales, _, _ = oracle_lib.quantize_weights(W, r, c, "INT4", 64)
        gc, gs, _ = dq.quantize_weights(to_dev(W), None if r is None else to_dev(r),
                                        None if c is None else to_dev(c), "INT4", group=64)
        torch.cuda.synchronize()
        assert gs.numel() == rows * cols // 64
        assert np.array_equal(gc.cpu().numpy(), codes)
        assert np.array_equal(scales_np(gs, "INT4"), scales)


def test_rescale_quantize_acts_int4_group64(oracle_lib):
    X = synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(96, 1024), 0)
    rng = np.random.default_rng(4)
    c = oracle_lib.project("INT4", np.exp2(rng.uniform(-3, 3, 1024)).astype(np.float32))
    for cc in (None, c):
        codes, scales, _, _ = oracle_lib.rescale_quantize_acts(X, cc, "INT4", 64)
        gc, gs, _ = dq.rescale_quantize_acts(to_dev(X), None if cc is None else to_dev(cc), "INT4", group=64)
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), codes)
        assert np.array_equal(scales_np(gs, "INT4"), scales)


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_rescale_quantize_acts_bit_exact(oracle_lib, fmt):
    X = synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(96, 1024), 0)
    rng = np.random.default_rng(3)
    c = oracle_lib.project(fmt, np.exp2(rng.uniform(-3, 3, 1024)).astype(np.float32))
    for cc in (None, c):
        codes, scales, ts, _ = oracle_lib.rescale_quantize_acts(X, cc, fmt)
        gc, gs, gt = dq.rescale_quantize_acts(to_dev(X), None if cc is None else to_dev(cc), fmt)
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), codes)
        assert np.array_equal(scales_np(gs, fmt), scales)
        if fmt == "NVFP4":
            assert gt.item() == np.float32(ts)


def _check_acts(oracle_lib, X, cc, fmt, group, got):
    gc, gs, gt = got
    codes, scales, ts, _ = oracle_lib.rescale_quantize_acts(X, cc, fmt, group)
    assert np.array_equal(gc.cpu().numpy(), codes)
    assert np.array_equal(scales_np(gs, fmt), scales)
    if fmt == "NVFP4":
        assert gt.item() == np.float32(ts)


@pytest.mark.parametrize("fmt", ALL_FORMATS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(70, 1024), (5, 4096), (1, 128)])
def test_rescale_quantize_acts_multi(oracle_lib, fmt, dtype, shape):
    """Several column-scale vectors over one activation matrix (q/k/v-style): every output
    bit-exact with the oracle and with the single-output entry point."""
    from dataclasses import replace

    tokens, cols = shape
    if cols % GROUPS[fmt]:
        pytest.skip("shape not a whole number of blocks")
    spec = replace(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(tokens, cols), dtype=dtype)
    X = synth.matrix(spec, 2)
    rng = np.random.default_rng(tokens + cols)
    cs = [oracle_lib.project(fmt, np.exp2(rng.uniform(-3, 3, cols)).astype(np.float32)),
          None,
          oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, cols)).astype(np.float32))]
    Xd = to_dev(X)
    got = dq.rescale_quantize_acts_multi(Xd, [None if c is None else to_dev(c) for c in cs], fmt)
    torch.cuda.synchronize()
    assert len(got) == 3
    for cc, g in zip(cs, got):
        if dtype == "bf16":   # the oracle's activation entry reads bf16 activations
            _check_acts(oracle_lib, X, cc, fmt, GROUPS[fmt], g)
        one = dq.rescale_quantize_acts(Xd, None if cc is None else to_dev(cc), fmt)
        torch.cuda.synchronize()
        for a, b in zip(g, one):
            assert torch.equal(a, b)


@pytest.mark.parametrize("fmt", ["NVFP4", "MXFP6_E3M2", "INT4"])
@pytest.mark.parametrize("n_out", [1, 3])
def test_rescale_quantize_acts_multi_wide(oracle_lib, fmt, n_out):
    """Rows wider than 16384 columns (two passes): column scales staged in LDS (one output)
    and read from global memory (three outputs), each output bit-exact with the oracle."""
    tokens, cols = 5, 18944
    X = synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(tokens, cols), 6)
    rng = np.random.default_rng(12)
    cs = [oracle_lib.project(fmt, np.exp2(rng.uniform(-3, 3, cols)).astype(np.float32))
          for _ in range(n_out)]
    got = dq.rescale_quantize_acts_multi(to_dev(X), [to_dev(c) for c in cs], fmt)
    torch.cuda.synchronize()
    for c, g in zip(cs, got):
        _check_acts(oracle_lib, X, c, fmt, GROUPS[fmt], g)


@pytest.mark.parametrize("fmt", ["NVFP4", "MXINT4", "INT8"])
def test_rescale_quantize_acts_multi_max_outputs(oracle_lib, fmt):
    """DQ_MAX_MULTI outputs in one call, then a smaller call reusing nothing: each output
    equals the single-output entry point's; the NVFP4 tensor scale is per output."""
    X = synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(33, 2048), 5)
    Xd = to_dev(X)
    rng = np.random.default_rng(11)
    cs = [to_dev(oracle_lib.project(fmt, np.exp2(rng.uniform(-4, 4, 2048)).astype(np.float32)))
          for _ in range(dq.DQ_MAX_MULTI)]
    for n in (dq.DQ_MAX_MULTI, 2):
        got = dq.rescale_quantize_acts_multi(Xd, cs[:n], fmt)
        torch.cuda.synchronize()
        tss = set()
        for c, g in zip(cs[:n], got):
            one = dq.rescale_quantize_acts(Xd, c, fmt)
            torch.cuda.synchronize()
            for a, b in zip(g, one):
                assert torch.equal(a, b)
            tss.add(float(g[2].item()))
        if fmt == "NVFP4":
            assert len(tss) > 1
    _check_acts(oracle_lib, X, cs[1].cpu().numpy(), fmt, GROUPS[fmt], got[1])


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_dequantize_matches_oracle(oracle_lib, fmt):
    W = _w(48, 512, "bf16", 4)
    codes, scales, ts, qhat = oracle_lib.quantize_weights(W, None, None, fmt)
    wide_scale = fmt in ("INT4", "INT8")
    sdt = torch.int16 if wide_scale else torch.uint8
    sc = torch.from_numpy(scales.view(np.int16) if wide_scale else scales).to(DEV)
    out = dq.dequantize(torch.from_numpy(codes).to(DEV), sc, torch.tensor([ts], dtype=torch.float32, device=DEV),
                        48, 512, fmt)
    torch.cuda.synchronize()
    assert sc.dtype == sdt
    assert np.array_equal(out.cpu().numpy().view(np.uint32), qhat.view(np.uint32))
    r = np.linspace(0.5, 2, 48).astype(np.float32)
    c = np.linspace(0.25, 4, 512).astype(np.float32)
    out2 = dq.dequantize(torch.from_numpy(codes).to(DEV), sc, torch.tensor([ts], dtype=torch.float32, device=DEV),
                         48, 512, fmt, r=to_dev(r), c=to_dev(c))
    torch.cuda.synchronize()
    want = ((r[:, None] * qhat).astype(np.float32) * c[None, :]).astype(np.float32)
    assert np.array_equal(out2.cpu().numpy(), want)


def test_empty_inputs():
    W = torch.empty(0, 256, dtype=torch.bfloat16, device=DEV)
    gc, gs, gt = dq.quantize_weights(W, None, None, "NVFP4")
    torch.cuda.synchronize()
    assert gc.numel() == 0


def test_k_proj_activation_sqnr(oracle_lib):
    """The k_proj workload end to end: solve W (MXINT4, T = 16) on the GPU, rescale the
    2048-token activations by the solved column scales and MXINT4-quantise them.  The
    activation codes must equal the oracle's for the same c, and the activation-domain
    SQNR (with and without the column scales) is reported."""
    W, X, fmt, g, T = synth.workload("k1024x4096_mxint4")
    res = dq.solve(to_dev(W), fmt, T)
    torch.cuda.synchronize()
    c = res["c"]
    ref = oracle_lib.solve(W, fmt, T)
    assert np.array_equal(c.cpu().numpy(), ref["c"])
    Xd = to_dev(X)
    out = {}
    for label, cv in (("with beta", c), ("without beta", None)):
        codes, scales, ts = dq.rescale_quantize_acts(Xd, cv, fmt)
        torch.cuda.synchronize()
        cn = None if cv is None else cv.cpu().numpy()
        rcodes, rscales, rts, _ = oracle_lib.rescale_quantize_acts(X, cn, fmt)
        assert np.array_equal(codes.cpu().numpy(), rcodes)
        assert np.array_equal(scales_np(scales, fmt), rscales)
        out[label] = oracle_lib.act_sqnr(X, cn, codes.cpu().numpy(), scales_np(scales, fmt),
                                         float(ts.item()), fmt)
        assert np.isfinite(out[label])
    print(f"[sqnr] k_proj MXINT4 activation SQNR: {out['with beta']:.3f} dB with the column "
          f"scales, {out['without beta']:.3f} dB without", flush=True)


def test_nvfp4_tensor_scale_limit(oracle_lib):
    """Around the NVFP4 limit derived from fp32 arithmetic (1 / (2^-9 s_t) overflows for s_t
    at or below about 2^-119): codes, block scales and tensor scale bit-exact with the
    oracle on both sides of it, zero codes and flag 16 in a solve below it."""
    rng = np.random.default_rng(8)
    base = (rng.standard_normal((4, 64)) * 0.25).astype(np.float32)
    edge = np.float32(2.0 ** -119) * np.float32(2688)
    for A in (np.nextafter(edge, np.float32(0)), edge, np.nextafter(edge, np.float32(1)),
              np.float32(edge * 1.001), np.float32(edge * 4), np.float32(2.0 ** -100), np.float32(1e-44)):
        V = (base / np.abs(base).max() * A).astype(np.float32)
        V[0, 0] = A
        codes, scales, ts, _ = oracle_lib.quantize_weights(V, None, None, "NVFP4")
        gc, gs, gt = dq.quantize_weights(to_dev(V), None, None, "NVFP4")
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), codes), A
        assert np.array_equal(gs.cpu().numpy(), scales), A
        assert gt.item() == np.float32(ts), A
    V = (base / np.abs(base).max() * np.float32(2.0 ** -112)).astype(np.float32)
    got = dq.solve(to_dev(V), "NVFP4", 2)
    torch.cuda.synchronize()
    assert got["flags"] & 16
    assert torch.count_nonzero(got["codes"]).item() == 0 and got["tscale"].item() == 0.0
