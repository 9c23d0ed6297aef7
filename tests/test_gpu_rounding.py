"""The library's device rounding and projection routines against the oracle's
brute-force implementations, on dense sets of fp32 inputs."""

import numpy as np
import pytest
import torch

import post_quantization_dq_amd as dq
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def _run(fn, x, out_dtype):
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    out = torch.empty(x.size, dtype=out_dtype, device=DEV)
    dq.dq_debug_round(fn, xt, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _binades(lo, hi):
    return np.arange(np.uint32((lo + 127) << 23), np.uint32((hi + 127) << 23), dtype=np.uint32).view(np.float32)


def test_e2m1_dense(oracle_lib):
    pos = _binades(-3, 3)
    specials = np.float32([0.0, -0.0, 1e-45, -1e-45, 1e-30, 7.0, 100.0, -1e30, 3.4e38, -6.5])
    for x in (pos, -pos[::3], specials):
        got = _run("e2m1", x, torch.uint8)
        want = oracle_lib.e2m1_encode(x)
        assert np.array_equal(got, want)


def test_e4m3_dense(oracle_lib):
    vals = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    bits = np.concatenate([vals, mids]).view(np.uint32).astype(np.int64)
    x = (bits[:, None] + np.arange(-2000, 2001)[None, :]).reshape(-1)
    x = x[(x >= 0) & (x < 0x7F800000)].astype(np.uint32).view(np.float32)
    rng = np.random.default_rng(0)
    x = np.concatenate([x, np.exp2(rng.uniform(-20, 12, 1 << 20)).astype(np.float32),
                        np.float32([0.0, 448.0, 464.0, 465.0, 1e9, 3.4e38])])
    got = _run("e4m3", x, torch.uint8)
    assert np.array_equal(got, oracle_lib.e4m3_encode(x))


def test_bf16_and_int4(oracle_lib):
    rng = np.random.default_rng(1)
    hi = rng.integers(0, 0x7F7F, 1 << 20, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    x = (hi[:, None] | lows[None, :]).reshape(-1).view(np.float32)
    x = np.concatenate([x, -x])
    got = _run("bf16", x, torch.float32)
    assert np.array_equal(got.view(np.uint32), oracle_lib.bf16_round(x).view(np.uint32))
    y = np.concatenate([np.arange(-9, 9, 0.125, dtype=np.float32),
                        rng.normal(0, 5, 1 << 20).astype(np.float32)])
    got = _run("int4", y, torch.int8)
    assert np.array_equal(got, oracle_lib.int_round(y, 7))


@pytest.mark.parametrize("fn,fmt", [("proj_mx", "MXFP4"), ("proj_e4m3", "NVFP4"), ("proj_bf16", "INT4")])
def test_projections(oracle_lib, fn, fmt):
    rng = np.random.default_rng(2)
    x = np.exp2(rng.uniform(-135, 130, 1 << 20)).astype(np.float32)
    ties = (np.float32(1.5) * np.exp2(np.arange(-126, 127))).astype(np.float32)
    x = np.concatenate([x, ties, np.float32([1e-45, 2.0 ** -127, 1.0, 448.0, 500.0, 3.4e38])])
    x = x[(x > 0) & np.isfinite(x)]
    got = _run(fn, x, torch.float32)
    assert np.array_equal(got.view(np.uint32), oracle_lib.project(fmt, x).view(np.uint32))
