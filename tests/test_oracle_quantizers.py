"""Pins for the oracle's block fake-quantisers FQ_f (INT4 with groups 128 and 64 -- the
listing page's tables use G = 64 -- MXINT4, MXFP4, NVFP4).

Pinned by what the format definitions fix independently of the oracle's code:
exact invariants (idempotence for MX, power-of-two equivariance, sign symmetry,
block-aligned permutation equivariance), the scale rules reduced to library routines
(torch's bf16 / float8_e4m3fn casts, frexp), the nearest-point error bound, and
brute-force nearest-point search on small blocks.
"""

import json
from pathlib import Path

import numpy as np
import pytest
import torch

import synth

FORMATS = ["INT4", "MXINT4", "MXFP4", "NVFP4"]
GROUPS = {"INT4": 128, "MXINT4": 32, "MXFP4": 32, "NVFP4": 16}
# (format, group): INT4 with both group sizes
CASES = [("INT4", 128), ("INT4", 64), ("MXINT4", 32), ("MXFP4", 32), ("NVFP4", 16)]
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _rand(rows, cols, seed, outliers=True):
    rng = np.random.default_rng(seed)
    V = rng.standard_t(4, (rows, cols)) * 0.02
    if outliers:
        V[:, rng.choice(cols, max(1, cols // 50), replace=False)] *= 20
    V[rng.random((rows, cols)) < 0.01] = 0.0
    return V.astype(np.float32)


def _blocks(x, g):
    return x.reshape(x.shape[0], -1, g)


@pytest.mark.parametrize("fmt,g", CASES)
def test_dequantize_roundtrip_and_grid(oracle_lib, fmt, g):
    V = _rand(24, 256, 1)
    codes, scales, ts, qhat, flags = oracle_lib.fq(V, fmt, g)
    assert codes.size == V.size // 2 and scales.size == V.size // g
    deq = oracle_lib.dequantize(codes, scales, ts, fmt, *V.shape, group=g)
    assert np.array_equal(deq.view(np.uint32), qhat.view(np.uint32))
    # every element lies on the element grid times its block scale
    nib = np.stack([codes & 0xF, codes >> 4], axis=1).reshape(V.shape)
    if fmt in ("INT4", "MXINT4"):
        q = np.where(nib & 8, nib.astype(np.int64) - 16, nib).astype(np.float64)
        assert np.all(np.abs(q) <= 7)
    else:
        q = np.where(nib & 8, -E2M1[nib & 7], E2M1[nib & 7])
    if fmt == "INT4":
        s = (scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.array_equal(qhat.astype(np.float64), (_blocks(q, g) * s.reshape(24, -1, 1)).reshape(V.shape))
    elif fmt in ("MXINT4", "MXFP4"):
        e = scales.astype(np.int64).reshape(24, -1, 1) - 127 - (2 if fmt == "MXINT4" else 0)
        assert np.array_equal(qhat.astype(np.float64), np.ldexp(_blocks(q, g), e).reshape(V.shape))
    else:
        sb = torch.from_numpy(scales).view(torch.float8_e4m3fn).float().numpy()
        d = (sb * np.float32(ts)).astype(np.float32).reshape(24, -1, 1)
        assert np.array_equal(qhat, (_blocks(q, g).astype(np.float32) * d).reshape(V.shape))


@pytest.mark.parametrize("fmt", ["MXINT4", "MXFP4"])
def test_mx_idempotent(oracle_lib, fmt):
    V = _rand(16, 512, 2)
    c1, s1, _, q1, _ = oracle_lib.fq(V, fmt)
    c2, s2, _, q2, _ = oracle_lib.fq(q1, fmt)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("fmt,g", CASES)
@pytest.mark.parametrize("k", [-5, 3])
def test_power_of_two_equivariance(oracle_lib, fmt, g, k):
    V = _rand(16, 256, 3)
    c1, s1, t1, q1, _ = oracle_lib.fq(V, fmt, g)
    c2, s2, t2, q2, _ = oracle_lib.fq(np.ldexp(V, k).astype(np.float32), fmt, g)
    assert np.array_equal(c1, c2)
    assert np.array_equal(np.ldexp(q1, k), q2)
    if fmt in ("MXINT4", "MXFP4"):
        assert np.array_equal(s1.astype(int) + k, s2.astype(int))
    if fmt == "NVFP4":
        assert np.array_equal(s1, s2) and t2 == np.ldexp(np.float32(t1), k)


@pytest.mark.parametrize("fmt,g", CASES)
def test_sign_symmetry_and_permutations(oracle_lib, fmt, g):
    V = _rand(12, 512, 4)
    _, s1, t1, q1, _ = oracle_lib.fq(V, fmt, g)
    _, s2, t2, q2, _ = oracle_lib.fq(-V, fmt, g)
    assert np.array_equal(-q1, q2) and np.array_equal(s1, s2) and t1 == t2
    rng = np.random.default_rng(5)
    rp = rng.permutation(V.shape[0])
    bp = rng.permutation(V.shape[1] // g)
    Vp = _blocks(V[rp], g)[:, bp].reshape(V.shape)
    _, s3, t3, q3, _ = oracle_lib.fq(np.ascontiguousarray(Vp), fmt, g)
    assert np.array_equal(q3, _blocks(q1[rp], g)[:, bp].reshape(V.shape))
    assert t3 == t1


@pytest.mark.parametrize("fmt,g", CASES)
def test_nearest_point_brute_force(oracle_lib, fmt, g):
    """Each element is the nearest point of its block's representable set (ties either)."""
    V = _rand(8, 128, 6)
    codes, scales, ts, qhat, _ = oracle_lib.fq(V, fmt, g)
    if fmt == "INT4":
        s = (scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        grid = np.arange(-7, 8, dtype=np.float64)[None, :] * s[:, None]
    elif fmt == "MXINT4":
        e = scales.astype(np.int64) - 127
        grid = np.ldexp(np.arange(-7, 8, dtype=np.float64)[None, :], (e - 2)[:, None])
    elif fmt == "MXFP4":
        e = scales.astype(np.int64) - 127
        full = np.concatenate([-E2M1[::-1], E2M1])
        grid = np.ldexp(full[None, :], e[:, None])
    else:
        sb = torch.from_numpy(scales).view(torch.float8_e4m3fn).float().numpy()
        d = (sb * np.float32(ts)).astype(np.float32).astype(np.float64)
        full = np.concatenate([-E2M1[::-1], E2M1])
        grid = full[None, :] * d[:, None]
    vb = V.reshape(-1, g).astype(np.float64)
    qb = qhat.reshape(-1, g).astype(np.float64)
    dist = np.abs(vb[:, :, None] - grid[:, None, :]).min(axis=2)
    err = np.abs(vb - qb)
    # nearest up to the fp32 rounding of the normalised value (relative 2^-22 slack)
    assert np.all(err <= dist + 4e-7 * np.abs(vb) + 1e-30)


def test_mx_scale_rule_and_top_binade(oracle_lib):
    V = _rand(16, 256, 7)
    amax = np.abs(V.reshape(16, -1, 32)).max(axis=2)
    m, e = np.frexp(amax.astype(np.float64))
    flog2 = (e - 1).reshape(-1)
    _, s_fp, _, q_fp, _ = oracle_lib.fq(V, "MXFP4")
    nz = amax.reshape(-1) > 0
    assert np.array_equal(s_fp.astype(int)[nz], flog2[nz] - 2 + 127)
    top = np.abs(q_fp.reshape(-1, 32)).max(axis=1)[nz] / np.ldexp(1.0, flog2[nz] - 2)
    assert set(np.unique(top)).issubset({4.0, 6.0})
    _, s_i, _, q_i, _ = oracle_lib.fq(V, "MXINT4")
    assert np.array_equal(s_i.astype(int)[nz], flog2[nz] + 127)
    topi = np.abs(q_i.reshape(-1, 32)).max(axis=1)[nz] / np.ldexp(1.0, flog2[nz] - 2)
    assert set(np.unique(topi)).issubset({4.0, 5.0, 6.0, 7.0})


@pytest.mark.parametrize("g", [128, 64])
def test_int4_scale_is_bf16_of_amax_over_7(oracle_lib, g):
    V = _rand(16, 512, 8)
    _, s, _, _, _ = oracle_lib.fq(V, "INT4", g)
    amax = np.abs(V.reshape(-1, g)).max(axis=1)
    want = torch.from_numpy((amax / np.float32(7)).astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(s, want.view(torch.int16).numpy().view(np.uint16))


def test_nvfp4_scales(oracle_lib):
    V = _rand(16, 512, 9)
    _, s, ts, q, _ = oracle_lib.fq(V, "NVFP4")
    A = np.float32(np.abs(V).max())
    assert ts == np.float32(A / np.float32(2688))
    k6 = np.float32(1) / (np.float32(6) * np.float32(ts))
    a = np.abs(V.reshape(-1, 16)).max(axis=1).astype(np.float32)
    want = torch.from_numpy((a * k6).astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(s, want.view(torch.uint8).numpy())
    # the block holding the global amax gets the top E4M3 scale, and its max maps to 6
    ib = np.argmax(a)
    assert s[ib] == 126
    assert np.abs(q.reshape(-1, 16)[ib]).max() == np.float32(np.float32(448) * ts) * np.float32(6)


def test_zero_blocks(oracle_lib):
    V = _rand(4, 256, 10)
    V[1] = 0
    V[2, :128] = 0
    for fmt in FORMATS:
        codes, scales, ts, q, _ = oracle_lib.fq(V, fmt)
        g = GROUPS[fmt]
        assert np.all(q[1] == 0) and np.all(codes.reshape(4, -1)[1] == 0)
        assert np.all(scales.reshape(4, -1)[1] == 0)
        assert np.all(scales.reshape(4, -1)[2, :128 // g] == 0)
    codes, scales, ts, q, _ = oracle_lib.fq(np.zeros((2, 64), np.float32), "NVFP4")
    assert ts == 0 and np.all(codes == 0) and np.all(scales == 0) and np.all(q == 0)


@pytest.mark.parametrize("fmt,g", CASES)
def test_quantize_weights_is_fq_of_normalised(oracle_lib, fmt, g):
    rng = np.random.default_rng(11)
    W = synth.f32_to_bf16_bits(_rand(16, 256, 12))
    r = oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, 16)).astype(np.float32))
    c = oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, 256)).astype(np.float32))
    codes, scales, ts, q = oracle_lib.quantize_weights(W, r, c, fmt, g)
    Wf = synth.bf16_bits_to_f32(W)
    ir = (np.float32(1) / r).astype(np.float32)
    ic = (np.float32(1) / c).astype(np.float32)
    V = ((Wf * ir[:, None]).astype(np.float32) * ic[None, :]).astype(np.float32)
    c2, s2, t2, q2, _ = oracle_lib.fq(V, fmt, g)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2) and ts == t2


def test_table12_byte_accounting(oracle_lib):
    gold = json.loads((Path(__file__).parent / "golden" / "table12_weight_memory.json").read_text())
    params = synth.LLAMA31_8B_LAYERS * sum(r * c for _, r, c in synth.LLAMA31_8B_PROJ)
    assert params == 6_979_321_856
    assert round(params * 2 / 1e9, 2) == gold["quantized_linear_weights_bf16_GB"]
    assert round(params * 0.5 / 1e9, 2) == gold["quantized_linear_weights_w4a4_GB"]
    assert round(params / gold["group"] * 2 / 1e9, 2) == gold["per_group_weight_scales_bf16_GB"]
    # the oracle's own output layout spends exactly 0.5 B per weight on codes
    V = _rand(8, 128, 13)
    codes, scales, _, _, _ = oracle_lib.fq(V, "INT4")
    assert codes.nbytes == V.size // 2 and scales.nbytes == V.size // 128 * 2
