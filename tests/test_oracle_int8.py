"""Pins for the oracle's 8-bit formats: INT8 (grouped, symmetric, bf16 group scale) and
MXINT8 (OCP MX v1.0: 8-bit two's-complement elements with an implicit 2^-6 under an E8M0
shared exponent).  The conference entry lists INT8 and the full MX family among the
formats the solver supports.

Pinned by what the definitions fix independently of the oracle's code: the dequantised
value is code x scale on the stated grid, the scale rules reduced to torch's bf16 cast and
frexp, the nearest-point property (brute force over the 255-point grid), MX idempotence,
power-of-two equivariance, sign symmetry, and the solve's invariants (monotone MSE, scale
steps that minimise their objective over the whole admissible set).
"""

import numpy as np
import pytest
import torch

import synth

FORMATS8 = ["INT8", "MXINT8"]
GROUPS8 = {"INT8": 128, "MXINT8": 32}


def _rand(rows, cols, seed):
    rng = np.random.default_rng(seed)
    V = rng.standard_t(4, (rows, cols)) * 0.02
    V[:, rng.choice(cols, max(1, cols // 50), replace=False)] *= 20
    V[rng.random((rows, cols)) < 0.01] = 0.0
    return V.astype(np.float32)


def _scale_values(fmt, scales, g, shape):
    if fmt == "INT8":
        s = (scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        s = np.ldexp(1.0, scales.astype(np.int64) - 127 - 6)
    return s.reshape(shape[0], -1, 1)


@pytest.mark.parametrize("fmt", FORMATS8)
def test_codes_grid_and_roundtrip(oracle_lib, fmt):
    g = GROUPS8[fmt]
    V = _rand(24, 512, 1)
    codes, scales, ts, qhat, flags = oracle_lib.fq(V, fmt)
    assert codes.size == V.size and scales.size == V.size // g
    q = codes.view(np.int8).astype(np.float64).reshape(V.shape)
    assert np.all(np.abs(q) <= 127)
    want = (q.reshape(V.shape[0], -1, g) * _scale_values(fmt, scales, g, V.shape)).reshape(V.shape)
    assert np.array_equal(qhat.astype(np.float64), want)
    deq = oracle_lib.dequantize(codes, scales, ts, fmt, *V.shape)
    assert np.array_equal(deq.view(np.uint32), qhat.view(np.uint32))


@pytest.mark.parametrize("fmt", FORMATS8)
def test_nearest_point_brute_force(oracle_lib, fmt):
    g = GROUPS8[fmt]
    V = _rand(8, 256, 2)
    codes, scales, ts, qhat, _ = oracle_lib.fq(V, fmt)
    s = _scale_values(fmt, scales, g, V.shape).reshape(-1)
    grid = np.arange(-127, 128, dtype=np.float64)[None, :] * s[:, None]
    vb = V.reshape(-1, g).astype(np.float64)
    dist = np.abs(vb[:, :, None] - grid[:, None, :]).min(axis=2)
    err = np.abs(vb - qhat.reshape(-1, g).astype(np.float64))
    assert np.all(err <= dist + 4e-7 * np.abs(vb) + 1e-30)


def test_scale_rules(oracle_lib):
    V = _rand(16, 512, 3)
    _, s, _, _, _ = oracle_lib.fq(V, "INT8")
    amax = np.abs(V.reshape(-1, 128)).max(axis=1)
    want = torch.from_numpy((amax / np.float32(127)).astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(s, want.view(torch.int16).numpy().view(np.uint16))
    _, sm, _, qm, _ = oracle_lib.fq(V, "MXINT8")
    am = np.abs(V.reshape(-1, 32)).max(axis=1).astype(np.float64)
    nz = am > 0
    _, e = np.frexp(am)
    assert np.array_equal(sm.astype(int)[nz], (e - 1)[nz] + 127)
    # the block maximum lands in the top binade of the element grid: |q| in [64, 127]
    top = np.abs(qm.reshape(-1, 32)).max(axis=1)[nz] / np.ldexp(1.0, (e - 1)[nz] - 6)
    assert np.all((top >= 64) & (top <= 127))


def test_mxint8_idempotent_and_equivariant(oracle_lib):
    V = _rand(16, 256, 4)
    c1, s1, _, q1, _ = oracle_lib.fq(V, "MXINT8")
    c2, s2, _, q2, _ = oracle_lib.fq(q1, "MXINT8")
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    for k in (-5, 3):
        c3, s3, _, q3, _ = oracle_lib.fq(np.ldexp(V, k).astype(np.float32), "MXINT8")
        assert np.array_equal(c1, c3) and np.array_equal(np.ldexp(q1, k), q3)
        assert np.array_equal(s1.astype(int) + k, s3.astype(int))


@pytest.mark.parametrize("fmt", FORMATS8)
def test_sign_symmetry_and_zero_blocks(oracle_lib, fmt):
    V = _rand(12, 256, 5)
    V[3, :GROUPS8[fmt]] = 0.0
    c1, s1, _, q1, _ = oracle_lib.fq(V, fmt)
    _, s2, _, q2, _ = oracle_lib.fq(-V, fmt)
    assert np.array_equal(-q1, q2) and np.array_equal(s1, s2)
    assert np.all(q1[3, :GROUPS8[fmt]] == 0) and s1.reshape(12, -1)[3, 0] == 0
    assert np.all(c1.reshape(12, -1)[3, :GROUPS8[fmt]] == 0)


@pytest.mark.parametrize("fmt", FORMATS8)
def test_scale_steps_minimise_over_admissible_set(oracle_lib, fmt):
    """The r-step result is the admissible value minimising the row objective (brute
    force over the 129 bf16 values around the closed form: bf16 is the dual scales'
    admissible set for INT8 and for the MX formats)."""
    rng = np.random.default_rng(6)
    W = (rng.standard_t(4, (6, 256)) * 0.02).astype(np.float32)
    res = oracle_lib.solve(W, fmt, 1)
    Q0 = oracle_lib.quantize_weights(W, None, None, fmt)[3].astype(np.float64)
    for i in range(W.shape[0]):
        f = lambda s: np.sum((W[i].astype(np.float64) - s * Q0[i]) ** 2)   # c = 1 at the r-step
        x = res["r_trace"][0][i]
        base = torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()
        cand = torch.tensor(np.arange(base - 64, base + 65), dtype=torch.int16).view(torch.bfloat16).double().numpy()
        cand = cand[cand > 0]
        best = min(f(s) for s in cand)
        assert f(float(res["r"][i])) <= best * (1 + 1e-12)


@pytest.mark.parametrize("fmt", FORMATS8)
def test_solve_monotone(oracle_lib, fmt):
    W = synth.matrix(synth.WORKLOADS["down4096x14336_nvfp4"]["W"].scaled(128, 1024), 0)
    res = oracle_lib.solve(W, fmt, 12)
    assert np.all(np.diff(res["nmse"]) <= 0.0) and res["nmse"][-1] <= res["nmse"][0]
    assert res["codes"].size == 128 * 1024
