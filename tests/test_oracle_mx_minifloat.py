"""Pins for the oracle's MX FP8 and FP6 element types (OCP MX v1.0: FP8 E4M3 and E5M2,
FP6 E2M3 and E3M2, each under an E8M0 shared exponent over blocks of 32).  The conference
entry names the MX family among the formats the solver supports.

Pinned by what the definitions fix independently of the oracle's code:
- the FP8 grids and their round-to-nearest-even equal torch's float8_e4m3fn / float8_e5m2
  casts;
- the FP6 grids share their mantissa width with the FP8 types, so their normal range
  rounds like torch's FP8 casts and their subnormal range is a fixed-point grid (numpy's
  half-to-even round);
- largest and smallest values, ties, saturation, negative zero;
- the shared exponent from frexp, the packing of 6-bit codes into a bit stream, the
  nearest-point property by brute force, and the solve's invariants.
"""

import numpy as np
import pytest
import torch

import synth

FP8 = {"MXFP8_E4M3": torch.float8_e4m3fn, "MXFP8_E5M2": torch.float8_e5m2}
FP6 = ["MXFP6_E2M3", "MXFP6_E3M2"]
MINI = list(FP8) + FP6
EMAX = {"MXFP8_E4M3": 8, "MXFP8_E5M2": 15, "MXFP6_E2M3": 2, "MXFP6_E3M2": 4}
LARGEST = {"MXFP8_E4M3": 448.0, "MXFP8_E5M2": 57344.0, "MXFP6_E2M3": 7.5, "MXFP6_E3M2": 28.0}
SMALLEST = {"MXFP8_E4M3": 2.0 ** -9, "MXFP8_E5M2": 2.0 ** -16, "MXFP6_E2M3": 0.125, "MXFP6_E3M2": 0.0625}
BITS = {"MXFP8_E4M3": 8, "MXFP8_E5M2": 8, "MXFP6_E2M3": 6, "MXFP6_E3M2": 6}
# FP6 type -> the FP8 type with the same mantissa width, and where FP6 normals start
FP6_TWIN = {"MXFP6_E2M3": (torch.float8_e4m3fn, 1.0, 8), "MXFP6_E3M2": (torch.float8_e5m2, 0.25, 16)}


def _grid(oracle_lib, fmt):
    codes = np.arange(1 << BITS[fmt], dtype=np.uint8)
    return codes, oracle_lib.mini_decode(fmt, codes)


@pytest.mark.parametrize("fmt", list(FP8))
def test_fp8_grid_is_torch_float8(oracle_lib, fmt):
    codes, v = _grid(oracle_lib, fmt)
    t = torch.from_numpy(codes).view(FP8[fmt]).float().numpy()
    fin = np.isfinite(t)
    assert np.array_equal(v[fin], t[fin])
    assert np.all(np.isnan(v[~fin]))


@pytest.mark.parametrize("fmt", MINI)
def test_grid_extremes_and_order(oracle_lib, fmt):
    codes, v = _grid(oracle_lib, fmt)
    half = 1 << (BITS[fmt] - 1)
    pos = v[:half]
    fin = np.isfinite(pos)
    assert np.nanmax(pos) == LARGEST[fmt] and pos[1] == SMALLEST[fmt] and pos[0] == 0.0
    assert np.all(np.diff(pos[fin]) > 0)                           # increasing with the code
    assert np.array_equal(v[half:][fin], -pos[fin])                # sign bit on top
    assert np.signbit(v[half]) and v[half] == 0.0


@pytest.mark.parametrize("fmt", FP6)
def test_fp6_grid_inside_fp8_twin(oracle_lib, fmt):
    """Every FP6 value is exactly an FP8 value of the type with the same mantissa width,
    and each binade above the subnormals holds 2^mbits values."""
    _, v = _grid(oracle_lib, fmt)
    twin, lo, sub = FP6_TWIN[fmt]
    t = torch.from_numpy(v).to(twin).float().numpy()
    assert np.array_equal(t, v)
    pos = v[: len(v) // 2]
    per = np.sum((pos >= 1.0) & (pos < 2.0))
    assert per == (8 if fmt == "MXFP6_E2M3" else 4)
    assert np.array_equal(pos[pos < lo], np.arange(np.sum(pos < lo)) / sub)


@pytest.mark.parametrize("fmt", list(FP8))
def test_fp8_rounding_is_torch_cast(oracle_lib, fmt):
    rng = np.random.default_rng(1)
    mx = LARGEST[fmt]
    x = np.concatenate([
        rng.uniform(-mx, mx, 20000),
        np.exp2(rng.uniform(np.log2(SMALLEST[fmt]) - 3, np.log2(mx), 20000)) * rng.choice([-1, 1], 20000),
    ]).astype(np.float32)
    # every midpoint between neighbouring values, and its two fp32 neighbours
    _, v = _grid(oracle_lib, fmt)
    pos = np.sort(v[np.isfinite(v) & (v >= 0)])
    mid = ((pos[1:].astype(np.float64) + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)]).astype(np.float32)
    got = oracle_lib.mini_decode(fmt, oracle_lib.mini_encode(fmt, x))
    want = torch.from_numpy(x).to(FP8[fmt]).float().numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


@pytest.mark.parametrize("fmt", FP6)
def test_fp6_rounding(oracle_lib, fmt):
    twin, lo, sub = FP6_TWIN[fmt]
    mx = LARGEST[fmt]
    rng = np.random.default_rng(2)
    _, v = _grid(oracle_lib, fmt)
    pos = np.sort(v[v >= 0])
    mid = ((pos[1:].astype(np.float64) + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([rng.uniform(0, mx, 50000), mid, np.nextafter(mid, 0),
                        np.nextafter(mid, np.inf)]).astype(np.float32)
    got = oracle_lib.mini_decode(fmt, oracle_lib.mini_encode(fmt, x)).astype(np.float64)
    normal = x >= lo
    # normal range: the FP8 type with the same mantissa width rounds identically
    want_n = torch.from_numpy(x[normal]).to(twin).double().numpy()
    assert np.array_equal(got[normal], np.minimum(want_n, mx))
    # subnormal range: a fixed-point grid of step 1/sub, half to even
    assert np.array_equal(got[~normal], np.round(x[~normal].astype(np.float64) * sub) / sub)
    # sign symmetry
    gneg = oracle_lib.mini_decode(fmt, oracle_lib.mini_encode(fmt, -x))
    assert np.array_equal(gneg, -got.astype(np.float32))


@pytest.mark.parametrize("fmt", MINI)
def test_saturation_and_negative_zero(oracle_lib, fmt):
    mx = LARGEST[fmt]
    x = np.array([mx * 1.01, mx * 4, 3.0e38, -mx * 2, -1e-30, 1e-30], dtype=np.float32)
    got = oracle_lib.mini_decode(fmt, oracle_lib.mini_encode(fmt, x))
    assert np.array_equal(got[:4], np.array([mx, mx, mx, -mx], dtype=np.float32))
    assert got[4] == 0.0 and np.signbit(got[4]) and got[5] == 0.0 and not np.signbit(got[5])


def _rand(rows, cols, seed):
    rng = np.random.default_rng(seed)
    V = rng.standard_t(4, (rows, cols)) * 0.02
    V[:, rng.choice(cols, max(1, cols // 50), replace=False)] *= 20
    V[rng.random((rows, cols)) < 0.01] = 0.0
    V[0, :32] = 0.0
    return V.astype(np.float32)


def _element_codes(fmt, codes, n):
    if BITS[fmt] == 8:
        return codes[:n].astype(np.uint8)
    bits = np.unpackbits(codes, bitorder="little")[: 6 * n].reshape(n, 6)
    return (bits.astype(np.uint8) << np.arange(6, dtype=np.uint8)).sum(axis=1).astype(np.uint8)


@pytest.mark.parametrize("fmt", MINI)
def test_block_quantiser(oracle_lib, fmt):
    V = _rand(16, 512, 3)
    codes, scales, ts, qhat, _ = oracle_lib.fq(V, fmt)
    assert codes.size == V.size * BITS[fmt] // 8 and scales.size == V.size // 32
    # shared exponent: floor(log2 amax) - emax, byte e + 127; zero blocks store 0
    am = np.abs(V.reshape(-1, 32)).max(axis=1).astype(np.float64)
    nz = am > 0
    _, fe = np.frexp(am)
    e = np.where(nz, fe - 1 - EMAX[fmt], -127)
    assert np.array_equal(scales.astype(int), e + 127)
    # codes in the stated layout decode to Qhat
    ec = _element_codes(fmt, codes, V.size)
    val = oracle_lib.mini_decode(fmt, ec).astype(np.float64).reshape(-1, 32)
    assert np.array_equal(val * np.ldexp(1.0, e)[:, None], qhat.reshape(-1, 32).astype(np.float64))
    assert np.all(ec.reshape(-1, 32)[~nz] == 0)
    # nearest point of the scaled grid (brute force)
    _, grid = _grid(oracle_lib, fmt)
    grid = grid[np.isfinite(grid)].astype(np.float64)
    vb = V.reshape(-1, 32).astype(np.float64)
    sg = grid[None, None, :] * np.ldexp(1.0, e)[:, None, None]
    dist = np.abs(vb[:, :, None] - sg).min(axis=2)
    err = np.abs(vb - qhat.reshape(-1, 32))
    assert np.all(err <= dist * (1 + 1e-12) + 1e-300)
    deq = oracle_lib.dequantize(codes, scales, ts, fmt, *V.shape)
    assert np.array_equal(deq.view(np.uint32), qhat.view(np.uint32))


@pytest.mark.parametrize("fmt", MINI)
def test_idempotent_and_pow2_equivariant(oracle_lib, fmt):
    V = _rand(8, 256, 4)
    c1, s1, _, q1, _ = oracle_lib.fq(V, fmt)
    c2, s2, _, q2, _ = oracle_lib.fq(q1, fmt)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    c3, s3, _, q3, _ = oracle_lib.fq(np.ldexp(V, 3).astype(np.float32), fmt)
    nz = s1 > 0
    assert np.array_equal(np.ldexp(q1, 3), q3) and np.array_equal(s1[nz].astype(int) + 3, s3[nz].astype(int))


@pytest.mark.parametrize("fmt", MINI)
def test_solve_invariants(oracle_lib, fmt):
    W = synth.matrix(synth.WORKLOADS["down4096x14336_nvfp4"]["W"].scaled(64, 512), 0)
    res = oracle_lib.solve(W, fmt, 8)
    assert np.all(np.diff(res["nmse"]) <= 0.0) and res["nmse"][-1] <= res["nmse"][0]
    for s in (res["r"], res["c"]):
        # bf16 values (the dual scales' admissible set; E8M0 is the block scale's)
        assert np.all(s.view(np.uint32) & 0xFFFF == 0) and np.all(s >= 2.0 ** -126)
    Wf = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Q = oracle_lib.dequantize(res["codes"], res["scales"], 0.0, fmt, *W.shape).astype(np.float64)
    R = res["r"].astype(np.float64)[:, None] * Q * res["c"].astype(np.float64)[None, :]
    nmse = np.sum((Wf - R) ** 2) / np.sum(Wf ** 2)
    assert abs(nmse - res["nmse"][-1]) <= 1e-9 * nmse
