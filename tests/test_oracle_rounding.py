"""Pins for the oracle's scalar rounding and scale projections.

Each oracle routine is a brute-force nearest-grid search.  Here it is checked against an
independent construction: a library rounding routine (numpy's half-to-even ``rint``,
torch's bf16 / float8_e4m3fn casts, ``frexp``) applied to the element grid's closed
form, over every fp32 bit pattern in the ranges where the decision thresholds lie.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _all_f32_in_binades(lo_exp: int, hi_exp: int) -> np.ndarray:
    """Every positive fp32 in [2^lo_exp, 2^hi_exp)."""
    lo = np.uint32((lo_exp + 127) << 23)
    hi = np.uint32((hi_exp + 127) << 23)
    return np.arange(lo, hi, dtype=np.uint32).view(np.float32)


def _e2m1_closed_form(x: np.ndarray) -> np.ndarray:
    """Nearest E2M1 value, ties to even mantissa, saturating at 6.

    On [0, 2) the grid is uniform with step 1/2, on [2, 4) step 1, on [4, 6] step 2; in
    each piece "ties to the even mantissa bit" is "ties to the even multiple of the step",
    which is exactly numpy's half-to-even rint of x/step.
    """
    ax = np.abs(x.astype(np.float64))
    y = np.where(ax < 2, np.rint(ax * 2) / 2, np.where(ax < 4, np.rint(ax), np.rint(ax / 2) * 2))
    return np.minimum(y, 6.0)


def _e2m1_value_of_code(code: np.ndarray) -> np.ndarray:
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    v = grid[code & 7]
    return np.where(code & 8, -v, v)


def test_e2m1_exhaustive_threshold_range(oracle_lib):
    # every fp32 with |x| in [2^-3, 2^3): covers all seven decision thresholds and saturation
    pos = _all_f32_in_binades(-3, 3)
    for sign in (1.0, -1.0):
        x = (pos * np.float32(sign)).astype(np.float32)
        for s in range(0, x.size, 1 << 24):
            xs = x[s:s + (1 << 24)]
            code = oracle_lib.e2m1_encode(xs)
            got = _e2m1_value_of_code(code)
            want = _e2m1_closed_form(xs) * sign
            assert np.array_equal(np.abs(got), np.abs(want))
            assert np.all((code >> 3) == (1 if sign < 0 else 0))


def test_e2m1_specials(oracle_lib):
    x = np.array([0.0, -0.0, 1e-30, -1e-30, 0.25, -0.25, 0.2500001, 5.0, 5.0000005, 6.0, 7.0,
                  100.0, -1e30, 3.4e38], dtype=np.float32)
    code = oracle_lib.e2m1_encode(x)
    assert list(code) == [0, 8, 0, 8, 0, 8, 1, 6, 7, 7, 7, 7, 15, 7]
    dec = oracle_lib.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert list(dec[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(-dec[8:]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert np.signbit(dec[8])


def _e4m3_values() -> np.ndarray:
    """The 127 non-negative finite E4M3FN values, decoded by torch."""
    return torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_decode_matches_torch(oracle_lib):
    codes = np.arange(127, dtype=np.uint8)
    assert np.array_equal(oracle_lib.e4m3_decode(codes), _e4m3_values())
    assert oracle_lib.e4m3_decode(np.array([126], np.uint8))[0] == 448.0
    assert oracle_lib.e4m3_decode(np.array([1], np.uint8))[0] == 2.0 ** -9


def test_e4m3_encode_against_torch_near_every_threshold(oracle_lib):
    vals = _e4m3_values().astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    anchors = np.concatenate([vals, mids, np.float32([464.0])])
    bits = anchors.view(np.uint32).astype(np.int64)
    offs = np.arange(-300, 301, dtype=np.int64)
    x = (bits[:, None] + offs[None, :]).reshape(-1)
    x = x[(x >= 0) & (x < 0x7F800000)].astype(np.uint32).view(np.float32)
    x = x[(x >= 0) & (x <= 464.0)]
    rng = np.random.default_rng(1)
    x = np.concatenate([x, rng.uniform(0, 464, 200_000).astype(np.float32),
                        np.exp2(rng.uniform(-16, 8.8, 200_000)).astype(np.float32)])
    x = x[x <= 464.0]
    code = oracle_lib.e4m3_encode(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(code, want)


def test_e4m3_saturates(oracle_lib):
    x = np.float32([448.0, 464.0, 464.1, 1000.0, 3e38])
    assert list(oracle_lib.e4m3_encode(x)) == [126] * 5


def test_bf16_round_against_torch(oracle_lib):
    rng = np.random.default_rng(2)
    hi = rng.integers(0, 0x7F7F, 400_000, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    bits = np.concatenate([bits, bits | 0x80000000])
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    got = oracle_lib.bf16_round(x)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    ok = np.isfinite(want)
    assert np.array_equal(got[ok].view(np.uint32), want[ok].view(np.uint32))


def test_int_round_against_rint(oracle_lib):
    x = np.concatenate([np.arange(-9, 9, 0.25, dtype=np.float32),
                        np.random.default_rng(3).normal(0, 4, 300_000).astype(np.float32),
                        np.nextafter(np.float32(np.arange(-8, 9) + 0.5), np.float32(np.inf)),
                        np.nextafter(np.float32(np.arange(-8, 9) + 0.5), np.float32(-np.inf))])
    got = oracle_lib.int_round(x, 7)
    want = np.clip(np.rint(x.astype(np.float64)), -7, 7)
    assert np.array_equal(got.astype(np.float64), want)


def test_project_mx_is_bf16(oracle_lib):
    """The MX formats' dual scales project onto bf16, like INT4's (their E8M0 power of two
    is the block scale's set, inside the quantiser)."""
    rng = np.random.default_rng(4)
    x = np.exp2(rng.uniform(-130, 127, 200_000)).astype(np.float32)
    x = np.concatenate([x, np.float32([1.0, 1.5, 1.4999999, 3.0, 0.75, 2.0 ** -127, 1e-45, 3e38]),
                        (1.5 * np.exp2(np.arange(-120, 120))).astype(np.float32)])
    x = x[(x > 0) & np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    want = np.clip(want, 2.0 ** -126, np.float32(torch.finfo(torch.bfloat16).max))
    for fmt in ("MXFP4", "MXINT4", "MXINT8", "MXFP8_E4M3", "MXFP8_E5M2", "MXFP6_E2M3", "MXFP6_E3M2"):
        assert np.array_equal(oracle_lib.project(fmt, x), want), fmt


def test_project_e4m3(oracle_lib):
    rng = np.random.default_rng(5)
    x = np.concatenate([np.exp2(rng.uniform(-14, 10, 300_000)), [448.0, 500.0, 1e-8, 2.0 ** -10,
                                                                 2.0 ** -9]]).astype(np.float32)
    got = oracle_lib.project("NVFP4", x)
    want = torch.from_numpy(np.minimum(x, 448.0)).to(torch.float8_e4m3fn).float().numpy()
    want = np.maximum(want, 2.0 ** -9)
    assert np.array_equal(got, want)


def test_project_bf16(oracle_lib):
    rng = np.random.default_rng(6)
    x = np.concatenate([np.exp2(rng.uniform(-130, 127, 300_000)), [1.0, 2.0 ** -127, 1e-40]])
    x = x.astype(np.float32)
    x = x[x > 0]
    got = oracle_lib.project("INT4", x)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    want = np.clip(want, 2.0 ** -126, np.float32(torch.finfo(torch.bfloat16).max))
    assert np.array_equal(got, want)
