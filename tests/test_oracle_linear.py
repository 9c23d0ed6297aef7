"""Pins for the oracle's quantised linear layer Y = deq(A) deq(B)^T diag(r) (the layer
that consumes the activation codes and the solved weight codes; listing page Tables 11-12).

Pinned by:
- hand-computed MXFP4, NVFP4 and INT4 (two groups of 64, nibble -8 included) examples,
  codes and scales written out bit by bit;
- one-hot weights, which turn the product into a gather of the activations and so expose
  any transposed operand or index slip;
- MXFP8 products recomputed with torch's float8 decoding and a float64 matmul, INT4
  products with the format's decode written out in numpy (nibble, bf16 bits);
- exact power-of-two scaling laws;
- the sampled-entry variant equal to the full product.
"""

import numpy as np
import pytest
import torch

FMTS = ["MXFP4", "MXFP6_E2M3", "MXFP6_E3M2", "MXFP8_E4M3", "MXFP8_E5M2"]
BITS = {"MXFP4": 4, "MXFP6_E2M3": 6, "MXFP6_E3M2": 6, "MXFP8_E4M3": 8, "MXFP8_E5M2": 8}


def _pack(elems: np.ndarray, bits: int) -> np.ndarray:
    """Row-major element codes -> the library's code layout (nibbles low-first, a 6-bit
    little-endian bit stream, or bytes)."""
    e = np.asarray(elems, dtype=np.uint8).reshape(-1)
    if bits == 8:
        return e.copy()
    if bits == 4:
        return (e[0::2] | (e[1::2] << 4)).astype(np.uint8)
    b = ((e[:, None] >> np.arange(6, dtype=np.uint8)) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(b, bitorder="little")


def _random_codes(rng, fmt, rows, cols):
    bits = BITS[fmt]
    e = rng.integers(0, 1 << bits, rows * cols).astype(np.uint8)
    if fmt == "MXFP8_E4M3":
        e[(e & 0x7F) == 0x7F] = 0x38
    if fmt == "MXFP8_E5M2":
        e[((e >> 2) & 31) == 31] = 0x3C
    return e


def test_hand_example_mxfp4(oracle_lib):
    # A row: 1.0, -2.0, 0.5, 6.0 (E2M1 codes 2, 8|4, 1, 7), block scale 2^1 (byte 128)
    # B row: 3.0, 1.5, -4.0, 0.5 (codes 5, 3, 8|6, 1), block scale 2^-1 (byte 126)
    # sum = 1*3 - 2*1.5 - 0.5*4 + 6*0.5 = 1;  times 2 * 0.5 = 1;  r = 0.25 -> 0.25
    a = np.zeros(32, np.uint8)
    a[:4] = [2, 12, 1, 7]
    b = np.zeros(32, np.uint8)
    b[:4] = [5, 3, 14, 1]
    y = oracle_lib.quantized_linear(_pack(a, 4), np.array([128], np.uint8), 1, _pack(b, 4),
                                    np.array([126], np.uint8), 1, 32, "MXFP4",
                                    r=np.array([0.25], np.float32))
    assert y.shape == (1, 1) and y[0, 0] == 0.25


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_weights_gather_activations(oracle_lib, fmt):
    rng = np.random.default_rng(1)
    M, N, K = 7, 5, 96
    ae = _random_codes(rng, fmt, M, K)
    asc = rng.integers(120, 135, M * K // 32).astype(np.uint8)
    one = oracle_lib.mini_encode(fmt, np.array([1.0], np.float32))[0] if fmt != "MXFP4" else 2
    perm = rng.permutation(K)[:N]
    be = np.zeros((N, K), np.uint8)
    be[np.arange(N), perm] = one
    bsc = np.full(N * K // 32, 127, np.uint8)
    r = np.exp2(rng.integers(-3, 4, N)).astype(np.float32)
    y = oracle_lib.quantized_linear(_pack(ae, BITS[fmt]), asc, M, _pack(be, BITS[fmt]), bsc, N, K,
                                    fmt, r=r)
    deqA = oracle_lib.dequantize(_pack(ae, BITS[fmt]), asc, 0.0, fmt, M, K).astype(np.float64)
    assert np.array_equal(y, deqA[:, perm] * r[None, :])


@pytest.mark.parametrize("fmt,dt", [("MXFP8_E4M3", torch.float8_e4m3fn), ("MXFP8_E5M2", torch.float8_e5m2)])
def test_fp8_against_torch(oracle_lib, fmt, dt):
    rng = np.random.default_rng(2)
    M, N, K = 9, 11, 160
    ae, be = _random_codes(rng, fmt, M, K), _random_codes(rng, fmt, N, K)
    asc = rng.integers(118, 137, M * K // 32).astype(np.uint8)
    bsc = rng.integers(118, 137, N * K // 32).astype(np.uint8)
    y = oracle_lib.quantized_linear(ae, asc, M, be, bsc, N, K, fmt)

    def deq(e, s, rows):
        v = torch.from_numpy(e.reshape(rows, K)).view(dt).double()
        return v * torch.from_numpy(np.ldexp(1.0, s.astype(np.int64) - 127)).repeat_interleave(32).reshape(rows, K)

    want = (deq(ae, asc, M) @ deq(be, bsc, N).T).numpy()
    assert np.allclose(y, want, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("fmt", FMTS)
def test_scaling_laws_and_entries(oracle_lib, fmt):
    rng = np.random.default_rng(3)
    M, N, K = 6, 8, 128
    ae, be = _random_codes(rng, fmt, M, K), _random_codes(rng, fmt, N, K)
    asc = rng.integers(122, 132, M * K // 32).astype(np.uint8)
    bsc = rng.integers(122, 132, N * K // 32).astype(np.uint8)
    pa, pb = _pack(ae, BITS[fmt]), _pack(be, BITS[fmt])
    y = oracle_lib.quantized_linear(pa, asc, M, pb, bsc, N, K, fmt)
    y2 = oracle_lib.quantized_linear(pa, asc + 1, M, pb, bsc, N, K, fmt)
    assert np.array_equal(y2, 2 * y)
    r = np.exp2(rng.integers(-2, 3, N)).astype(np.float32)
    yr = oracle_lib.quantized_linear(pa, asc, M, pb, bsc, N, K, fmt, r=r)
    assert np.array_equal(yr, y * r[None, :])
    mi, ni = rng.integers(0, M, 20), rng.integers(0, N, 20)
    ye, ay = oracle_lib.quantized_linear_entries(pa, asc, M, pb, bsc, N, K, fmt, mi, ni, r=r)
    assert np.array_equal(ye, yr[mi, ni]) and np.all(ay >= np.abs(ye))


def test_hand_example_nvfp4(oracle_lib):
    # A block: 1.0, -2.0, 0.5, 6.0 (codes 2, 12, 1, 7), E4M3 block scale 1.5 (0x3C), s_t 3.0
    # B block: 3.0, 1.5, -4.0, 0.5 (codes 5, 3, 14, 1), E4M3 block scale 0.25 (0x28), s_t 0.125
    # sum = 1;  times 1.5 * 0.25 * 3 * 0.125 = 0.140625;  r = 2 -> 0.28125
    a = np.zeros(32, np.uint8)
    a[:4] = [2, 12, 1, 7]
    b = np.zeros(32, np.uint8)
    b[:4] = [5, 3, 14, 1]
    # second block: A 0.5 (code 1) at scale 0.001953125 (subnormal 0x01 = 2^-9), B -6 at
    # scale 448 (0x7E): adds 0.5 * 2^-9 * -6 * 448 * 0.375 = -0.984375 before r
    a[16], b[16] = 1, 15
    y = oracle_lib.quantized_linear(_pack(a, 4), np.array([0x3C, 0x01], np.uint8), 1, _pack(b, 4),
                                    np.array([0x28, 0x7E], np.uint8), 1, 32, "NVFP4",
                                    r=np.array([2.0], np.float32), a_ts=3.0, b_ts=0.125)
    assert y.shape == (1, 1) and y[0, 0] == 2.0 * (0.140625 - 0.984375)


def test_nvfp4_one_hot_and_tensor_scales(oracle_lib):
    rng = np.random.default_rng(4)
    M, N, K = 7, 5, 96
    ae = rng.integers(0, 16, M * K).astype(np.uint8)
    asc = rng.integers(0, 0x7F, M * K // 16).astype(np.uint8)
    perm = rng.permutation(K)[:N]
    be = np.zeros((N, K), np.uint8)
    be[np.arange(N), perm] = 2                       # e2m1 1.0
    bsc = np.full(N * K // 16, 0x38, np.uint8)       # e4m3 1.0
    r = np.exp2(rng.integers(-3, 4, N)).astype(np.float32)
    pa, pb = _pack(ae, 4), _pack(be.reshape(-1), 4)
    y = oracle_lib.quantized_linear(pa, asc, M, pb, bsc, N, K, "NVFP4", r=r, a_ts=0.25, b_ts=1.0)
    deqA = oracle_lib.dequantize(pa, asc, 0.25, "NVFP4", M, K).astype(np.float64)
    assert np.array_equal(y, deqA[:, perm] * r[None, :])
    # the two tensor scales multiply the result (exactly, for powers of two)
    y2 = oracle_lib.quantized_linear(pa, asc, M, pb, bsc, N, K, "NVFP4", r=r, a_ts=0.5, b_ts=4.0)
    assert np.array_equal(y2, 8 * y)
    ye, ay = oracle_lib.quantized_linear_entries(pa, asc, M, pb, bsc, N, K, "NVFP4", [0, M - 1],
                                                 [N - 1, 0], r=r, a_ts=0.25, b_ts=1.0)
    assert np.array_equal(ye, y[[0, M - 1], [N - 1, 0]]) and np.all(ay >= np.abs(ye))


# ---------------------------------------------------------------- INT4, bf16 group scales
# INT4 (the listing page's W4A4 rows; Table 12's packed 4-bit weights with one bf16 scale
# per group of 64 or 128 along K): element = two's-complement nibble q in [-8, 7] times the
# group's bf16 scale.
def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _int4_deq_numpy(nib, sc_bits, rows, K, g):
    """The format's definition written out independently of the oracle: nibble -> signed
    integer, bf16 bits -> float32 -> float64, one scale per g consecutive elements."""
    q = ((nib.astype(np.int64) ^ 8) - 8).reshape(rows, K)
    s = (sc_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(rows, K // g)
    return q * np.repeat(s, g, axis=1)


def test_hand_example_int4_g64(oracle_lib):
    # K = 128, two groups of 64.
    # group 0: A 3, -2, 6 at K 0, 1, 5 (scale 0.375);  B 5, 4, -1 (scale 1.25)
    #          sum 15 - 8 - 6 = 1, times 0.375 * 1.25 = 0.46875
    # group 1: A -8, 1 at K 64, 100 (scale 0.125);  B 3, -7 (scale 6.0)
    #          sum -24 - 7 = -31, times 0.125 * 6 = -23.25
    # total -22.78125, times r = 0.5 -> -11.390625
    a = np.zeros(128, np.int64)
    a[[0, 1, 5, 64, 100]] = [3, -2, 6, -8, 1]
    b = np.zeros(128, np.int64)
    b[[0, 1, 5, 64, 100]] = [5, 4, -1, 3, -7]
    asc = np.array([0x3EC0, 0x3E00], np.uint16)   # 0.375, 0.125
    bsc = np.array([0x3FA0, 0x40C0], np.uint16)   # 1.25, 6.0
    y = oracle_lib.quantized_linear(_pack(a & 15, 4), asc, 1, _pack(b & 15, 4), bsc, 1, 128,
                                    "INT4", group=64, r=np.array([0.5], np.float32))
    assert y.shape == (1, 1) and y[0, 0] == -11.390625


@pytest.mark.parametrize("g", [64, 128])
def test_int4_one_hot_weights_gather_activations(oracle_lib, g):
    rng = np.random.default_rng(11)
    M, N, K = 6, 9, 4 * g
    an = rng.integers(0, 16, M * K).astype(np.uint8)             # every nibble, -8 included
    asc = _bf16_bits(rng.uniform(0.01, 4.0, M * K // g))
    perm = rng.permutation(K)[:N]
    bn = np.zeros((N, K), np.uint8)
    bn[np.arange(N), perm] = 1
    bsc = np.full(N * K // g, 0x3F80, np.uint16)                  # 1.0
    r = np.exp2(rng.integers(-3, 4, N)).astype(np.float32)
    pa, pb = _pack(an, 4), _pack(bn.reshape(-1), 4)
    y = oracle_lib.quantized_linear(pa, asc, M, pb, bsc, N, K, "INT4", group=g, r=r)
    deqA = _int4_deq_numpy(an, asc, M, K, g)
    assert np.array_equal(y, deqA[:, perm] * r[None, :])
    # the sampled entries equal the full product, and bound it
    mi, ni = rng.integers(0, M, 15), rng.integers(0, N, 15)
    ye, ay = oracle_lib.quantized_linear_entries(pa, asc, M, pb, bsc, N, K, "INT4", mi, ni,
                                                 group=g, r=r)
    assert np.array_equal(ye, y[mi, ni]) and np.all(ay >= np.abs(ye))


@pytest.mark.parametrize("g", [64, 128])
def test_int4_against_independent_decode(oracle_lib, g):
    rng = np.random.default_rng(12)
    M, N, K = 5, 7, 3 * g
    an, bn = rng.integers(0, 16, M * K).astype(np.uint8), rng.integers(0, 16, N * K).astype(np.uint8)
    asc = _bf16_bits(np.exp2(rng.uniform(-6, 6, M * K // g)))
    bsc = _bf16_bits(np.exp2(rng.uniform(-6, 6, N * K // g)))
    y = oracle_lib.quantized_linear(_pack(an, 4), asc, M, _pack(bn, 4), bsc, N, K, "INT4", group=g)
    want = _int4_deq_numpy(an, asc, M, K, g) @ _int4_deq_numpy(bn, bsc, N, K, g).T
    assert np.allclose(y, want, rtol=1e-13, atol=0.0)
    # a group's scale doubled (bf16 exponent + 1) doubles exactly that group's share
    asc2 = asc.reshape(M, K // g).copy()
    asc2[:, 1] += 0x80
    y2 = oracle_lib.quantized_linear(_pack(an, 4), asc2.reshape(-1), M, _pack(bn, 4), bsc, N, K,
                                     "INT4", group=g)
    qa = _int4_deq_numpy(an, asc, M, K, g)
    qb = _int4_deq_numpy(bn, bsc, N, K, g)
    share = qa[:, g:2 * g] @ qb[:, g:2 * g].T
    assert np.allclose(y2, want + share, rtol=1e-13, atol=1e-300)
