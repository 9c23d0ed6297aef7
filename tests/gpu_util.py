"""Helpers shared by the GPU tests (not collected by pytest)."""

import numpy as np
import torch

FORMATS = ["INT4", "MXINT4", "MXFP4", "NVFP4"]
FORMATS8 = ["INT8", "MXINT8"]
FORMATS_MINI = ["MXFP8_E4M3", "MXFP8_E5M2", "MXFP6_E2M3", "MXFP6_E3M2"]
ALL_FORMATS = FORMATS + FORMATS8 + FORMATS_MINI
GROUPS = {"INT4": 128, "MXINT4": 32, "MXFP4": 32, "NVFP4": 16, "INT8": 128, "MXINT8": 32,
          "MXFP8_E4M3": 32, "MXFP8_E5M2": 32, "MXFP6_E2M3": 32, "MXFP6_E3M2": 32}
BITS = {f: 4 for f in FORMATS}
BITS.update({"INT8": 8, "MXINT8": 8, "MXFP8_E4M3": 8, "MXFP8_E5M2": 8, "MXFP6_E2M3": 6,
             "MXFP6_E3M2": 6})
DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    """float32 stays float32; uint16 is read as bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def scales_np(t: torch.Tensor, fmt: str) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if fmt in ("INT4", "INT8") else a


def nibbles(codes: np.ndarray) -> np.ndarray:
    return np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(-1)


def elements(codes: np.ndarray, fmt: str) -> np.ndarray:
    """One entry per element: nibbles of the 4-bit formats, 6-bit fields of the bit stream
    of the 6-bit ones, bytes of the 8-bit ones."""
    codes = np.ascontiguousarray(codes).reshape(-1).view(np.uint8)
    if BITS[fmt] == 8:
        return codes
    if BITS[fmt] == 6:
        bits = np.unpackbits(codes, bitorder="little").reshape(-1, 6)
        return (bits << np.arange(6, dtype=np.uint8)).sum(axis=1).astype(np.uint8)
    return nibbles(codes)


def rel_err(a, b, floor=1e-30):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b) / np.maximum(np.abs(b), floor)


def near_projection_boundary(oracle, fmt: str, x: np.ndarray, tol: float = 1e-5) -> np.ndarray:
    """True where the projection of x changes within a relative distance tol."""
    x = np.asarray(x, np.float32)
    lo = oracle.project(fmt, (x * (1 - tol)).astype(np.float32))
    hi = oracle.project(fmt, (x * (1 + tol)).astype(np.float32))
    return lo != hi


def pack_codes(elems: np.ndarray, bits: int) -> np.ndarray:
    """Row-major element codes -> the library's code layout (nibbles low first, the 6-bit
    little-endian bit stream, or bytes)."""
    e = np.asarray(elems, dtype=np.uint8).reshape(-1)
    if bits == 8:
        return e.copy()
    if bits == 4:
        return (e[0::2] | (e[1::2] << 4)).astype(np.uint8)
    b = ((e[:, None] >> np.arange(6, dtype=np.uint8)) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(b, bitorder="little")


def random_codes(rng, fmt: str, rows: int, cols: int) -> np.ndarray:
    """Uniformly random finite element codes of an MX format (row-major, one per element)."""
    e = rng.integers(0, 1 << BITS[fmt], rows * cols).astype(np.uint8)
    if fmt == "MXFP8_E4M3":
        e[(e & 0x7F) == 0x7F] = 0x38
    if fmt == "MXFP8_E5M2":
        e[((e >> 2) & 31) == 31] = 0x3C
    return e
