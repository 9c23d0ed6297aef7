"""Helpers shared by the GPU tests (not collected by pytest)."""

import numpy as np
import torch

FORMATS = ["INT4", "MXINT4", "MXFP4", "NVFP4"]
FORMATS8 = ["INT8", "MXINT8"]
ALL_FORMATS = FORMATS + FORMATS8
GROUPS = {"INT4": 128, "MXINT4": 32, "MXFP4": 32, "NVFP4": 16, "INT8": 128, "MXINT8": 32}
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
    """One entry per element: nibbles of the 4-bit formats, bytes of the 8-bit ones."""
    return codes.reshape(-1) if fmt in ("INT8", "MXINT8") else nibbles(codes)


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
