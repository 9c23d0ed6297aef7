"""Seeded synthetic inputs shaped like the workloads DualQuant is evaluated on.

The DualQuant pages measure on real Llama/Qwen weights and activations, which are not
available here.  These generators stand in for them: projection-shaped matrices with
heavy-tailed entries and a few outlier input columns (the structure the pages' Fig. 1
and the "one outlier inflates the entire row" remark describe), and activations with
outlier channels (the pages' Table 6 discussion of k/v activation outliers).

This module holds no quantization arithmetic: only random draws, outlier-column
placement and the fp64 -> fp32 -> bf16 cast.  The CPU oracle and the GPU path
consume the very same buffers, so only same-host reproducibility is needed.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def outlier_count(n: int, frac: float) -> int:
    """round-half-up(frac * n)."""
    return int(math.floor(frac * n + 0.5))


def outlier_columns(n: int, k: int, seed: int, stream: int) -> np.ndarray:
    """k distinct column indices, drawn on a stream of their own."""
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    rng = _rng(seed, stream + 1_000_003)
    return np.sort(rng.choice(n, size=k, replace=False)).astype(np.int64)


def draw(dist: str, shape, std: float, seed: int, stream: int, nu: int = 0) -> np.ndarray:
    """fp64 draws with the requested standard deviation."""
    rng = _rng(seed, stream)
    if dist == "normal":
        return rng.standard_normal(shape) * std
    if dist == "student_t":
        if nu <= 2:
            raise ValueError("Student-t needs nu > 2 for a finite variance")
        return rng.standard_t(nu, shape) * (std / math.sqrt(nu / (nu - 2.0)))
    if dist == "laplace":
        return rng.laplace(0.0, std / math.sqrt(2.0), shape)
    raise ValueError(f"unknown distribution {dist!r}")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class MatrixSpec:
    rows: int
    cols: int
    dist: str
    std: float
    nu: int = 0
    outliers: int = 0          # number of outlier columns
    outlier_scale: float = 1.0
    dtype: str = "bf16"        # "bf16" (uint16 bit patterns) or "f32"
    stream: int = 1

    def scaled(self, rows: int, cols: int) -> "MatrixSpec":
        """Same recipe at another size (outlier fraction kept)."""
        frac = self.outliers / self.cols
        return replace(self, rows=rows, cols=cols, outliers=outlier_count(cols, frac))


def matrix(spec: MatrixSpec, seed: int = 0) -> np.ndarray:
    """Row-major rows x cols matrix: float32, or uint16 bf16 bit patterns."""
    x = draw(spec.dist, (spec.rows, spec.cols), spec.std, seed, spec.stream, spec.nu)
    cols = outlier_columns(spec.cols, spec.outliers, seed, spec.stream)
    if cols.size:
        x[:, cols] *= spec.outlier_scale
    x32 = x.astype(np.float32)
    del x
    if spec.dtype == "f32":
        return x32
    if spec.dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {spec.dtype!r}")


# Workloads (out x in, row-major).  Formats: INT4 g=128, MXFP4 g=32, NVFP4 g=16, MXINT4 g=32.
WORKLOADS = {
    # 256x512 fp32, N(0, 0.02), 5 outlier input columns x20; INT4 symmetric g=128, 16 iterations
    "w256x512_int4": dict(
        W=MatrixSpec(256, 512, "normal", 0.02, outliers=5, outlier_scale=20.0, dtype="f32", stream=1),
        fmt="INT4", group=128, iters=16),
    # q_proj-shaped 4096x4096 bf16, Student-t nu=4 std 0.02, 1% outlier columns x15; MXFP4, 16 iterations
    "q4096x4096_mxfp4": dict(
        W=MatrixSpec(4096, 4096, "student_t", 0.02, nu=4, outliers=outlier_count(4096, 0.01),
                     outlier_scale=15.0, stream=2),
        fmt="MXFP4", group=32, iters=16),
    # down_proj-shaped 4096x14336 bf16, Student-t nu=3 std 0.015, 0.5% outlier columns x25; NVFP4, 16 iterations
    "down4096x14336_nvfp4": dict(
        W=MatrixSpec(4096, 14336, "student_t", 0.015, nu=3, outliers=outlier_count(14336, 0.005),
                     outlier_scale=25.0, stream=3),
        fmt="NVFP4", group=16, iters=16),
    # down_proj-shaped 3584x18944 bf16 (Qwen2.5-7B widths: wider than the row pass keeps in LDS),
    # same recipe as the 4096x14336 one; NVFP4, 16 iterations
    "down3584x18944_nvfp4": dict(
        W=MatrixSpec(3584, 18944, "student_t", 0.015, nu=3, outliers=outlier_count(18944, 0.005),
                     outlier_scale=25.0, stream=6),
        fmt="NVFP4", group=16, iters=16),
    # down_proj-shaped 5120x17408 bf16 (Qwen3-14B widths: 20 rows per row-pass workgroup), same
    # recipe; NVFP4, 16 iterations
    "down5120x17408_nvfp4": dict(
        W=MatrixSpec(5120, 17408, "student_t", 0.015, nu=3, outliers=outlier_count(17408, 0.005),
                     outlier_scale=25.0, stream=7),
        fmt="NVFP4", group=16, iters=16),
    # k_proj-shaped 1024x4096 bf16, Laplace std 0.02, 2% outlier columns x20; MXINT4, 16 iterations;
    # activations 2048x4096 N(0,1) with 1% channels x50 (drawn independently of W's columns)
    "k1024x4096_mxint4": dict(
        W=MatrixSpec(1024, 4096, "laplace", 0.02, outliers=outlier_count(4096, 0.02),
                     outlier_scale=20.0, stream=4),
        X=MatrixSpec(2048, 4096, "normal", 1.0, outliers=outlier_count(4096, 0.01),
                     outlier_scale=50.0, stream=5),
        fmt="MXINT4", group=32, iters=16),
}

# Llama-3.1-8B projection shapes (out x in) for the 32-layer batched set; NVFP4, 20 iterations.
LLAMA31_8B_PROJ = (
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336),
)
LLAMA31_8B_LAYERS = 32


def llama_projection_spec(layer: int, proj_index: int) -> MatrixSpec:
    name, rows, cols = LLAMA31_8B_PROJ[proj_index]
    return MatrixSpec(rows, cols, "student_t", 0.02, nu=4, outliers=outlier_count(cols, 0.01),
                      outlier_scale=15.0, stream=100 + 7 * layer + proj_index)


def matrix_device(spec: MatrixSpec, seed: int, device):
    """The same recipe drawn on a GPU with torch's seeded generator (its own random stream,
    not the numpy draws above): for large batches whose members are checked by properties
    rather than against the oracle.  Returns a bf16 (or fp32) torch tensor on `device`."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed((int(seed) * 1_000_003 + int(spec.stream)) & 0x7FFFFFFFFFFF)
    shape = (spec.rows, spec.cols)
    if spec.dist == "normal":
        x = torch.randn(shape, generator=gen, device=device) * spec.std
    elif spec.dist == "student_t":
        z = torch.randn(shape, generator=gen, device=device)
        chi2 = torch.zeros(shape, device=device)
        for _ in range(int(spec.nu)):   # chi-square with nu degrees of freedom
            chi2 += torch.randn(shape, generator=gen, device=device) ** 2
        x = z / torch.sqrt(chi2 / spec.nu) * (spec.std / math.sqrt(spec.nu / (spec.nu - 2.0)))
        del z, chi2
    elif spec.dist == "laplace":
        u = torch.rand(shape, generator=gen, device=device) - 0.5
        x = -torch.sign(u) * torch.log1p(-2.0 * u.abs()) * (spec.std / math.sqrt(2.0))
    else:
        raise ValueError(f"unknown distribution {spec.dist!r}")
    if spec.outliers:
        cg = torch.Generator()
        cg.manual_seed((int(seed) * 1_000_003 + int(spec.stream) + 1_000_003) & 0x7FFFFFFFFFFF)
        cols = torch.randperm(spec.cols, generator=cg)[:spec.outliers].to(device)
        x[:, cols] *= spec.outlier_scale
    return x.to(torch.bfloat16 if spec.dtype == "bf16" else torch.float32).contiguous()


def workload(name: str, seed: int = 0):
    """(W, X or None, fmt, group, iters) for a named workload."""
    w = WORKLOADS[name]
    W = matrix(w["W"], seed)
    X = matrix(w["X"], seed) if "X" in w else None
    return W, X, w["fmt"], w["group"], w["iters"]
