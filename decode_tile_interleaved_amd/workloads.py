"""Seeded synthetic weight matrices for the lattice-rANS decode workloads.

These generators hold none of the method's arithmetic: they only draw the
inputs (torch CPU generator, float32, then cast to the container dtype with
round-to-nearest-even).  Both the product path and the CPU oracle are fed
from here.  The pages measure on Z-Image-Turbo's linear weights, which are
not available; these matrices stand in with the shapes and distributions
listed below.
"""
from __future__ import annotations

import math

import torch

# name -> (rows, cols, container, target_bpp, seed)
WORKLOADS = {
    "gauss256_bf16_3.5": (256, 256, torch.bfloat16, 3.5, 1001),
    "rowscale4096_bf16_4.0": (4096, 4096, torch.bfloat16, 4.0, 1002),
    "t4outlier3072x12288_bf16_2.75": (3072, 12288, torch.bfloat16, 2.75, 1003),
    "absmax8192_int8_3.0": (8192, 8192, torch.int8, 3.0, 1004),
    "absmax8192_fp8_3.0": (8192, 8192, torch.float8_e4m3fn, 3.0, 1004),
    # the 4096x4096 matrix at a low rate (its stream has 16 states per tile)
    "rowscale4096_bf16_0.2": (4096, 4096, torch.bfloat16, 0.2, 1002),
}

# DiT-like stack: 30 blocks x {4 x (3840,3840), (10240,3840), (3840,10240)} as (out, in)
DIT_BLOCKS = 30
DIT_SHAPES = [(3840, 3840)] * 4 + [(10240, 3840), (3840, 10240)]


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def gaussian(rows: int, cols: int, std: float, seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    """i.i.d. N(0, std^2) entries."""
    g = _gen(seed)
    return (torch.randn(rows, cols, generator=g, dtype=torch.float32) * std).to(dtype)


def rowscale_gaussian(rows: int, cols: int, seed: int, lo: float = 0.005, hi: float = 0.05,
                      dtype=torch.bfloat16) -> torch.Tensor:
    """Row r has std exp(U[ln lo, ln hi]); entries N(0, std_r^2)."""
    g = _gen(seed)
    sig = torch.exp(torch.empty(rows, 1, dtype=torch.float64).uniform_(math.log(lo), math.log(hi), generator=g))
    w = torch.randn(rows, cols, generator=g, dtype=torch.float32) * sig.to(torch.float32)
    return w.to(dtype)


def t4_outliers(rows: int, cols: int, seed: int, std: float = 0.02, frac: float = 0.001, mult: float = 20.0,
                dtype=torch.bfloat16) -> torch.Tensor:
    """Student-t (nu=4) scaled to std `std`, then floor(frac*numel) positions
    (seeded, without replacement) replaced by +-mult*std with random sign."""
    g = _gen(seed)
    n = rows * cols
    z = torch.randn(n, generator=g, dtype=torch.float32)
    u1 = torch.rand(n, generator=g, dtype=torch.float32).clamp_min_(1e-30)
    u2 = torch.rand(n, generator=g, dtype=torch.float32).clamp_min_(1e-30)
    chi2_4 = -2.0 * (torch.log(u1) + torch.log(u2))       # chi-square with 4 dof
    t = z / torch.sqrt(chi2_4 / 4.0)                        # Student-t, nu = 4, variance 2
    w = t * (std / math.sqrt(2.0))
    k = int(frac * n)
    idx = torch.randperm(n, generator=g)[:k]
    sign = torch.where(torch.rand(k, generator=g) < 0.5, -1.0, 1.0)
    w[idx] = sign * (mult * std)
    return w.reshape(rows, cols).to(dtype)


def absmax_weights(rows: int, cols: int, seed: int, kind: str) -> tuple[torch.Tensor, torch.Tensor]:
    """The N(0,1) float32 weights behind absmax_codes and their per-row code
    scale (absmax/127 for INT8, absmax/448 for FP8): weight ~ code * scale."""
    if kind not in ("int8", "fp8"):
        raise ValueError(kind)
    g = _gen(seed)
    w = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    amax = w.abs().amax(dim=1, keepdim=True).clamp_min(1e-30)
    return w, amax / (127.0 if kind == "int8" else 448.0)


def absmax_codes(rows: int, cols: int, seed: int, kind: str) -> torch.Tensor:
    """Symmetric per-row absmax codes of N(0,1) weights: INT8 in [-127, 127]
    (round half to even) or FP8-E4M3FN in [-448, 448]."""
    w, scale = absmax_weights(rows, cols, seed, kind)
    if kind == "int8":
        return torch.clamp(torch.round(w / scale), -127, 127).to(torch.int8)
    return torch.clamp(w / scale, -448.0, 448.0).to(torch.float8_e4m3fn)


def make(name: str) -> tuple[torch.Tensor, float]:
    """(matrix, target_bpp) for a named workload."""
    rows, cols, dtype, target, seed = WORKLOADS[name]
    if name.startswith("gauss"):
        return gaussian(rows, cols, 0.02, seed, dtype), target
    if name.startswith("rowscale"):
        return rowscale_gaussian(rows, cols, seed, dtype=dtype), target
    if name.startswith("t4outlier"):
        return t4_outliers(rows, cols, seed, dtype=dtype), target
    if name.startswith("absmax"):
        return absmax_codes(rows, cols, seed, "int8" if dtype == torch.int8 else "fp8"), target
    raise KeyError(name)


def dit_matrix(block: int, j: int) -> torch.Tensor:
    """Weight j (0..5) of DiT block `block`, BF16 N(0, 0.02^2), seed 5000 + 6*block + j."""
    rows, cols = DIT_SHAPES[j]
    return gaussian(rows, cols, 0.02, 5000 + 6 * block + j)


def dit_activation(cols: int = 3840) -> torch.Tensor:
    """Prefill activation X (4096 x cols) BF16 N(0, 1), seed 4999."""
    return gaussian(4096, cols, 1.0, 4999)
