"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the copy's or the
GEMM's arithmetic, and neither the GPU library nor the oracle is imported here.

The five workloads follow the shapes and value distributions of the GEMM page ("GEMM: la
moltiplicazione di matrici sull'hardware": the thousand-side product, the 8192-cube discussed
under tiling) and of the descriptor pages (a 128×64 bf16 box with 128-byte swizzle, a 5-D tensor
with element strides and NaN fill):

  c1  256³ GEMM, A/B uniform[-1,1], fp32 out; plus one 2-D copy of a {64,128} bf16 box
  c2  1024³ GEMM, N(0,1), bf16 out
  c3  3001×2049×777 GEMM, N(0,1), fp32 out (tiles overhang every edge); plus 5-D copies of a
      3×5×7×129×200 bf16 tensor, element strides {1,2,1,1,1}, NaN fill
  c4  8192³ GEMM, uniform[-1,1], bf16 out
  c5  M=16384, K=4096, N=14336; activations N(0,1); weights N(0, sd 0.02) stored N×K; bf16 out

Seeds: workload k draws A from seed 1000k+1 and B from 1000k+2 (torch.Generator, CPU);
"uniform[-1,1]" is 2·U[0,1)−1 in fp32 and N(0,σ) is σ·randn, both rounded to bf16 by torch's
round-to-nearest-even conversion.  Padding columns of a padded leading dimension are filled with
NaN so that any read of them shows up in the product.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

BF16_NAN_BITS = 0x7FC0


@dataclass(frozen=True)
class GemmWorkload:
    name: str
    M: int
    N: int
    K: int
    dist_a: Tuple[str, float]      # ("uniform", 1.0) or ("normal", sigma)
    dist_b: Tuple[str, float]
    b_layout: str                  # "kn" (row-major K×N) or "nk" (N×K, K contiguous)
    out_dtype: str                 # "f32" or "bf16"
    seed_a: int
    seed_b: int
    lda: Optional[int] = None      # default: dense
    ldb: Optional[int] = None
    ldc: Optional[int] = None

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def lds(self):
        lda = self.lda if self.lda is not None else self.K
        ldb = self.ldb if self.ldb is not None else (self.N if self.b_layout == "kn" else self.K)
        ldc = self.ldc if self.ldc is not None else self.N
        return lda, ldb, ldc


@dataclass(frozen=True)
class CopyWorkload:
    name: str
    shape_outer_first: Tuple[int, ...]   # as written in the workload text (outermost first)
    dtype: str
    box: Tuple[int, ...]                 # innermost first
    estr: Tuple[int, ...]                # innermost first
    swizzle: str
    oob: str                             # "zero" or "nan"
    seed: int
    dist: Tuple[str, float]
    coords: Tuple[Tuple[int, ...], ...] = field(default_factory=tuple)

    @property
    def dims(self):
        return tuple(reversed(self.shape_outer_first))


GEMMS = {
    "c1": GemmWorkload("c1", 256, 256, 256, ("uniform", 1.0), ("uniform", 1.0), "kn", "f32", 1001, 1002),
    "c2": GemmWorkload("c2", 1024, 1024, 1024, ("normal", 1.0), ("normal", 1.0), "kn", "bf16", 2001, 2002),
    "c3": GemmWorkload("c3", 3001, 2049, 777, ("normal", 1.0), ("normal", 1.0), "kn", "f32", 3001, 3002),
    "c3_bf16": GemmWorkload("c3_bf16", 3001, 2049, 777, ("normal", 1.0), ("normal", 1.0), "kn", "bf16", 3001, 3002),
    "c3_padded": GemmWorkload("c3_padded", 3001, 2049, 777, ("normal", 1.0), ("normal", 1.0), "kn", "f32",
                              3001, 3002, lda=784, ldb=2056, ldc=2056),
    "c4": GemmWorkload("c4", 8192, 8192, 8192, ("uniform", 1.0), ("uniform", 1.0), "kn", "bf16", 4001, 4002),
    "c5": GemmWorkload("c5", 16384, 14336, 4096, ("normal", 1.0), ("normal", 0.02), "nk", "bf16", 5001, 5002),
}


def _c1_copy_coords():
    inb = tuple((x, y) for y in (0, 128) for x in (0, 64, 128, 192))
    return ((0, 0),) + inb[1:] + ((224, 192), (-32, -64))


def _c3_copy_coords():
    out = []
    for x4 in (0, 2):
        for x3 in (0, 2, 4):
            for x2 in (0, 4):
                for x1 in range(0, 129, 16):
                    for x0 in (0, 64, 128, 192):
                        out.append((x0, x1, x2, x3, x4))
    return tuple(out)


COPIES = {
    "c1_copy": CopyWorkload("c1_copy", (256, 256), "bf16", (64, 128), (1, 1), "128B", "zero", 1001,
                            ("uniform", 1.0), _c1_copy_coords()),
    "c3_copy": CopyWorkload("c3_copy", (3, 5, 7, 129, 200), "bf16", (64, 16, 4, 2, 2), (1, 2, 1, 1, 1), "none",
                            "nan", 3003, ("normal", 1.0), _c3_copy_coords()),
}


def _draw(shape, dist, seed) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    kind, p = dist
    if kind == "uniform":
        x = torch.rand(shape, generator=g, dtype=torch.float32) * (2.0 * p) - p
    elif kind == "normal":
        x = torch.randn(shape, generator=g, dtype=torch.float32) * p
    else:
        raise ValueError(kind)
    return x.to(torch.bfloat16)


def matrix(rows: int, cols: int, ld: int, dist, seed: int) -> torch.Tensor:
    """A rows×cols bf16 matrix in a row-major buffer of leading dimension ld (CPU tensor of
    rows×ld); columns cols..ld-1 hold NaN."""
    vals = _draw((rows, cols), dist, seed)
    if ld == cols:
        return vals.contiguous()
    buf = torch.empty((rows, ld), dtype=torch.bfloat16)
    buf.view(torch.int16).fill_(BF16_NAN_BITS)
    buf[:, :cols] = vals
    return buf


def gemm_inputs(w: GemmWorkload):
    """(A, B) as CPU bf16 tensors laid out with the workload's leading dimensions."""
    lda, ldb, _ = w.lds()
    A = matrix(w.M, w.K, lda, w.dist_a, w.seed_a)
    if w.b_layout == "kn":
        B = matrix(w.K, w.N, ldb, w.dist_b, w.seed_b)
    else:
        B = matrix(w.N, w.K, ldb, w.dist_b, w.seed_b)
    return A, B


def copy_source(w: CopyWorkload) -> torch.Tensor:
    """The tensor a copy workload reads, as a contiguous CPU tensor (outermost dim first)."""
    if w.name == "c1_copy":
        g = GEMMS["c1"]
        return matrix(g.M, g.K, g.K, g.dist_a, g.seed_a)
    return _draw(w.shape_outer_first, w.dist, w.seed).contiguous()


def random_gemm_shape(rng: np.random.Generator, max_dim: int = 300):
    """A small random GEMM case: sizes in [1, max_dim], layout, output dtype, padded leads."""
    M, N, K = (int(rng.integers(1, max_dim + 1)) for _ in range(3))
    b_layout = "kn" if rng.integers(0, 2) == 0 else "nk"
    out = "f32" if rng.integers(0, 2) == 0 else "bf16"
    pad = int(rng.integers(0, 3))
    return M, N, K, b_layout, out, pad


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a bf16 CPU tensor as a numpy uint16 array."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
