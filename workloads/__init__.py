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

Convolution workloads (the im2col copy mode of "2 · Le Tensor Memory Accelerator" turns a 2-D
convolution into a GEMM; the pages give no convolution sizes): layers in the shape of an image
network's — 3×3 filters with padding 1, a strided 3×3, a dilated 3×3, a 1×1, a 7×7 stem on three
channels — plus the benchmark layer conv_b (batch 32, 56×56, 128 → 128 channels, 3×3).  Inputs
and filters are N(0,1) scaled by 1/sqrt(R·S·C) for the filters (the usual initialisation), seeds
6000+2i and 6000+2i+1 for workload i.

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


@dataclass(frozen=True)
class ConvWorkload:
    name: str
    n: int
    h: int
    w: int
    c: int
    k: int
    r: int
    s: int
    pad: Tuple[int, int, int, int] = (0, 0, 0, 0)   # top, left, bottom, right
    stride: Tuple[int, int] = (1, 1)                # h, w
    dil: Tuple[int, int] = (1, 1)                   # h, w
    out_dtype: str = "bf16"
    seed: int = 6000

    def out_dims(self):
        oh = (self.h + self.pad[0] + self.pad[2] - self.dil[0] * (self.r - 1) - 1) // self.stride[0] + 1
        ow = (self.w + self.pad[1] + self.pad[3] - self.dil[1] * (self.s - 1) - 1) // self.stride[1] + 1
        return oh, ow

    @property
    def M(self) -> int:
        oh, ow = self.out_dims()
        return self.n * oh * ow

    @property
    def flops(self) -> int:
        """2 · (output elements) · (taps inside or outside the image) · C: the GEMM's count."""
        return 2 * self.M * self.k * self.r * self.s * self.c


CONVS = {
    "conv_3x3": ConvWorkload("conv_3x3", 2, 17, 17, 24, 36, 3, 3, (1, 1, 1, 1), out_dtype="f32", seed=6000),
    "conv_c20": ConvWorkload("conv_c20", 2, 15, 13, 20, 40, 3, 3, (1, 1, 1, 1), seed=6002),
    "conv_stride2": ConvWorkload("conv_stride2", 3, 23, 23, 64, 80, 3, 3, (1, 1, 0, 1), (2, 2), out_dtype="f32",
                                 seed=6004),
    "conv_dil2": ConvWorkload("conv_dil2", 2, 20, 25, 32, 64, 3, 3, (2, 2, 2, 2), dil=(2, 2), seed=6006),
    "conv_1x1": ConvWorkload("conv_1x1", 4, 14, 14, 128, 96, 1, 1, out_dtype="f32", seed=6008),
    "conv_stem": ConvWorkload("conv_stem", 2, 32, 32, 3, 64, 7, 7, (3, 3, 3, 3), (2, 2), seed=6010),
    "conv_b": ConvWorkload("conv_b", 32, 56, 56, 128, 128, 3, 3, (1, 1, 1, 1), seed=6012),
    # stride-1 layers for the halo kernel: tiles of whole output rows, the last one of an image
    # partial, output channels past a multiple of 128, 1..4 window atoms per wave and tap; 3×3
    # filters (the unrolled nine-tap loop) over one, two and three 32-channel blocks
    "conv_halo_rows": ConvWorkload("conv_halo_rows", 2, 30, 30, 64, 160, 3, 3, (1, 1, 1, 1), out_dtype="f32",
                                   seed=6014),
    "conv_halo_wide": ConvWorkload("conv_halo_wide", 3, 9, 100, 96, 64, 3, 2, (1, 0, 1, 1), seed=6016),
    "conv_halo_small": ConvWorkload("conv_halo_small", 4, 8, 8, 32, 48, 3, 3, (1, 1, 1, 1), out_dtype="f32",
                                    seed=6018),
    "conv_halo_1x3": ConvWorkload("conv_halo_1x3", 2, 12, 24, 32, 40, 1, 3, (0, 1, 0, 1), seed=6020),
    "conv_halo_c96": ConvWorkload("conv_halo_c96", 2, 20, 20, 96, 72, 3, 3, (1, 1, 1, 1), out_dtype="f32",
                                  seed=6022),
    # a window of 4 × 202 = 808 pixels (51 atoms), in the range the unpadded 64-byte pixels opened
    "conv_halo_808": ConvWorkload("conv_halo_808", 1, 6, 200, 32, 40, 3, 3, (1, 1, 1, 1), seed=6024),
    # the largest window the halo kernel takes, 3 × 336 = 1008 pixels (63 atoms), and one past it
    # (3 × 337 = 1011: refused)
    "conv_halo_max": ConvWorkload("conv_halo_max", 1, 2, 334, 32, 16, 3, 3, (1, 1, 1, 1), out_dtype="f32",
                                  seed=6026),
    "conv_halo_over": ConvWorkload("conv_halo_over", 1, 2, 335, 32, 16, 3, 3, (1, 1, 1, 1), seed=6028),
}


def conv_inputs(w: ConvWorkload):
    """(X NHWC, W KRSC) as contiguous CPU bf16 tensors."""
    x = _draw((w.n, w.h, w.w, w.c), ("normal", 1.0), w.seed)
    f = _draw((w.k, w.r, w.s, w.c), ("normal", 1.0 / float(np.sqrt(w.r * w.s * w.c))), w.seed + 1)
    return x.contiguous(), f.contiguous()


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


def _a_box_coords(rows: int, cols: int, bx: int, by: int):
    """Every box of a rows×cols matrix in a grid of bx columns × by rows (innermost first)."""
    return tuple((x, y) for y in range(0, rows, by) for x in range(0, cols, bx))


COPIES = {
    "c1_copy": CopyWorkload("c1_copy", (256, 256), "bf16", (64, 128), (1, 1), "128B", "zero", 1001,
                            ("uniform", 1.0), _c1_copy_coords()),
    "c3_copy": CopyWorkload("c3_copy", (3, 5, 7, 129, 200), "bf16", (64, 16, 4, 2, 2), (1, 2, 1, 1, 1), "none",
                            "nan", 3003, ("normal", 1.0), _c3_copy_coords()),
    # The 8192x8192 GEMM's A operand cut into all of its 8192 boxes of 64 columns x 128 rows with
    # the 128-byte swizzle: the worked box's copy at a size where HBM bandwidth, not launch
    # latency, bounds the kernel (128 MiB read, 128 MiB of images written).
    "c4_a_boxes": CopyWorkload("c4_a_boxes", (8192, 8192), "bf16", (64, 128), (1, 1), "128B", "zero", 4001,
                               ("uniform", 1.0), _a_box_coords(8192, 8192, 64, 128)),
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
    if w.name in ("c1_copy", "c4_a_boxes"):
        g = GEMMS["c1" if w.name == "c1_copy" else "c4"]
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
