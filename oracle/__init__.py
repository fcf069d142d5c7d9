"""CPU oracle for the tiled copy and the bf16 GEMM — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may import this
package.  The GPU library never loads it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, built into ``liboracle.so`` by ``oracle/build.py``);
this module only marshals numpy arrays into it.  Every routine cites the passage it follows:

* ``swizzle`` — "H100 · cuTensorMap" §11.3 (XOR swizzle, per-mode bit lists).
* ``tiled_copy`` — "H100 · cuTensorMap" §8.2, §8.3, §9.1, §9.2, §14; "2 · Le Tensor Memory
  Accelerator" §2.2, §2.5 (box copy with element strides and out-of-bounds fill).
* ``gemm`` / ``gemm_points`` — "GEMM: la moltiplicazione di matrici sull'hardware", section
  "Il conto, e il problema della versione ingenua" (C = A·B, 2MNK) and the tensor-core section
  (16-bit inputs, wide accumulation).
* ``im2col_copy`` / ``conv2d`` — "2 · Le Tensor Memory Accelerator", section "im2col" (a copy
  mode that forms the im2col matrix of a convolution on the fly, so the convolution becomes a
  GEMM); the convolution itself by its definition.

Parity status: all routines pinned by ``tests/test_oracle_pins.py``; the GEMM is exact only up
to the summation order, which the pages leave open (tolerance 1e-2 relative / 1e-3 absolute).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

SWIZZLE_MODES = {"none": 0, "32B": 1, "64B": 2, "128B": 3, "128B_2ROW": 4, "128B_TR": 5}
# element type -> (element size, NaN kind understood by oracle.c; 0 = integer, no NaN)
DTYPES = {
    "u8": (1, 0), "u16": (2, 0), "u32": (4, 0),
    "f16": (2, 2), "bf16": (2, 1), "f32": (4, 3), "f8e4m3": (1, 4), "f8e5m2": (1, 5),
}

_u64p = ctypes.POINTER(ctypes.c_uint64)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)


class Oracle:
    """Handle on one build of ``liboracle.so`` (tests may load a deliberately broken build)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            from oracle import build as _b
            _b.build(out=path)
        lib = ctypes.CDLL(path)
        lib.oracle_swizzle.restype = ctypes.c_uint64
        lib.oracle_swizzle.argtypes = [ctypes.c_uint64, ctypes.c_int]
        lib.oracle_swizzle_array.restype = None
        lib.oracle_swizzle_array.argtypes = [_u64p, _u64p, ctypes.c_int64, ctypes.c_int]
        lib.oracle_tiled_copy.restype = ctypes.c_uint64
        lib.oracle_tiled_copy.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, _u64p, _u64p,
                                          _u32p, _u32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          _i32p, ctypes.c_void_p]
        lib.oracle_tiled_store.restype = ctypes.c_uint64
        lib.oracle_tiled_store.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, _u64p, _u64p, _u32p,
                                           _u32p, ctypes.c_int, _i32p, ctypes.c_void_p, ctypes.c_uint64]
        lib.oracle_gemm_rows.restype = None
        lib.oracle_gemm_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _u16p,
                                         ctypes.c_int64, _u16p, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_int64, ctypes.c_int64, _f64p, _f32p,
                                         ctypes.c_int64, ctypes.c_int, _f64p, ctypes.c_int]
        lib.oracle_gemm_points.restype = None
        lib.oracle_gemm_points.argtypes = [ctypes.c_int64, _u16p, ctypes.c_int64, _u16p,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_int64, _i64p,
                                           _i64p, _f64p, _f32p, ctypes.c_int]
        lib.oracle_f8_to_f64_array.restype = None
        lib.oracle_f8_to_f64_array.argtypes = [ctypes.c_void_p, _f64p, ctypes.c_int64, ctypes.c_int]
        lib.oracle_gemm_f8_rows.restype = None
        lib.oracle_gemm_f8_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                            ctypes.c_int64, _f64p, _f32p, ctypes.c_int64, ctypes.c_int]
        lib.oracle_f16_to_f64_array.restype = None
        lib.oracle_f16_to_f64_array.argtypes = [_u16p, _f64p, ctypes.c_int64]
        lib.oracle_f32_to_bf16_array.restype = None
        lib.oracle_f32_to_bf16_array.argtypes = [_f32p, _u16p, ctypes.c_int64]
        lib.oracle_conv_out_dim.restype = ctypes.c_int64
        lib.oracle_conv_out_dim.argtypes = [ctypes.c_int64] * 6
        lib.oracle_im2col_copy.restype = ctypes.c_uint64
        lib.oracle_im2col_copy.argtypes = [ctypes.c_int, ctypes.c_void_p, _u64p, _u64p, _i32p, _i32p, _i32p, _i32p,
                                           _i32p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, _i32p, ctypes.c_void_p]
        lib.oracle_conv2d_rows.restype = None
        lib.oracle_conv2d_rows.argtypes = [_u16p, _u16p] + [ctypes.c_int64] * 7 + [_i32p, ctypes.c_int64,
                                                                                     ctypes.c_int64, _f64p, _f32p,
                                                                                     ctypes.c_int64, ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        self.lib = lib
        self.path = path

    # -- O1 ---------------------------------------------------------------------------------
    def swizzle(self, offsets, mode: str | int):
        m = SWIZZLE_MODES[mode] if isinstance(mode, str) else int(mode)
        a = np.ascontiguousarray(np.asarray(offsets, dtype=np.uint64).reshape(-1))
        out = np.empty_like(a)
        self.lib.oracle_swizzle_array(a.ctypes.data_as(_u64p), out.ctypes.data_as(_u64p), a.size, m)
        return out.reshape(np.shape(offsets))

    # -- O2 ---------------------------------------------------------------------------------
    def tiled_copy(self, src: np.ndarray, dtype: str, dims: Sequence[int], strides_bytes: Sequence[int],
                   box: Sequence[int], estr: Sequence[int], swizzle: str | int, oob_nan: bool,
                   coords: Sequence[int]) -> np.ndarray:
        """Copy one box of ``src`` (raw bytes of the tensor; dims innermost first) to an image.

        Returns the image as a uint8 array.  Raises ValueError where the plain reference
        declines the arguments (rank, element stride 0, image not a whole number of swizzle
        spans, NaN fill of an integer type)."""
        elsize, nan_kind = DTYPES[dtype]
        rank = len(dims)
        m = SWIZZLE_MODES[swizzle] if isinstance(swizzle, str) else int(swizzle)
        n = [(int(b) + int(e) - 1) // int(e) for b, e in zip(box, estr)]
        image = elsize * int(np.prod(n))
        dst = np.zeros(max(image, 1), dtype=np.uint8)
        srcb = np.ascontiguousarray(src).view(np.uint8)
        d = np.array(list(dims) + [1] * (5 - rank), dtype=np.uint64)
        s = np.array(list(strides_bytes) + [0] * (5 - len(strides_bytes)), dtype=np.uint64)
        b = np.array(list(box) + [1] * (5 - rank), dtype=np.uint32)
        e = np.array(list(estr) + [1] * (5 - rank), dtype=np.uint32)
        c = np.array(list(coords) + [0] * (5 - rank), dtype=np.int32)
        got = self.lib.oracle_tiled_copy(elsize, rank, srcb.ctypes.data, d.ctypes.data_as(_u64p),
                                         s.ctypes.data_as(_u64p), b.ctypes.data_as(_u32p),
                                         e.ctypes.data_as(_u32p), m, int(bool(oob_nan)), nan_kind,
                                         c.ctypes.data_as(_i32p), dst.ctypes.data)
        if got == 0:
            raise ValueError("oracle_tiled_copy declined these arguments")
        assert got == image
        return dst[:image]

    def tiled_store(self, tensor: np.ndarray, dtype: str, dims: Sequence[int], strides_bytes: Sequence[int],
                    box: Sequence[int], estr: Sequence[int], swizzle: str | int, coords: Sequence[int],
                    image: np.ndarray) -> np.ndarray:
        """Store one box image into ``tensor`` (raw bytes; dims innermost first): the other
        direction of ``tiled_copy`` ("2 · Le Tensor Memory Accelerator" §2.5).  Returns a new
        uint8 array; positions of the box outside the tensor are not written."""
        elsize, _ = DTYPES[dtype]
        rank = len(dims)
        m = SWIZZLE_MODES[swizzle] if isinstance(swizzle, str) else int(swizzle)
        out = np.array(np.ascontiguousarray(tensor).view(np.uint8).reshape(-1), copy=True)
        img = np.ascontiguousarray(image).view(np.uint8).reshape(-1)
        d = np.array(list(dims) + [1] * (5 - rank), dtype=np.uint64)
        s = np.array(list(strides_bytes) + [0] * (5 - len(strides_bytes)), dtype=np.uint64)
        b = np.array(list(box) + [1] * (5 - rank), dtype=np.uint32)
        e = np.array(list(estr) + [1] * (5 - rank), dtype=np.uint32)
        c = np.array(list(coords) + [0] * (5 - rank), dtype=np.int32)
        got = self.lib.oracle_tiled_store(elsize, rank, out.ctypes.data, d.ctypes.data_as(_u64p),
                                          s.ctypes.data_as(_u64p), b.ctypes.data_as(_u32p),
                                          e.ctypes.data_as(_u32p), m, c.ctypes.data_as(_i32p),
                                          img.ctypes.data, img.size)
        if got == 0:
            raise ValueError("oracle_tiled_store declined these arguments")
        return out

    # -- O3 ---------------------------------------------------------------------------------
    def gemm(self, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int, lda: int, ldb: int,
             b_layout: str = "kn", rows: Optional[tuple] = None, want64: bool = False,
             threads: int = 0, ab: str = "bf16"):
        """C rows [m0, m1) of A·B.  A, B: uint16 bit arrays of bf16 (ab="bf16") or binary16
        (ab="f16") values (flat or 2-D, row-major with the given leading dimensions).  Returns
        float32 (m1-m0, N), plus the float64 sums if asked."""
        A = np.ascontiguousarray(A, dtype=np.uint16).reshape(-1)
        B = np.ascontiguousarray(B, dtype=np.uint16).reshape(-1)
        m0, m1 = rows if rows is not None else (0, M)
        bl = {"kn": 0, "nk": 1}[b_layout]
        out32 = np.empty((m1 - m0, N), dtype=np.float32)
        out64 = np.empty((m1 - m0, N), dtype=np.float64) if want64 else None
        nthr = threads if threads > 0 else self.lib.oracle_max_threads()
        scratch = np.empty(max(1, nthr) * max(N, 1) + 1, dtype=np.float64)
        if m1 > m0 and N > 0:
            self.lib.oracle_gemm_rows(M, N, K, A.ctypes.data_as(_u16p), lda, B.ctypes.data_as(_u16p), ldb,
                                      bl, m0, m1,
                                      out64.ctypes.data_as(_f64p) if want64 else None,
                                      out32.ctypes.data_as(_f32p), N, nthr, scratch.ctypes.data_as(_f64p),
                                      {"bf16": 0, "f16": 1}[ab])
        return (out32, out64) if want64 else out32

    def gemm_ex(self, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int, lda: int, ldb: int,
                b_layout: str, alpha: float, beta: float, C_old: Optional[np.ndarray] = None,
                rows: Optional[tuple] = None, threads: int = 0, ab: str = "bf16") -> np.ndarray:
        """C <- alpha·A·B + beta·C, the general BLAS form the "GEMM" page's tensor-core section
        gives for the matrix units.  alpha and beta are binary32 values; the sum S is gemm()'s
        binary64 sum; alpha·S + beta·C_old is formed in binary64 and rounded once to binary32.
        With beta == 0, C_old is not read (a NaN in it does not reach the result).  C_old: the
        old C rows as float32 (bf16 values widen exactly)."""
        _, s64 = self.gemm(A, B, M, N, K, lda, ldb, b_layout, rows=rows, want64=True, threads=threads, ab=ab)
        a = float(np.float32(alpha))
        b = float(np.float32(beta))
        r = a * s64
        if b != 0.0:
            r = r + b * np.asarray(C_old, dtype=np.float64)
        return r.astype(np.float32)

    def gemm_points(self, A: np.ndarray, B: np.ndarray, K: int, lda: int, ldb: int, ms, ns,
                    b_layout: str = "kn", want64: bool = False, ab: str = "bf16"):
        A = np.ascontiguousarray(A, dtype=np.uint16).reshape(-1)
        B = np.ascontiguousarray(B, dtype=np.uint16).reshape(-1)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        out32 = np.empty(ms.size, dtype=np.float32)
        out64 = np.empty(ms.size, dtype=np.float64)
        self.lib.oracle_gemm_points(K, A.ctypes.data_as(_u16p), lda, B.ctypes.data_as(_u16p), ldb,
                                    {"kn": 0, "nk": 1}[b_layout], ms.size, ms.ctypes.data_as(_i64p),
                                    ns.ctypes.data_as(_i64p), out64.ctypes.data_as(_f64p),
                                    out32.ctypes.data_as(_f32p), {"bf16": 0, "f16": 1}[ab])
        return (out32, out64) if want64 else out32

    # -- O2i / O5 ----------------------------------------------------------------------------
    def conv_out_dim(self, n: int, pad_lo: int, pad_hi: int, stride: int, dil: int, filt: int) -> int:
        return int(self.lib.oracle_conv_out_dim(n, pad_lo, pad_hi, stride, dil, filt))

    def im2col_copy(self, src: np.ndarray, dtype: str, dims: Sequence[int], strides_bytes: Sequence[int],
                    pad_lo: Sequence[int], pad_hi: Sequence[int], cstride: Sequence[int], dil: Sequence[int],
                    filt: Sequence[int], channels: int, pixels: int, swizzle: str | int, oob_nan: bool,
                    coords: Sequence[int]) -> np.ndarray:
        """One im2col block of the NHWC tensor ``src`` (raw bytes; dims {C, W, H, N}, strides
        {sW, sH, sN} in bytes; per-spatial arrays {along W, along H}; coords {c0, m0, s, r}).
        Returns the image as uint8 (pixels rows of channels elements, channel fastest)."""
        elsize, nan_kind = DTYPES[dtype]
        m = SWIZZLE_MODES[swizzle] if isinstance(swizzle, str) else int(swizzle)
        image = elsize * int(channels) * int(pixels)
        dst = np.zeros(max(image, 1), dtype=np.uint8)
        srcb = np.ascontiguousarray(src).view(np.uint8)
        arr = lambda v, t: np.array(list(v), dtype=t)  # noqa: E731
        d, st = arr(dims, np.uint64), arr(strides_bytes, np.uint64)
        pl, ph, cs, dl, fl, c = (arr(v, np.int32) for v in (pad_lo, pad_hi, cstride, dil, filt, coords))
        got = self.lib.oracle_im2col_copy(elsize, srcb.ctypes.data, d.ctypes.data_as(_u64p), st.ctypes.data_as(_u64p),
                                          pl.ctypes.data_as(_i32p), ph.ctypes.data_as(_i32p),
                                          cs.ctypes.data_as(_i32p), dl.ctypes.data_as(_i32p),
                                          fl.ctypes.data_as(_i32p), int(channels), int(pixels), m,
                                          int(bool(oob_nan)), nan_kind, c.ctypes.data_as(_i32p), dst.ctypes.data)
        if got == 0:
            raise ValueError("oracle_im2col_copy declined these arguments")
        assert got == image
        return dst[:image]

    def conv2d(self, X: np.ndarray, Wt: np.ndarray, n: int, h: int, w: int, c: int, k: int, r: int, s: int,
               pad=(0, 0, 0, 0), stride=(1, 1), dil=(1, 1), rows: Optional[tuple] = None, want64: bool = False,
               threads: int = 0):
        """Rows [m0, m1) of the 2-D convolution Y (N*OH*OW × K), X NHWC and Wt KRSC as uint16
        bf16 bits.  pad = (top, left, bottom, right), stride/dil = (h, w).  Returns float32
        rows (and the float64 sums if asked)."""
        X = np.ascontiguousarray(X, dtype=np.uint16).reshape(-1)
        Wt = np.ascontiguousarray(Wt, dtype=np.uint16).reshape(-1)
        geom = np.array([pad[0], pad[1], pad[2], pad[3], stride[0], stride[1], dil[0], dil[1]], dtype=np.int32)
        oh = self.conv_out_dim(h, pad[0], pad[2], stride[0], dil[0], r)
        ow = self.conv_out_dim(w, pad[1], pad[3], stride[1], dil[1], s)
        M = n * oh * ow
        m0, m1 = rows if rows is not None else (0, M)
        out32 = np.empty((m1 - m0, k), dtype=np.float32)
        out64 = np.empty((m1 - m0, k), dtype=np.float64) if want64 else None
        nthr = threads if threads > 0 else self.lib.oracle_max_threads()
        if m1 > m0 and k > 0:
            self.lib.oracle_conv2d_rows(X.ctypes.data_as(_u16p), Wt.ctypes.data_as(_u16p), n, h, w, c, k, r, s,
                                        geom.ctypes.data_as(_i32p), m0, m1,
                                        out64.ctypes.data_as(_f64p) if want64 else None,
                                        out32.ctypes.data_as(_f32p), k, nthr)
        return (out32, out64) if want64 else out32

    def f8_to_f64(self, bits: np.ndarray, fmt: str) -> np.ndarray:
        """OCP 8-bit float bit patterns (fmt "e4m3" or "e5m2") -> float64."""
        b = np.ascontiguousarray(bits, dtype=np.uint8)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_f8_to_f64_array(b.ctypes.data, out.reshape(-1).ctypes.data_as(_f64p), b.size,
                                        {"e4m3": 0, "e5m2": 1}[fmt])
        return out

    def gemm_f8(self, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int, lda: int, ldb: int, fmt: str,
                rows: Optional[tuple] = None, want64: bool = False, threads: int = 0):
        """C rows [m0, m1) of A·Bᵀ for 8-bit float inputs: A (M×K, lda) and B stored N×K (ldb) as
        uint8 bit arrays.  Returns float32 (m1-m0, N), plus the float64 sums if asked."""
        A = np.ascontiguousarray(A, dtype=np.uint8).reshape(-1)
        B = np.ascontiguousarray(B, dtype=np.uint8).reshape(-1)
        m0, m1 = rows if rows is not None else (0, M)
        out32 = np.empty((m1 - m0, N), dtype=np.float32)
        out64 = np.empty((m1 - m0, N), dtype=np.float64) if want64 else None
        nthr = threads if threads > 0 else self.lib.oracle_max_threads()
        if m1 > m0 and N > 0:
            self.lib.oracle_gemm_f8_rows(N, K, A.ctypes.data, lda, B.ctypes.data, ldb, {"e4m3": 0, "e5m2": 1}[fmt],
                                         m0, m1, out64.ctypes.data_as(_f64p) if want64 else None,
                                         out32.ctypes.data_as(_f32p), N, nthr)
        return (out32, out64) if want64 else out32

    def f16_to_f64(self, bits: np.ndarray) -> np.ndarray:
        """binary16 bit patterns -> float64, decoded from the format's definition."""
        b = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_f16_to_f64_array(b.reshape(-1).ctypes.data_as(_u16p), out.reshape(-1).ctypes.data_as(_f64p),
                                         b.size)
        return out

    def f32_to_bf16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_bf16_array(x.reshape(-1).ctypes.data_as(_f32p),
                                          out.reshape(-1).ctypes.data_as(_u16p), x.size)
        return out

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from ``oracle.c`` as committed (built on first use if absent)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact: bf16 is the top half of a binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def gemm_check(got: np.ndarray, ref32: np.ndarray, rtol: float = 1e-2, atol: float = 1e-3,
               extra: Optional[np.ndarray] = None) -> dict:
    """O4: a GPU value g passes iff it is finite and |g − r| ≤ max(rtol·|r|, atol) (+ extra, when
    given: a per-entry widening of the bound, see gemm_check_f8), where r is the oracle's binary32
    result (before any bf16 rounding).  The tolerance is the one the GEMM's contract fixes: 1e-2
    relative, 1e-3 absolute on entries below 0.1 in magnitude, where 1e-2·|r| < 1e-3.  `got` and
    `ref32` must have the same shape (no broadcasting).  Returns the statistics and the verdict."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref32, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"result shape {g.shape} differs from the reference shape {r.shape}")
    err = np.abs(g - r)
    bound = np.maximum(rtol * np.abs(r), atol)
    if extra is not None:
        e = np.asarray(extra, dtype=np.float64)
        if e.shape != r.shape:
            raise ValueError(f"bound widening shape {e.shape} differs from the reference shape {r.shape}")
        bound = bound + e
    finite = np.isfinite(g)
    ok = finite & (err <= bound)
    rel = err / np.maximum(np.abs(r), 1e-30)
    return {
        "pass": bool(ok.all()),
        "n": int(g.size),
        "n_fail": int((~ok).sum()),
        "max_abs_err": float(err.max()) if g.size else 0.0,
        "max_rel_err": float(np.where(np.abs(r) >= atol / rtol, rel, 0.0).max()) if g.size else 0.0,
        "n_abs_branch": int((np.abs(r) < atol / rtol).sum()),
    }


# The 8-bit matrix instruction's own error, a hardware characterisation (not from the pages, which
# fix only fp32 accumulation): gfx950's 16×16×128 fp8 product adds its 128 exact products with
# about 16 significant bits relative to the sum of their magnitudes.  The GPU test
# test_fp8_instruction_error measures it on single instructions (K = 128) and requires at most
# 2^-15 · Σ|a_k·b_k|; fp8 results are checked with four times that.
F8_DOT_BOUND = 2.0 ** -13


def gemm_check_f8(got: np.ndarray, ref32: np.ndarray, a_vals: np.ndarray, b_vals_nk: np.ndarray,
                  dot_bound: float = F8_DOT_BOUND) -> dict:
    """O4 for 8-bit float inputs: gemm_check with each entry's bound widened by
    dot_bound · Σ_k |A[m,k]|·|B[n,k]| (binary64), the matrix instruction's forward error.
    a_vals (M×K) and b_vals_nk (N×K) are the decoded input values; B is stored N×K."""
    a = np.abs(np.asarray(a_vals, dtype=np.float64))
    b = np.abs(np.asarray(b_vals_nk, dtype=np.float64))
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"operands {a.shape} and {b.shape} are not M×K and N×K")
    absum = a @ b.T
    r = gemm_check(got, ref32, extra=dot_bound * absum)
    g = np.asarray(got, dtype=np.float64)
    err = np.abs(g - np.asarray(ref32, dtype=np.float64))
    r["max_err_over_abs_dot"] = float((err / np.maximum(absum, 1e-30)).max()) if g.size else 0.0
    return r
