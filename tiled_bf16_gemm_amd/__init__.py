"""Python binding of the gfx950 tiled bf16 GEMM / tiled-copy library (``include/tbg.h``).

Argument marshalling only: every function forwards to the C ABI of ``libtbg.so`` (built in-tree
by ``tiled_bf16_gemm_amd/build.py``), whose kernels do all of the work.  Importing this package
fails loudly when the library has not been built; there is no fallback path.

Names follow the C ABI without the ``tbg_`` prefix.  Pointers are plain integers (device
addresses, e.g. ``tensor.data_ptr()``); ``stream`` is a HIP stream handle as an integer
(``torch.cuda.current_stream().cuda_stream``) or ``None`` for the default stream.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtbg.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tbg.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python tiled_bf16_gemm_amd/build.py` "
                      "(or __graft_entry__.build()); there is no non-GPU fallback")

# The library must bind to the same HIP runtime as the framework that owns the device memory and
# streams it is handed.  PyTorch ships its own libamdhip64 (same soname); importing torch first
# makes the dynamic linker resolve libtbg.so's dependency to that already-loaded runtime instead
# of loading a second runtime instance, which could not see torch's streams or allocations.
try:
    import torch  # noqa: F401
except ImportError:  # plain C-ABI use without PyTorch: the system ROCm runtime is used
    pass

_lib = ctypes.CDLL(LIB_PATH)

# ---- enums (values as in tbg.h) -------------------------------------------------------------
OK, ERR_INVALID_VALUE, ERR_MISALIGNED, ERR_UNSUPPORTED, ERR_OUT_OF_RANGE, ERR_NO_DEVICE, ERR_HIP = range(7)
DTYPES = {"u8": 0, "u16": 1, "u32": 2, "f16": 3, "bf16": 4, "f32": 5, "f8e4m3": 6, "f8e5m2": 7}
ELSIZE = {"u8": 1, "u16": 2, "u32": 4, "f16": 2, "bf16": 2, "f32": 4, "f8e4m3": 1, "f8e5m2": 1}
SWIZZLES = {"none": 0, "32B": 1, "64B": 2, "128B": 3, "128B_2ROW": 4, "128B_TR": 5}
OOB = {"zero": 0, "nan": 1}
L2 = {"none": 0, "64B": 1, "128B": 2, "256B": 3}
B_LAYOUTS = {"kn": 0, "nk": 1}
PIPELINES = {"auto": 0, "ring": 1, "producer": 2}
INTERLEAVES = {"none": 0, "16B": 1, "32B": 2}


class TensorDesc(ctypes.Structure):
    """tbg_tensor_desc: 128 bytes, plain data."""
    _fields_ = [("opaque", ctypes.c_uint64 * 16)]


class GemmConfig(ctypes.Structure):
    """tbg_gemm_config: workgroup tile, ring stages and copy pipeline (0 = the library's choice)."""
    _fields_ = [("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("pipeline", ctypes.c_int32)]


def gemm_config(tile=None, stages: int = 0, pipeline="auto") -> GemmConfig:
    """Build a GemmConfig; tile is None, (bm, bn) or "BMxBN"."""
    if tile is None:
        bm = bn = 0
    elif isinstance(tile, str):
        bm, bn = (int(x) for x in tile.lower().split("x"))
    else:
        bm, bn = tile
    return GemmConfig(int(bm), int(bn), int(stages), _enum(PIPELINES, pipeline))


class Conv2dShape(ctypes.Structure):
    """tbg_conv2d_shape: NHWC input, KRSC filters, padding (before/after), strides, dilations."""
    _fields_ = [("n", ctypes.c_int64), ("h", ctypes.c_int64), ("w", ctypes.c_int64), ("c", ctypes.c_int64),
                ("k", ctypes.c_int64), ("r", ctypes.c_int32), ("s", ctypes.c_int32), ("pad_h", ctypes.c_int32),
                ("pad_w", ctypes.c_int32), ("pad_h_end", ctypes.c_int32), ("pad_w_end", ctypes.c_int32),
                ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32), ("dil_h", ctypes.c_int32),
                ("dil_w", ctypes.c_int32)]


def conv2d_shape(n, h, w, c, k, r, s, pad=(0, 0, 0, 0), stride=(1, 1), dil=(1, 1)) -> Conv2dShape:
    """pad = (top, left, bottom, right); stride and dil = (h, w)."""
    return Conv2dShape(n, h, w, c, k, r, s, pad[0], pad[1], pad[2], pad[3], stride[0], stride[1], dil[0], dil[1])


class Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status
        self.message = message


_u64p = ctypes.POINTER(ctypes.c_uint64)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p  # device addresses and streams are passed as plain ints (None for null)
_i64 = ctypes.c_int64

_lib.tbg_encode_tiled.restype = ctypes.c_int
_lib.tbg_encode_tiled.argtypes = [ctypes.POINTER(TensorDesc), ctypes.c_int, ctypes.c_uint32, _vp, _u64p, _u64p,
                                  _u32p, _u32p, ctypes.c_int, ctypes.c_int, ctypes.c_int]
_lib.tbg_encode_tiled_interleaved.restype = ctypes.c_int
_lib.tbg_encode_tiled_interleaved.argtypes = [ctypes.POINTER(TensorDesc), ctypes.c_int, ctypes.c_uint32, _vp, _u64p,
                                              _u64p, _u32p, _u32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int]
_lib.tbg_box_bytes.restype = ctypes.c_size_t
_lib.tbg_box_bytes.argtypes = [ctypes.POINTER(TensorDesc)]
_lib.tbg_tiled_copy.restype = ctypes.c_int
_lib.tbg_tiled_copy.argtypes = [ctypes.POINTER(TensorDesc), _i32p, _vp, _vp]
_lib.tbg_tiled_copy_many.restype = ctypes.c_int
_lib.tbg_tiled_copy_many.argtypes = [ctypes.POINTER(TensorDesc), _vp, ctypes.c_uint32, _vp, _vp]
_lib.tbg_gemm_workspace_bytes.restype = ctypes.c_size_t
_lib.tbg_tiled_store.restype = ctypes.c_int
_lib.tbg_tiled_store.argtypes = [ctypes.POINTER(TensorDesc), _i32p, _vp, _vp]
_lib.tbg_tiled_store_many.restype = ctypes.c_int
_lib.tbg_tiled_store_many.argtypes = [ctypes.POINTER(TensorDesc), _vp, ctypes.c_uint32, _vp, _vp]
_lib.tbg_gemm_ex.restype = ctypes.c_int
_lib.tbg_gemm_ex.argtypes = [_i64, _i64, _i64, ctypes.c_float, _vp, _i64, _vp, _i64, ctypes.c_int, ctypes.c_float, _vp,
                             _i64, ctypes.c_int, _vp, ctypes.c_size_t, _vp]
_lib.tbg_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int]
_lib.tbg_gemm.restype = ctypes.c_int
_lib.tbg_gemm.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, ctypes.c_int, _vp, _i64, ctypes.c_int, _vp,
                          ctypes.c_size_t, _vp]
_lib.tbg_gemm_configured.restype = ctypes.c_int
_lib.tbg_gemm_configured.argtypes = [_i64, _i64, _i64, ctypes.c_float, _vp, _i64, _vp, _i64, ctypes.c_int,
                                     ctypes.c_float, _vp, _i64, ctypes.c_int, ctypes.POINTER(GemmConfig), _vp,
                                     ctypes.c_size_t, _vp]
_lib.tbg_encode_im2col.restype = ctypes.c_int
_lib.tbg_encode_im2col.argtypes = [ctypes.POINTER(TensorDesc), ctypes.c_int, _vp, _u64p, _u64p, _i32p, _i32p, _i32p,
                                   _i32p, _i32p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int]
_lib.tbg_im2col_copy.restype = ctypes.c_int
_lib.tbg_im2col_copy.argtypes = [ctypes.POINTER(TensorDesc), _i32p, _vp, _vp]
_lib.tbg_im2col_copy_many.restype = ctypes.c_int
_lib.tbg_im2col_copy_many.argtypes = [ctypes.POINTER(TensorDesc), _vp, ctypes.c_uint32, _vp, _vp]
_lib.tbg_conv2d_out_dims.restype = ctypes.c_int
_lib.tbg_conv2d_out_dims.argtypes = [ctypes.POINTER(Conv2dShape), ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_int64)]
_lib.tbg_conv2d_workspace_bytes.restype = ctypes.c_size_t
_lib.tbg_conv2d_workspace_bytes.argtypes = [ctypes.POINTER(Conv2dShape)]
_lib.tbg_conv2d_workspace_query.restype = ctypes.c_size_t
_lib.tbg_conv2d_workspace_query.argtypes = [ctypes.POINTER(Conv2dShape), _vp, _vp]
_lib.tbg_gemm_noalloc.restype = ctypes.c_int
_lib.tbg_gemm_noalloc.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, ctypes.c_int, _vp, _i64, ctypes.c_int, _vp]
_lib.tbg_gemm_noalloc_scratch_bytes.restype = ctypes.c_size_t
_lib.tbg_gemm_noalloc_scratch_bytes.argtypes = []
_lib.tbg_gemm_workspace_query.restype = ctypes.c_size_t
_lib.tbg_gemm_workspace_query.argtypes = [_i64, _i64, _i64, ctypes.c_int, _vp, _i64, _vp, _i64, ctypes.c_int]
_lib.tbg_conv2d_fwd.restype = ctypes.c_int
_lib.tbg_conv2d_fwd.argtypes = [ctypes.POINTER(Conv2dShape), ctypes.c_float, _vp, _vp, ctypes.c_float, _vp, _i64,
                                ctypes.c_int, ctypes.POINTER(GemmConfig), _vp, ctypes.c_size_t, _vp]
_lib.tbg_gemm_typed.restype = ctypes.c_int
_lib.tbg_gemm_typed.argtypes = [_i64, _i64, _i64, ctypes.c_float, _vp, _i64, _vp, _i64, ctypes.c_int, ctypes.c_int,
                                ctypes.c_float, _vp, _i64, ctypes.c_int, ctypes.POINTER(GemmConfig), _vp,
                                ctypes.c_size_t, _vp]
_lib.tbg_status_string.restype = ctypes.c_char_p
_lib.tbg_status_string.argtypes = [ctypes.c_int]
_lib.tbg_last_error.restype = ctypes.c_char_p
_lib.tbg_last_error.argtypes = []


def status_string(status: int) -> str:
    return _lib.tbg_status_string(int(status)).decode()


def last_error() -> str:
    return _lib.tbg_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise Error(status, last_error())


def _enum(table, v):
    return table[v] if isinstance(v, str) else int(v)


def _arr(ctype, values):
    values = list(values)
    return (ctype * max(1, len(values)))(*values)


def encode_tiled(dtype, rank: int, global_address: int, global_dim: Sequence[int],
                 global_strides: Optional[Sequence[int]], box_dim: Sequence[int], element_strides: Sequence[int],
                 swizzle="none", l2="none", oob="zero") -> TensorDesc:
    """tbg_encode_tiled.  Per-dimension arrays innermost first; strides in bytes (rank-1)."""
    d = TensorDesc()
    strides = None if global_strides is None else _arr(ctypes.c_uint64, global_strides)
    st = _lib.tbg_encode_tiled(ctypes.byref(d), _enum(DTYPES, dtype), int(rank), int(global_address),
                               _arr(ctypes.c_uint64, global_dim), strides, _arr(ctypes.c_uint32, box_dim),
                               _arr(ctypes.c_uint32, element_strides), _enum(SWIZZLES, swizzle), _enum(L2, l2),
                               _enum(OOB, oob))
    _check(st)
    return d


def encode_tiled_interleaved(dtype, rank: int, global_address: int, global_dim: Sequence[int],
                             global_strides: Sequence[int], box_dim: Sequence[int], element_strides: Sequence[int],
                             interleave="16B", swizzle="none", l2="none", oob="zero") -> TensorDesc:
    """tbg_encode_tiled_interleaved: an NC/xHWCx tensor, dimension 0 one 16- or 32-byte slice."""
    d = TensorDesc()
    st = _lib.tbg_encode_tiled_interleaved(ctypes.byref(d), _enum(DTYPES, dtype), int(rank), int(global_address),
                                           _arr(ctypes.c_uint64, global_dim), _arr(ctypes.c_uint64, global_strides),
                                           _arr(ctypes.c_uint32, box_dim), _arr(ctypes.c_uint32, element_strides),
                                           _enum(INTERLEAVES, interleave), _enum(SWIZZLES, swizzle), _enum(L2, l2),
                                           _enum(OOB, oob))
    _check(st)
    return d


def encode_tiled_interleaved_status(*args, **kwargs) -> int:
    try:
        encode_tiled_interleaved(*args, **kwargs)
        return OK
    except Error as e:
        return e.status


def encode_tiled_status(*args, **kwargs) -> int:
    """Like encode_tiled but returns the status code instead of raising."""
    try:
        encode_tiled(*args, **kwargs)
        return OK
    except Error as e:
        return e.status


def box_bytes(desc: TensorDesc) -> int:
    return int(_lib.tbg_box_bytes(ctypes.byref(desc)))


def tiled_copy(desc: TensorDesc, coords: Sequence[int], dst_image: int, stream: Optional[int] = None) -> None:
    _check(_lib.tbg_tiled_copy(ctypes.byref(desc), _arr(ctypes.c_int32, coords), int(dst_image),
                               stream or None))


def tiled_copy_many(desc: TensorDesc, coords_dev: int, n: int, dst_images: int, stream: Optional[int] = None) -> None:
    _check(_lib.tbg_tiled_copy_many(ctypes.byref(desc), int(coords_dev), int(n), int(dst_images),
                                    stream or None))


def tiled_store(desc: TensorDesc, coords: Sequence[int], src_image: int, stream: Optional[int] = None) -> None:
    _check(_lib.tbg_tiled_store(ctypes.byref(desc), _arr(ctypes.c_int32, coords), int(src_image),
                                stream or None))


def tiled_store_many(desc: TensorDesc, coords_dev: int, n: int, src_images: int, stream: Optional[int] = None) -> None:
    _check(_lib.tbg_tiled_store_many(ctypes.byref(desc), int(coords_dev), int(n), int(src_images),
                                     stream or None))


def encode_im2col(dtype, global_address: int, global_dim: Sequence[int], global_strides: Sequence[int],
                  pad_lo: Sequence[int], pad_hi: Sequence[int], conv_stride: Sequence[int], dilation: Sequence[int],
                  filter: Sequence[int], channels: int, pixels: int, swizzle="none", l2="none",
                  oob="zero") -> TensorDesc:
    """tbg_encode_im2col.  dims {C, W, H, N}; strides {W, H, N} in bytes; per-spatial arrays
    {along W, along H}."""
    d = TensorDesc()
    st = _lib.tbg_encode_im2col(ctypes.byref(d), _enum(DTYPES, dtype), int(global_address),
                                _arr(ctypes.c_uint64, global_dim), _arr(ctypes.c_uint64, global_strides),
                                _arr(ctypes.c_int32, pad_lo), _arr(ctypes.c_int32, pad_hi),
                                _arr(ctypes.c_int32, conv_stride), _arr(ctypes.c_int32, dilation),
                                _arr(ctypes.c_int32, filter), int(channels), int(pixels), _enum(SWIZZLES, swizzle),
                                _enum(L2, l2), _enum(OOB, oob))
    _check(st)
    return d


def encode_im2col_status(*args, **kwargs) -> int:
    try:
        encode_im2col(*args, **kwargs)
        return OK
    except Error as e:
        return e.status


def im2col_copy(desc: TensorDesc, coords: Sequence[int], dst_image: int, stream: Optional[int] = None) -> None:
    """tbg_im2col_copy: coords = {c0, m0, s, r}."""
    _check(_lib.tbg_im2col_copy(ctypes.byref(desc), _arr(ctypes.c_int32, coords), int(dst_image),
                                stream or None))


def im2col_copy_many(desc: TensorDesc, coords_dev: int, n: int, dst_images: int, stream: Optional[int] = None) -> None:
    _check(_lib.tbg_im2col_copy_many(ctypes.byref(desc), int(coords_dev), int(n), int(dst_images),
                                     stream or None))


def conv2d_out_dims(shape: Conv2dShape):
    oh, ow = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.tbg_conv2d_out_dims(ctypes.byref(shape), ctypes.byref(oh), ctypes.byref(ow)))
    return oh.value, ow.value


def conv2d_workspace_bytes(shape: Conv2dShape) -> int:
    return int(_lib.tbg_conv2d_workspace_bytes(ctypes.byref(shape)))


def conv2d_workspace_query(shape: Conv2dShape, x: int, w: int) -> int:
    return int(_lib.tbg_conv2d_workspace_query(ctypes.byref(shape), int(x), int(w)))


def conv2d_fwd(shape: Conv2dShape, alpha: float, x: int, w: int, beta: float, y: int, ldy: int, y_dtype,
               config: Optional[GemmConfig] = None, workspace: int = 0, workspace_bytes: int = 0,
               stream: Optional[int] = None) -> None:
    """tbg_conv2d_fwd: Y <- alpha·conv2d(X, W) + beta·Y (X NHWC, W KRSC, Y (N·OH·OW) × K)."""
    cfg = ctypes.byref(config) if config is not None else None
    _check(_lib.tbg_conv2d_fwd(ctypes.byref(shape), float(alpha), int(x), int(w), float(beta), int(y),
                               int(ldy), _enum(DTYPES, y_dtype), cfg, int(workspace), int(workspace_bytes),
                               stream or None))


def conv2d_fwd_status(*args, **kwargs) -> int:
    try:
        conv2d_fwd(*args, **kwargs)
        return OK
    except Error as e:
        return e.status


def gemm_workspace_bytes(M: int, N: int, K: int, lda: int, ldb: int, b_layout="kn") -> int:
    return int(_lib.tbg_gemm_workspace_bytes(M, N, K, lda, ldb, _enum(B_LAYOUTS, b_layout)))


def gemm_workspace_query(M: int, N: int, K: int, ab_dtype, A: int, lda: int, B: int, ldb: int, b_layout="kn") -> int:
    return int(_lib.tbg_gemm_workspace_query(M, N, K, _enum(DTYPES, ab_dtype), int(A), lda, int(B), ldb,
                                             _enum(B_LAYOUTS, b_layout)))


def gemm(M: int, N: int, K: int, A: int, lda: int, B: int, ldb: int, b_layout, C: int, ldc: int, c_dtype,
         workspace: int = 0, workspace_bytes: int = 0, stream: Optional[int] = None) -> None:
    """tbg_gemm: C = A·B (bf16 in, fp32 accumulate, fp32 or bf16 out) on `stream`."""
    _check(_lib.tbg_gemm(M, N, K, int(A), lda, int(B), ldb, _enum(B_LAYOUTS, b_layout), int(C), ldc,
                         _enum(DTYPES, c_dtype), int(workspace), int(workspace_bytes), stream or None))


def gemm_noalloc(M: int, N: int, K: int, A: int, lda: int, B: int, ldb: int, b_layout, C: int, ldc: int, c_dtype,
                 stream: Optional[int] = None) -> None:
    """tbg_gemm_noalloc: tbg_gemm with any repack in the library's own scratch array (no workspace)."""
    _check(_lib.tbg_gemm_noalloc(M, N, K, int(A), lda, int(B), ldb, _enum(B_LAYOUTS, b_layout), int(C),
                                 ldc, _enum(DTYPES, c_dtype), stream or None))


def gemm_noalloc_scratch_bytes() -> int:
    return int(_lib.tbg_gemm_noalloc_scratch_bytes())


def gemm_ex(M: int, N: int, K: int, alpha: float, A: int, lda: int, B: int, ldb: int, b_layout, beta: float, C: int,
            ldc: int, c_dtype, workspace: int = 0, workspace_bytes: int = 0, stream: Optional[int] = None) -> None:
    """tbg_gemm_ex: C = alpha·A·B + beta·C on `stream`."""
    _check(_lib.tbg_gemm_ex(M, N, K, float(alpha), int(A), lda, int(B), ldb, _enum(B_LAYOUTS, b_layout),
                            float(beta), int(C), ldc, _enum(DTYPES, c_dtype), int(workspace),
                            int(workspace_bytes), stream or None))


def gemm_configured(M: int, N: int, K: int, alpha: float, A: int, lda: int, B: int, ldb: int, b_layout, beta: float,
                    C: int, ldc: int, c_dtype, config: Optional[GemmConfig], workspace: int = 0,
                    workspace_bytes: int = 0, stream: Optional[int] = None) -> None:
    """tbg_gemm_configured: C = alpha·A·B + beta·C with an explicit kernel configuration."""
    cfg = ctypes.byref(config) if config is not None else None
    _check(_lib.tbg_gemm_configured(M, N, K, float(alpha), int(A), lda, int(B), ldb,
                                    _enum(B_LAYOUTS, b_layout), float(beta), int(C), ldc, _enum(DTYPES, c_dtype),
                                    cfg, int(workspace), int(workspace_bytes), stream or None))


def gemm_typed(M: int, N: int, K: int, alpha: float, A: int, lda: int, B: int, ldb: int, b_layout, ab_dtype,
               beta: float, C: int, ldc: int, c_dtype, config: Optional[GemmConfig] = None, workspace: int = 0,
               workspace_bytes: int = 0, stream: Optional[int] = None) -> None:
    """tbg_gemm_typed: C = alpha·A·B + beta·C with A, B of type ab_dtype ("bf16" or "f16")."""
    cfg = ctypes.byref(config) if config is not None else None
    _check(_lib.tbg_gemm_typed(M, N, K, float(alpha), int(A), lda, int(B), ldb, _enum(B_LAYOUTS, b_layout),
                               _enum(DTYPES, ab_dtype), float(beta), int(C), ldc, _enum(DTYPES, c_dtype), cfg,
                               int(workspace), int(workspace_bytes), stream or None))


def gemm_typed_status(*args, **kwargs) -> int:
    try:
        gemm_typed(*args, **kwargs)
        return OK
    except Error as e:
        return e.status


def gemm_configured_status(*args, **kwargs) -> int:
    """Like gemm_configured but returns the status code instead of raising."""
    try:
        gemm_configured(*args, **kwargs)
        return OK
    except Error as e:
        return e.status


def gemm_status(*args, **kwargs) -> int:
    """Like gemm but returns the status code instead of raising."""
    try:
        gemm(*args, **kwargs)
        return OK
    except Error as e:
        return e.status


def declared_functions() -> list:
    """Names of the functions include/tbg.h declares (used to check the library's exports)."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tbg_[a-z0-9_]+)\s*\(", text)))


def library_path() -> str:
    return LIB_PATH
