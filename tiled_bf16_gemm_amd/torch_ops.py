"""Torch-facing helpers over the C ABI: device memory and streams come from PyTorch, every step
of the computation runs in the library's kernels.  Marshalling only."""
from __future__ import annotations

from typing import Optional, Sequence

import torch

import tiled_bf16_gemm_amd as tbg

_AB_OF = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float8_e4m3fn: "f8e4m3", torch.float8_e5m2: "f8e5m2"}
_TORCH_OF = {"u8": torch.uint8, "u16": torch.int16, "u32": torch.int32, "f16": torch.float16,
             "bf16": torch.bfloat16, "f32": torch.float32}


def stream_handle(stream: Optional[torch.cuda.Stream] = None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _require(t: torch.Tensor, name: str, device: Optional[torch.device] = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major view (unit inner stride)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, A on {device}: every operand must be on one device")


# tbg_gemm_workspace_query's answers.  The query reads the sizes, the operand type and layout, the
# leading dimensions and only the operands' addresses modulo 16 (their 16-byte alignment), so
# that is the key; the table is cleared when it grows past a few thousand shapes.
_WS_NEED: dict = {}


def _gemm_workspace_need(M, N, K, ab, a_ptr, lda, b_ptr, ldb, b_layout) -> int:
    key = (M, N, K, ab, a_ptr & 15, lda, b_ptr & 15, ldb, b_layout)
    need = _WS_NEED.get(key)
    if need is None:
        if len(_WS_NEED) > 4096:
            _WS_NEED.clear()
        need = _WS_NEED[key] = tbg.gemm_workspace_query(M, N, K, ab, a_ptr, lda, b_ptr, ldb, b_layout)
    return need


def _require_workspace(ws: Optional[torch.Tensor], device: torch.device):
    if ws is not None and (not ws.is_cuda or ws.device != device or not ws.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous CUDA tensor on {device}")


def gemm(A: torch.Tensor, B: torch.Tensor, b_layout: str = "kn", out_dtype: str = "bf16",
         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
         stream: Optional[torch.cuda.Stream] = None, alpha: float = 1.0, beta: float = 0.0,
         config: Optional[tbg.GemmConfig] = None) -> torch.Tensor:
    """C = alpha·A·B + beta·C through tbg_gemm (alpha = 1, beta = 0), tbg_gemm_ex, or
    tbg_gemm_configured when `config` (tbg.gemm_config(...)) is given; fp16 and 8-bit float
    operands (float8_e4m3fn, float8_e5m2; B stored "nk" only) go through tbg_gemm_typed.
    A: (M, K) view; B: (K, N) for "kn" or (N, K) for "nk".  Row strides become the leading
    dimensions.  `out` (M, N) may be a strided view; with beta != 0 it must hold the old C."""
    _require(A, "A")
    _require(B, "B", A.device)
    ab = _AB_OF.get(A.dtype)
    if ab is None or B.dtype != A.dtype:
        raise ValueError("A and B must have the same dtype: bfloat16, float16, float8_e4m3fn or float8_e5m2")
    M, K = A.shape
    if b_layout == "kn":
        Kb, N = B.shape
    else:
        N, Kb = B.shape
    if Kb != K:
        raise ValueError(f"inner sizes differ: {K} vs {Kb}")
    if out_dtype not in ("f32", "bf16"):
        raise ValueError(f"out_dtype must be 'f32' or 'bf16' (got {out_dtype!r})")
    if out is None:
        out = torch.empty((M, N), dtype=_TORCH_OF[out_dtype], device=A.device)
    _require(out, "out", A.device)
    # the kernel writes M rows of N elements of out_dtype at out's row stride: out must be exactly that
    if tuple(out.shape) != (M, N) or out.dtype != _TORCH_OF[out_dtype]:
        raise ValueError(f"out must be a ({M}, {N}) {_TORCH_OF[out_dtype]} view (got {tuple(out.shape)} {out.dtype})")
    _require_workspace(workspace, A.device)
    lda, ldb, ldc = A.stride(0), B.stride(0), out.stride(0)
    a_ptr, b_ptr, c_ptr = A.data_ptr(), B.data_ptr(), out.data_ptr()
    need = _gemm_workspace_need(M, N, K, ab, a_ptr, lda, b_ptr, ldb, b_layout)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if need and ws_bytes < need:
        # twice the need: successive calls alternate the halves their repacks land in
        workspace = torch.empty(2 * need, dtype=torch.uint8, device=A.device)
        ws_bytes = 2 * need
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    s = stream_handle(stream)
    if ab != "bf16":
        tbg.gemm_typed(M, N, K, alpha, a_ptr, lda, b_ptr, ldb, b_layout, ab, beta, c_ptr, ldc, out_dtype, config,
                       ws_ptr, ws_bytes, s)
    elif config is not None:
        tbg.gemm_configured(M, N, K, alpha, a_ptr, lda, b_ptr, ldb, b_layout, beta, c_ptr, ldc, out_dtype, config,
                            ws_ptr, ws_bytes, s)
    elif alpha == 1.0 and beta == 0.0:
        tbg.gemm(M, N, K, a_ptr, lda, b_ptr, ldb, b_layout, c_ptr, ldc, out_dtype, ws_ptr, ws_bytes, s)
    else:
        tbg.gemm_ex(M, N, K, alpha, a_ptr, lda, b_ptr, ldb, b_layout, beta, c_ptr, ldc, out_dtype, ws_ptr, ws_bytes, s)
    return out


def encode(t: torch.Tensor, dtype: str, dims: Sequence[int], strides_bytes: Sequence[int], box: Sequence[int],
           estr: Sequence[int], swizzle: str = "none", oob: str = "zero", l2: str = "none") -> tbg.TensorDesc:
    """Descriptor for the tensor whose element (0, ..., 0) is t's first element."""
    return tbg.encode_tiled(dtype, len(dims), t.data_ptr(), dims, list(strides_bytes), box, estr, swizzle, l2, oob)


def tiled_copy(desc: tbg.TensorDesc, coords: Sequence[int], out: Optional[torch.Tensor] = None,
               device="cuda", stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    nbytes = tbg.box_bytes(desc)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=device)
    tbg.tiled_copy(desc, coords, out.data_ptr(), stream_handle(stream))
    return out


def tiled_copy_many(desc: tbg.TensorDesc, coords: torch.Tensor, out: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """coords: (n, rank) int32 CUDA tensor.  Returns n images of box_bytes each (uint8, flat)."""
    if coords.dtype != torch.int32 or not coords.is_cuda or not coords.is_contiguous():
        raise ValueError("coords must be a contiguous int32 CUDA tensor")
    n = coords.shape[0]
    nbytes = tbg.box_bytes(desc)
    if out is None:
        out = torch.empty(n * nbytes, dtype=torch.uint8, device=coords.device)
    tbg.tiled_copy_many(desc, coords.data_ptr(), n, out.data_ptr(), stream_handle(stream))
    return out


def tiled_store(desc: tbg.TensorDesc, coords: Sequence[int], image: torch.Tensor,
                stream: Optional[torch.cuda.Stream] = None) -> None:
    """Store one box image (a CUDA tensor of box_bytes bytes) into the descriptor's tensor."""
    if not image.is_cuda or image.numel() * image.element_size() < tbg.box_bytes(desc):
        raise ValueError("image must be a CUDA tensor of at least box_bytes bytes")
    tbg.tiled_store(desc, coords, image.data_ptr(), stream_handle(stream))


def tiled_store_many(desc: tbg.TensorDesc, coords: torch.Tensor, images: torch.Tensor,
                     stream: Optional[torch.cuda.Stream] = None) -> None:
    """coords: (n, rank) int32 CUDA tensor; images: n images of box_bytes each, back to back."""
    if coords.dtype != torch.int32 or not coords.is_cuda or not coords.is_contiguous():
        raise ValueError("coords must be a contiguous int32 CUDA tensor")
    n = coords.shape[0]
    if images.numel() * images.element_size() < n * tbg.box_bytes(desc):
        raise ValueError("images holds fewer than n box images")
    tbg.tiled_store_many(desc, coords.data_ptr(), n, images.data_ptr(), stream_handle(stream))


def conv2d(x: torch.Tensor, w: torch.Tensor, pad=(0, 0, 0, 0), stride=(1, 1), dil=(1, 1), out_dtype: str = "bf16",
           out: Optional[torch.Tensor] = None, alpha: float = 1.0, beta: float = 0.0,
           workspace: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None,
           config: Optional[tbg.GemmConfig] = None) -> torch.Tensor:
    """Y = alpha·conv2d(x, w) + beta·Y through tbg_conv2d_fwd.  x: (N, H, W, C) bf16 contiguous
    (NHWC); w: (K, R, S, C) bf16 contiguous (KRSC); pad = (top, left, bottom, right); stride and
    dil = (h, w).  Returns / fills out: (N·OH·OW, K) rows, row stride = ldy."""
    for t, name in ((x, "x"), (w, "w")):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 CUDA tensor")
    n, h, wd, c = x.shape
    k, r, s, c2 = w.shape
    if c2 != c:
        raise ValueError(f"channel counts differ: {c} vs {c2}")
    shp = tbg.conv2d_shape(n, h, wd, c, k, r, s, pad, stride, dil)
    oh, ow = tbg.conv2d_out_dims(shp)
    if out is None:
        out = torch.empty((n * oh * ow, k), dtype=_TORCH_OF[out_dtype], device=x.device)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != n * oh * ow or out.shape[1] != k:
        raise ValueError("out must be a (N·OH·OW, K) row-major view")
    if w.device != x.device or out.device != x.device:
        raise ValueError("x, w and out must be on one device")
    if out.dtype != _TORCH_OF[out_dtype]:
        raise ValueError(f"out must hold {_TORCH_OF[out_dtype]} for out_dtype {out_dtype!r} (got {out.dtype})")
    _require_workspace(workspace, x.device)
    need = tbg.conv2d_workspace_query(shp, x.data_ptr(), w.data_ptr())
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(2 * need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    tbg.conv2d_fwd(shp, alpha, x.data_ptr(), w.data_ptr(), beta, out.data_ptr(), out.stride(0), out_dtype, config,
                   ws_ptr, ws_bytes, stream_handle(stream))
    return out


def encode_im2col(t: torch.Tensor, dtype: str, pad=(0, 0, 0, 0), stride=(1, 1), dil=(1, 1), filt=(1, 1),
                  channels: int = 64, pixels: int = 64, swizzle: str = "none", oob: str = "zero") -> tbg.TensorDesc:
    """im2col descriptor of a contiguous NHWC tensor t; pad = (top, left, bottom, right), stride,
    dil and filt = (h, w)."""
    n, h, w, c = t.shape
    es = t.element_size()
    return tbg.encode_im2col(dtype, t.data_ptr(), [c, w, h, n], [c * es, c * es * w, c * es * w * h],
                             [pad[1], pad[0]], [pad[3], pad[2]], [stride[1], stride[0]], [dil[1], dil[0]],
                             [filt[1], filt[0]], channels, pixels, swizzle, "none", oob)


def im2col_copy(desc: tbg.TensorDesc, coords, out: Optional[torch.Tensor] = None, device="cuda",
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    nbytes = tbg.box_bytes(desc)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=device)
    tbg.im2col_copy(desc, coords, out.data_ptr(), stream_handle(stream))
    return out


def im2col_copy_many(desc: tbg.TensorDesc, coords: torch.Tensor, out: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """coords: (n, 4) int32 CUDA tensor of {c0, m0, s, r}.  Returns n images back to back."""
    if coords.dtype != torch.int32 or not coords.is_cuda or not coords.is_contiguous() or coords.shape[1] != 4:
        raise ValueError("coords must be a contiguous (n, 4) int32 CUDA tensor")
    n = coords.shape[0]
    nbytes = tbg.box_bytes(desc)
    if out is None:
        out = torch.empty(n * nbytes, dtype=torch.uint8, device=coords.device)
    tbg.im2col_copy_many(desc, coords.data_ptr(), n, out.data_ptr(), stream_handle(stream))
    return out
