"""Race check of the stage hand-offs ("1 · Asynchronisme et mbarrier" §1.5: a stage may be read
only once its copies have landed, and refilled only once every reader is done with it).

The lean kernels wait at each hand-off for exactly the copies the next stage needs and leave
later tiles in flight (the ring's `s_waitcnt vmcnt(N)` before its barrier, the producers'
partial waits, unmasked interior iterations, copy atoms interleaved with the products).  The
library is also built with TBG_HANDOFF_CHECK=1 (tiled_bf16_gemm_amd/diag/libtbg_check.so, the
same C ABI), where every hand-off drains all of the wave's copies and LDS reads first.  A
schedule that let a wave read a stage before its data landed, or overwrite a stage another wave
still read, gives different bits from the drained build; these tests require identical bits on
every configuration of the barrier ring, the producer/consumer ring, the fp8 ring, the
convolution ring and the halo convolution."""
import ctypes
import os

import numpy as np
import pytest
import torch

import workloads
from tests.test_gpu_gemm import CONFIG_CASES, CONFIGS, _say, gpu

CHECK_LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tiled_bf16_gemm_amd", "diag",
                         "libtbg_check.so")


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_bf16_gemm_amd as tbg
    check = ctypes.CDLL(CHECK_LIB)
    vp, i64, ci, cf = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    for lib in (check,):
        lib.tbg_gemm_typed.restype = ci
        lib.tbg_gemm_typed.argtypes = [i64, i64, i64, cf, vp, i64, vp, i64, ci, ci, cf, vp, i64, ci,
                                       ctypes.POINTER(tbg.GemmConfig), vp, ctypes.c_size_t, vp]
        lib.tbg_conv2d_fwd.restype = ci
        lib.tbg_conv2d_fwd.argtypes = [ctypes.POINTER(tbg.Conv2dShape), cf, vp, vp, cf, vp, i64, ci,
                                       ctypes.POINTER(tbg.GemmConfig), vp, ctypes.c_size_t, vp]
        lib.tbg_last_error.restype = ctypes.c_char_p
    return tbg, check


def _typed(tbg, lib, M, N, K, A, lda, B, ldb, bl, ab, C, ldc, out, cfg, ws):
    """One product through the given library's tbg_gemm_typed (the product library through the
    binding, the checking build through its own handle)."""
    stream = torch.cuda.current_stream().cuda_stream
    if lib is None:
        tbg.gemm_typed(M, N, K, 1.0, A.data_ptr(), lda, B.data_ptr(), ldb, bl, ab, 0.0, C.data_ptr(), ldc, out, cfg,
                       ws.data_ptr(), ws.numel(), stream)
        return
    st = lib.tbg_gemm_typed(M, N, K, 1.0, A.data_ptr(), lda, B.data_ptr(), ldb, tbg.B_LAYOUTS[bl], tbg.DTYPES[ab],
                            0.0, C.data_ptr(), ldc, tbg.DTYPES[out], ctypes.byref(cfg) if cfg is not None else None,
                            ws.data_ptr(), ws.numel(), stream)
    assert st == 0, lib.tbg_last_error().decode()


def _same(a: torch.Tensor, b: torch.Tensor, what: str):
    ai = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    bi = b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    bad = int((ai != bi).sum())
    assert bad == 0, f"{what}: {bad} entries differ between the lean and the drained hand-offs"


@gpu
@pytest.mark.parametrize("pipeline,tile,stages", CONFIGS)
def test_handoffs_match_the_drained_build(libs, pipeline, tile, stages):
    tbg, check = libs
    cfg = tbg.gemm_config(tile, stages, pipeline)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for i, (M, N, K, bl, out) in enumerate(CONFIG_CASES):
        A = workloads.matrix(M, K, K, ("normal", 1.0), 800 + i).cuda()
        B = (workloads.matrix(K, N, N, ("normal", 1.0), 900 + i) if bl == "kn" else
             workloads.matrix(N, K, K, ("normal", 1.0), 900 + i)).cuda()
        tdt = torch.float32 if out == "f32" else torch.bfloat16
        ldc = N + 3
        got = [torch.full((M, ldc), float("nan"), dtype=tdt, device="cuda") for _ in range(2)]
        _say(f"{pipeline} {tile}/{stages}: M={M} N={N} K={K} {bl} {out}, lean and drained")
        for lib, C in zip((None, check), got):
            _typed(tbg, lib, M, N, K, A, K, B, B.shape[1], bl, "bf16", C, ldc, out, cfg, ws)
        torch.cuda.synchronize()
        _same(got[0], got[1], f"{pipeline} {tile}/{stages} case {i}")


@gpu
def test_fp8_and_convolution_handoffs(libs):
    tbg, check = libs
    ws = torch.empty(4 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    M, N, K = 700, 520, 1000
    g = torch.Generator().manual_seed(4711)
    A8 = torch.randn((M, K), generator=g).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
    B8 = torch.randn((N, K), generator=g).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
    for tile in ("256x256", "128x128", "64x64"):
        cfg = tbg.gemm_config(tile, 2, "ring")
        got = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for _ in range(2)]
        _say(f"fp8 {tile}: lean and drained")
        for lib, C in zip((None, check), got):
            _typed(tbg, lib, M, N, K, A8, K, B8, K, "nk", "f8e4m3", C, N, "f32", cfg, ws)
        torch.cuda.synchronize()
        _same(got[0], got[1], f"fp8 {tile}")
    w = workloads.CONVS["conv_3x3"]
    x, f = workloads.conv_inputs(w)
    x, f = x.cuda(), f.cuda()
    shp = tbg.conv2d_shape(w.n, w.h, w.w, w.c, w.k, w.r, w.s, w.pad, w.stride, w.dil)
    for tile in ("256x256", "256x128", "128x128", "64x64"):
        cfg = tbg.gemm_config(tile, 2, "ring")
        got = [torch.full((w.M, w.k), float("nan"), dtype=torch.float32, device="cuda") for _ in range(2)]
        _say(f"conv {tile}: lean and drained")
        tbg.conv2d_fwd(shp, 1.0, x.data_ptr(), f.data_ptr(), 0.0, got[0].data_ptr(), w.k, "f32", cfg, ws.data_ptr(),
                       ws.numel(), stream)
        st = check.tbg_conv2d_fwd(ctypes.byref(shp), 1.0, x.data_ptr(), f.data_ptr(), 0.0, got[1].data_ptr(), w.k,
                                  tbg.DTYPES["f32"], ctypes.byref(cfg), ws.data_ptr(), ws.numel(), stream)
        assert st == 0, check.tbg_last_error().decode()
        torch.cuda.synchronize()
        _same(got[0], got[1], f"conv {tile}")
    # the halo kernel: its filter ring and its two window images (atoms per wave and tap 1..4)
    for name in ("conv_halo_rows", "conv_halo_wide", "conv_halo_small", "conv_halo_1x3", "conv_halo_c96",
                 "conv_halo_808", "conv_halo_max"):
        w = workloads.CONVS[name]
        x, f = workloads.conv_inputs(w)
        x, f = x.cuda(), f.cuda()
        shp = tbg.conv2d_shape(w.n, w.h, w.w, w.c, w.k, w.r, w.s, w.pad, w.stride, w.dil)
        cfg = tbg.gemm_config("448x128", 0, "ring")
        got = [torch.full((w.M, w.k), float("nan"), dtype=torch.float32, device="cuda") for _ in range(2)]
        _say(f"halo conv {name}: lean and drained")
        tbg.conv2d_fwd(shp, 1.0, x.data_ptr(), f.data_ptr(), 0.0, got[0].data_ptr(), w.k, "f32", cfg, ws.data_ptr(),
                       ws.numel(), stream)
        st = check.tbg_conv2d_fwd(ctypes.byref(shp), 1.0, x.data_ptr(), f.data_ptr(), 0.0, got[1].data_ptr(), w.k,
                                  tbg.DTYPES["f32"], ctypes.byref(cfg), ws.data_ptr(), ws.numel(), stream)
        assert st == 0, check.tbg_last_error().decode()
        torch.cuda.synchronize()
        _same(got[0], got[1], f"halo conv {name}")
