"""tbg_gemm_noalloc, the product for callers that cannot allocate: through the C ABI, against
tbg_gemm with a caller workspace (the same kernels, so the same bits) and the oracle, on two calls
in a row, the second smaller than the first; the repack runs in the library's scratch array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads

gpu = pytest.mark.gpu


def _lib():
    import tiled_bf16_gemm_amd as tbg
    lib = ctypes.CDLL(tbg.library_path())
    lib.tbg_gemm_noalloc.restype = ctypes.c_int
    lib.tbg_gemm_noalloc.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_void_p]
    lib.tbg_gemm_noalloc_scratch_bytes.restype = ctypes.c_size_t
    return lib


def _ragged(M, N, K, lda, ldb, bl, seed, a_off=0):
    """bf16 operands at pitches that force the repack (and an A that starts off a 16-byte boundary
    when a_off is odd), as flat device buffers with NaN past every row."""
    A = workloads.matrix(M, K, lda, ("normal", 1.0), seed)
    B = workloads.matrix(K, N, ldb, ("normal", 1.0), seed + 1) if bl == "kn" else \
        workloads.matrix(N, K, ldb, ("normal", 1.0), seed + 1)
    Ad = torch.empty(A.numel() + 16, dtype=torch.bfloat16, device="cuda")
    Ad[a_off:a_off + A.numel()] = A.reshape(-1).cuda()
    return A, B, Ad[a_off:], B.cuda()


@gpu
def test_noalloc_matches_the_workspace_product():
    import tiled_bf16_gemm_amd as tbg
    lib = _lib()
    orc = oracle.get()
    assert lib.tbg_gemm_noalloc_scratch_bytes() == 32 << 20
    stream = torch.cuda.current_stream().cuda_stream
    cases = [(3001, 2049, 777, 777, 2049, "kn", "f32", 0), (300, 257, 136, 137, 259, "nk", "bf16", 1)]
    for i, (M, N, K, lda, ldb, bl, out, a_off) in enumerate(cases):
        A, B, Ad, Bd = _ragged(M, N, K, lda, ldb, bl, 9100 + 10 * i, a_off)
        need = tbg.gemm_workspace_query(M, N, K, "bf16", Ad.data_ptr(), lda, Bd.data_ptr(), ldb, bl)
        assert 0 < need <= 32 << 20
        tdt = torch.float32 if out == "f32" else torch.bfloat16
        ldc = N + 3
        C_ws = torch.full((M, ldc), float("nan"), dtype=tdt, device="cuda")
        C_na = torch.full((M, ldc), float("nan"), dtype=tdt, device="cuda")
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        print(f"call {i}: M={M} N={N} K={K} lda={lda} ldb={ldb} {bl} {out}, repack {need} bytes", flush=True)
        tbg.gemm(M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, bl, C_ws.data_ptr(), ldc, out, ws.data_ptr(), need,
                 stream)
        st = lib.tbg_gemm_noalloc(M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, 0 if bl == "kn" else 1,
                                  C_na.data_ptr(), ldc, 5 if out == "f32" else 4, stream)
        assert st == 0, tbg.last_error()
        torch.cuda.synchronize()
        a, b = C_ws.float().cpu().numpy(), C_na.float().cpu().numpy()
        assert np.array_equal(a, b, equal_nan=True), f"call {i}: {int((a != b).sum())} entries differ from tbg_gemm"
        assert np.all(np.isnan(b[:, N:])), "columns past N were written"
        ref = orc.gemm(workloads.bits(A), workloads.bits(B), M, N, K, lda, ldb, bl)
        r = oracle.gemm_check(b[:, :N], ref)
        assert r["pass"], r


@gpu
def test_noalloc_refuses_what_does_not_fit():
    import tiled_bf16_gemm_amd as tbg
    lib = _lib()
    # a repack of 2 * 8191 * 8200 * 2 bytes > 32 MiB: refused on the host, nothing launched
    st = lib.tbg_gemm_noalloc(8191, 8191, 8191, 0x7F0000000000, 8191, 0x7F0000000000, 8191, 0, 0x7F0000000000, 8191,
                              5, None)
    assert st == tbg.ERR_OUT_OF_RANGE and "allocation-free" in tbg.last_error()


@gpu
def test_noalloc_under_graph_capture():
    """The allocation-free product captured into a HIP graph (torch.cuda.graph) on operands that
    need the repack, replayed three times with eager work (and an eager call of the same entry
    point on other operands, which overwrites the scratch array) between the replays: every replay
    equals the eager result bit for bit."""
    lib = _lib()
    M, N, K, lda, ldb = 300, 257, 777, 777, 257
    _, _, Ad, Bd = _ragged(M, N, K, lda, ldb, "kn", 9300)
    _, _, Ad2, Bd2 = _ragged(200, 130, 100, 101, 131, "kn", 9400)

    def call(A, B, C, m, n, k, la, lb, stream):
        st = lib.tbg_gemm_noalloc(m, n, k, A.data_ptr(), la, B.data_ptr(), lb, 0, C.data_ptr(), n, 5, stream)
        assert st == 0

    eager = torch.empty((M, N), dtype=torch.float32, device="cuda")
    call(Ad, Bd, eager, M, N, K, lda, ldb, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    other = torch.empty((200, 130), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm-up on the capture stream
        call(Ad, Bd, out, M, N, K, lda, ldb, stream.cuda_stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call(Ad, Bd, out, M, N, K, lda, ldb, stream.cuda_stream)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"noalloc graph replay {rep}", flush=True)
        assert torch.equal(out, eager), f"replay {rep} differs from the eager result"
        call(Ad2, Bd2, other, 200, 130, 100, 101, 131, torch.cuda.current_stream().cuda_stream)
        x = torch.randn(512, 512, device="cuda") @ torch.randn(512, 512, device="cuda")
        torch.cuda.synchronize()
        del x
    del g
