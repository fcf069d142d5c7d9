"""The GEMM on the GPU against the oracle ("GEMM: la moltiplicazione di matrici sull'hardware").

Bar: every output finite and within max(1e-2·|r|, 1e-3) of the oracle's binary32 result r; bit
for bit where the inputs are small integers (every partial sum is then exact in binary32, so any
summation order gives the same bits).  The workload sizes that the oracle finishes in seconds
are compared in full; the 8192³ and 16384×14336×4096 workloads — in the launch configuration the
benchmark times — are compared on sampled whole rows and scattered points, and checked for
finiteness and run-to-run determinism everywhere; with integer operands whose product the output
type holds exactly, every entry of those two products is checked through Freivalds' identities
(C·x and yᵀ·C against A·(B·x) and (yᵀ·A)·B, exact in binary64)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

gpu = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tiled_bf16_gemm_amd import torch_ops
    return torch_ops


def _run(ops, A_cpu, B_cpu, M, N, K, b_layout, out_dtype, ldc=None, a_offset=0, b_offset=0, config=None):
    """A_cpu/B_cpu: row-major buffers (rows × ld).  Offsets shift the operands' start by whole
    elements inside a larger device buffer (to test bases off a 16-byte boundary)."""
    lda, ldb = A_cpu.shape[1], B_cpu.shape[1]
    Ad = torch.empty(A_cpu.numel() + 8, dtype=torch.bfloat16, device="cuda")
    Bd = torch.empty(B_cpu.numel() + 8, dtype=torch.bfloat16, device="cuda")
    Ad[a_offset:a_offset + A_cpu.numel()] = A_cpu.reshape(-1).cuda()
    Bd[b_offset:b_offset + B_cpu.numel()] = B_cpu.reshape(-1).cuda()
    A = Ad[a_offset:a_offset + A_cpu.numel()].view(A_cpu.shape)[:, :K]
    B = Bd[b_offset:b_offset + B_cpu.numel()].view(B_cpu.shape)
    B = B[:, :N] if b_layout == "kn" else B[:, :K]
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    ldc = ldc or N
    Cbuf = torch.full((M, ldc), float("nan"), dtype=tdt, device="cuda")
    C = Cbuf[:, :N]
    ops.gemm(A, B, b_layout, out_dtype, out=C, config=config)
    torch.cuda.synchronize()
    return Cbuf


def _to_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def _check(got: np.ndarray, ref: np.ndarray, what: str):
    r = oracle.gemm_check(got, ref)
    _say(f"  {what}: n={r['n']} max_abs={r['max_abs_err']:.3g} max_rel={r['max_rel_err']:.3g} fail={r['n_fail']}")
    assert r["pass"], f"{what}: {r}"


def _full_case(ops, orc, w: workloads.GemmWorkload):
    A, B = workloads.gemm_inputs(w)
    lda, ldb, ldc = w.lds()
    _say(f"gemm {w.name}: M={w.M} N={w.N} K={w.K} {w.b_layout} {w.out_dtype} lda={lda} ldb={ldb} ldc={ldc}")
    Cbuf = _run(ops, A, B, w.M, w.N, w.K, w.b_layout, w.out_dtype, ldc=ldc)
    ref = orc.gemm(workloads.bits(A), workloads.bits(B), w.M, w.N, w.K, lda, ldb, w.b_layout)
    got = _to_f32(Cbuf)
    _check(got[:, :w.N], ref, w.name)
    if ldc > w.N:
        assert np.all(np.isnan(got[:, w.N:])), "columns past N were written"
    return got[:, :w.N], ref


@gpu
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c3_bf16", "c3_padded"])
def test_workloads_full(ops, orc, name):
    got, ref = _full_case(ops, orc, workloads.GEMMS[name])
    if workloads.GEMMS[name].out_dtype == "bf16":
        # informative: entries whose bf16 differs from the correctly rounded oracle value
        want16 = orc.f32_to_bf16(ref)
        got16 = torch.from_numpy(got).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        _say(f"  bf16 entries differing from RNE(oracle): {int((want16 != got16).sum())} of {got.size}")


def _sampled(ops, orc, w: workloads.GemmWorkload, rows, npts=4096):
    A, B = workloads.gemm_inputs(w)
    lda, ldb, _ = w.lds()
    _say(f"gemm {w.name} (sampled): M={w.M} N={w.N} K={w.K} {w.b_layout} {w.out_dtype}")
    Cbuf = _run(ops, A, B, w.M, w.N, w.K, w.b_layout, w.out_dtype)
    Cbuf2 = _run(ops, A, B, w.M, w.N, w.K, w.b_layout, w.out_dtype)
    assert torch.equal(Cbuf.view(torch.int16) if Cbuf.dtype == torch.bfloat16 else Cbuf.view(torch.int32),
                       Cbuf2.view(torch.int16) if Cbuf2.dtype == torch.bfloat16 else Cbuf2.view(torch.int32)), \
        "two runs differ"
    assert bool(torch.isfinite(Cbuf).all()), "non-finite output"
    Ab, Bb = workloads.bits(A), workloads.bits(B)
    got_rows = _to_f32(Cbuf[rows])
    for i, m in enumerate(rows):
        ref = orc.gemm(Ab, Bb, w.M, w.N, w.K, lda, ldb, w.b_layout, rows=(m, m + 1))
        _check(got_rows[i:i + 1], ref, f"{w.name} row {m}")
    rng = np.random.default_rng(99)
    ms = rng.integers(0, w.M, npts)
    ns = rng.integers(0, w.N, npts)
    ref = orc.gemm_points(Ab, Bb, w.K, lda, ldb, ms, ns, w.b_layout)
    got = _to_f32(Cbuf)[ms, ns]
    _check(got, ref, f"{w.name} {npts} points")


@gpu
def test_c4_8192_sampled(ops, orc):
    w = workloads.GEMMS["c4"]
    _sampled(ops, orc, w, rows=[0, 1, 255, 256, 4097, 8190, 8191])


@gpu
def test_c5_mlp_sampled(ops, orc):
    w = workloads.GEMMS["c5"]
    _sampled(ops, orc, w, rows=[0, 300, 8191, 12345, 16383])


def _freivalds_exact(C: np.ndarray, A: np.ndarray, B: np.ndarray, bl: str, seed: int, what: str):
    """Every entry of C at once: with integer operands every partial sum below is an integer
    under 2^53, so C·x == A·(B·x) and yᵀ·C == (yᵀ·A)·B hold exactly in binary64 for the true
    product and fail for almost any wrong entry (x, y: random integers in [1, 2^16], so an error
    cancels only if weights coincide).  B is K×N for "kn", N×K for "nk"."""
    rng = np.random.default_rng(seed)
    M, N = C.shape
    x = rng.integers(1, 1 << 16, N).astype(np.float64)
    y = rng.integers(1, 1 << 16, M).astype(np.float64)
    C64, A64, B64 = C.astype(np.float64), A.astype(np.float64), B.astype(np.float64)
    Bx = B64 @ x if bl == "kn" else B64.T @ x
    yA = y @ A64
    yAB = yA @ B64 if bl == "kn" else B64 @ yA
    bad_rows = np.nonzero(C64 @ x != A64 @ Bx)[0]
    bad_cols = np.nonzero(y @ C64 != yAB)[0]
    assert bad_rows.size == 0 and bad_cols.size == 0, \
        f"{what}: {bad_rows.size} rows and {bad_cols.size} columns differ from the exact product " \
        f"(first rows {bad_rows[:8]}, first columns {bad_cols[:8]})"


def _int_operands(rng, M, N, K, bl, sparse_a):
    """Integer operands.  sparse_a: 16 entries of ±1 per row of A (some may coincide) and B in
    [-16, 16], so |C| <= 256 and every product is an integer that bf16 holds exactly; else A and
    B dense in [-8, 8] (|C| <= 64·K, exact in binary32 up to K = 2^18)."""
    shape_b = (K, N) if bl == "kn" else (N, K)
    if sparse_a:
        A = np.zeros((M, K), np.float32)
        cols = rng.integers(0, K, (M, 16))
        np.add.at(A, (np.repeat(np.arange(M), 16), cols.reshape(-1)), rng.choice([-1.0, 1.0], M * 16))
        B = rng.integers(-16, 17, shape_b).astype(np.float32)
    else:
        A = rng.integers(-8, 9, (M, K)).astype(np.float32)
        B = rng.integers(-8, 9, shape_b).astype(np.float32)
    return A, B


@gpu
@pytest.mark.parametrize("name,out,sparse", [("c4", "bf16", True), ("c4", "f32", False), ("c5", "bf16", True),
                                             ("c5", "f32", False)])
def test_full_size_exact(ops, name, out, sparse):
    """The 8192³ and 16384×14336×4096 products in full, in the launch configuration the benchmark
    times (bf16 out: the benchmark's own kernel instance), with integer operands whose product
    the output type holds exactly: every entry is then checked by Freivalds' identities."""
    w = workloads.GEMMS[name]
    rng = np.random.default_rng({"c4": 40, "c5": 50}[name] + (out == "bf16"))
    A, B = _int_operands(rng, w.M, w.N, w.K, w.b_layout, sparse)
    _say(f"full-size exact gemm {name}: M={w.M} N={w.N} K={w.K} {w.b_layout} {out} sparse_a={sparse}")
    Cbuf = _run(ops, torch.from_numpy(A).to(torch.bfloat16), torch.from_numpy(B).to(torch.bfloat16), w.M, w.N, w.K,
                w.b_layout, out)
    C = _to_f32(Cbuf)
    assert np.isfinite(C).all(), "non-finite output"
    _freivalds_exact(C, A, B, w.b_layout, 7, f"{name} {out}")


@gpu
@pytest.mark.parametrize("M,N,K,bl", [(300, 257, 136, "kn"), (300, 257, 136, "nk"), (3001, 2049, 777, "kn"),
                                      (256, 512, 8192, "kn"), (17, 1000, 520, "nk")])
def test_integer_inputs_bit_exact(ops, orc, M, N, K, bl):
    """Small integer operands: every partial sum is an integer below 2^24, so the GPU result
    must equal the oracle bit for bit, whatever order the matrix cores add in."""
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    Ai = torch.from_numpy(rng.integers(-8, 9, (M, K)).astype(np.float32)).to(torch.bfloat16)
    shape_b = (K, N) if bl == "kn" else (N, K)
    Bi = torch.from_numpy(rng.integers(-8, 9, shape_b).astype(np.float32)).to(torch.bfloat16)
    _say(f"integer gemm M={M} N={N} K={K} {bl}")
    Cbuf = _run(ops, Ai, Bi, M, N, K, bl, "f32")
    ref = orc.gemm(workloads.bits(Ai), workloads.bits(Bi), M, N, K, K, shape_b[1], bl)
    got = _to_f32(Cbuf)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} entries differ"


@gpu
def test_random_shapes(ops, orc):
    """Sizes 1..300 on every axis, both B layouts, both output types, padded leading dimensions
    (padding holds NaN) and bases off a 16-byte boundary (the repacking path)."""
    rng = np.random.default_rng(2024)
    for case in range(40):
        M, N, K, bl, out, pad = workloads.random_gemm_shape(rng)
        lda = K + (8 * pad if pad else 0)
        ldb = (N if bl == "kn" else K) + (8 * pad if pad else 0)
        A = workloads.matrix(M, K, lda, ("normal", 1.0), 100 + case)
        B = workloads.matrix(K, N, ldb, ("normal", 1.0), 200 + case) if bl == "kn" else \
            workloads.matrix(N, K, ldb, ("normal", 1.0), 200 + case)
        off = int(rng.integers(0, 3)) if case % 5 == 4 else 0
        ldc = N + int(rng.integers(0, 5))
        _say(f"random gemm {case}: M={M} N={N} K={K} {bl} {out} lda={lda} ldb={ldb} ldc={ldc} offset={off}")
        Cbuf = _run(ops, A, B, M, N, K, bl, out, ldc=ldc, a_offset=off, b_offset=off)
        ref = orc.gemm(workloads.bits(A), workloads.bits(B), M, N, K, lda, ldb, bl)
        got = _to_f32(Cbuf)
        _check(got[:, :N], ref, f"case {case}")
        assert np.all(np.isnan(got[:, N:])), "columns past N were written"


@gpu
def test_degenerate_sizes(ops):
    A = torch.randn(64, 64, device="cuda").to(torch.bfloat16)
    B = torch.randn(64, 64, device="cuda").to(torch.bfloat16)
    _say("K = 0 writes zeros")
    C = torch.full((64, 64), float("nan"), device="cuda")
    ops.gemm(A[:, :0], B[:0, :], "kn", "f32", out=C)
    torch.cuda.synchronize()
    assert bool((C == 0).all())
    _say("M = 0 and N = 0 are no-ops")
    C = torch.full((1, 64), 7.0, device="cuda")
    ops.gemm(A[:0], B, "kn", "f32", out=C[:0])
    ops.gemm(A, B[:, :0], "kn", "f32", out=torch.empty(64, 0, device="cuda"))
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
    _say("1 x 1 x 1")
    C = ops.gemm(A[:1, :1], B[:1, :1], "kn", "f32")
    torch.cuda.synchronize()
    assert float(C[0, 0]) == float(A[0, 0].float() * B[0, 0].float())


@gpu
def test_repack_many_rows(ops, orc):
    """An A of 2^22 + 5 rows with K = 7 (rows of 14 bytes: repacked to 16) is more than 2^20
    blocks of the repack, which then steps through its blocks by the grid size; B K×N with a pitch
    of 27 elements is repacked in the same launch.  Integer operands: exact.  Checked on sampled
    rows (first, last, block and grid-stride boundaries) and through Freivalds' identities."""
    M, N, K = (1 << 22) + 5, 24, 7
    rng = np.random.default_rng(23)
    A = rng.integers(-8, 9, (M, K)).astype(np.float32)
    Bbuf = np.full((K, 27), np.nan, np.float32)
    Bbuf[:, :N] = rng.integers(-8, 9, (K, N))
    _say(f"repack of {M} rows (K={K}), B pitch 27")
    Ad = torch.from_numpy(A).to(torch.bfloat16).cuda()
    Bd = torch.from_numpy(Bbuf).to(torch.bfloat16).cuda()
    C = ops.gemm(Ad, Bd[:, :N], "kn", "f32")
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    want_rows = [0, 1, 3, 4, 5, 4 * (1 << 20) - 1, 4 * (1 << 20), 4 * (1 << 20) + 1, M - 2, M - 1]
    exact = A[want_rows].astype(np.float64) @ Bbuf[:, :N].astype(np.float64)
    assert np.array_equal(got[want_rows], exact.astype(np.float32))
    _freivalds_exact(got, A, Bbuf[:, :N], "kn", 3, "repacked rows")


@gpu
def test_repack_alternates_workspace_halves(ops, orc):
    """With a workspace of twice the exact need, two successive calls put their repacked operands
    in different halves (each half then holds A's rows at the 16-byte pitch, zero padded), and
    the products are the same bits; with less than twice the need every call repacks at offset 0
    and the rest of the workspace is not written."""
    import tiled_bf16_gemm_amd as tbg
    M, N, K = 300, 257, 777  # A rows of 1554 bytes, B (K×N) rows of 514 bytes: both repacked
    A = workloads.matrix(M, K, K, ("normal", 1.0), 71)
    B = workloads.matrix(K, N, N, ("normal", 1.0), 72)
    ref = orc.gemm(workloads.bits(A), workloads.bits(B), M, N, K, K, N, "kn")
    Ad, Bd = A.cuda(), B.cuda()
    need = tbg.gemm_workspace_query(M, N, K, "bf16", Ad.data_ptr(), K, Bd.data_ptr(), N, "kn")
    a_bytes = M * 784 * 2  # lda rounded up to 8 elements, 256-byte rounded below
    assert need >= a_bytes and need % 256 == 0
    packed_a = torch.zeros((M, 784), dtype=torch.bfloat16)
    packed_a[:, :K] = A
    packed_a = packed_a.view(torch.uint8).reshape(-1)
    stream = torch.cuda.current_stream().cuda_stream
    for size, halves in ((2 * need, 2), (2 * need - 256, 1)):
        ws = torch.full((size,), 0xAB, dtype=torch.uint8, device="cuda")
        outs = []
        for call in range(2):
            C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            _say(f"workspace {size} bytes (need {need}): call {call}")
            tbg.gemm(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, "kn", C.data_ptr(), N, "f32", ws.data_ptr(), size,
                     stream)
            torch.cuda.synchronize()
            outs.append(C.cpu().numpy())
        _check(outs[0], ref, "first call")
        assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), "the two calls differ"
        host = ws.cpu()
        for h in range(halves):
            got = host[h * need: h * need + a_bytes]
            assert torch.equal(got, packed_a), f"half {h} does not hold the repacked A"
        if halves == 1:
            assert int((host[need:] != 0xAB).sum()) == 0


@gpu
def test_log_reports_the_choice(ops):
    """TBG_LOG=1 makes each call print the configuration it launches; a child process (the
    variable is read once per process) runs the 1024³ product and the ragged 3001×2049×777 one."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    child = (
        "import sys; sys.path.insert(0, %r)\n"
        "import torch\n"
        "from tiled_bf16_gemm_amd import torch_ops\n"
        "a = torch.ones(1024, 1024, dtype=torch.bfloat16, device='cuda')\n"
        "torch_ops.gemm(a, a, 'kn', 'bf16')\n"
        "b = torch.ones(3001, 777, dtype=torch.bfloat16, device='cuda')\n"
        "c = torch.ones(777, 2049, dtype=torch.bfloat16, device='cuda')\n"
        "torch_ops.gemm(b, c, 'kn', 'f32')\n"
        "torch.cuda.synchronize()\n"
    ) % root
    _say("TBG_LOG child process")
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, TBG_LOG="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("tbg: gemm")]
    assert len(lines) == 2, r.stderr[-2000:]
    assert "M=1024 N=1024 K=1024 B=kn in=bf16 out=bf16: ring 64x64, 3 stages; repack A no, B no" in lines[0]
    assert "M=3001 N=2049 K=777" in lines[1] and "repack A yes, B yes" in lines[1]


@gpu
def test_concurrent_streams(ops):
    """Products on two streams at once (the library keeps no device state between calls: every
    kernel's scratch is its own LDS, the repack goes to each caller's workspace) give the same
    bits as the same products run one after another."""
    rng = np.random.default_rng(31)
    shapes = [(1024, 1024, 1024, "kn"), (3001, 2049, 777, "kn"), (512, 768, 4096, "nk"), (300, 257, 136, "nk")]
    cases = []
    for M, N, K, bl in shapes:
        A = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16).cuda()
        Bs = (K, N) if bl == "kn" else (N, K)
        B = torch.from_numpy(rng.standard_normal(Bs).astype(np.float32)).to(torch.bfloat16).cuda()
        cases.append((A, B, bl))
    torch.cuda.synchronize()
    want = [ops.gemm(A, B, bl, "f32") for A, B, bl in cases]
    torch.cuda.synchronize()
    _say("two streams, four products each, interleaved")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[None] * len(cases) for _ in streams]
    for _ in range(4):
        for si, st in enumerate(streams):
            with torch.cuda.stream(st):
                order = list(range(si, len(cases), 2)) + list(range(1 - si, len(cases), 2))
                for idx in order:
                    A, B, bl = cases[idx]
                    outs[si][idx] = ops.gemm(A, B, bl, "f32", stream=st)
    torch.cuda.synchronize()
    for si in range(2):
        for ci in range(len(cases)):
            assert torch.equal(outs[si][ci].view(torch.int32), want[ci].view(torch.int32)), f"stream {si} case {ci}"


TILES = ["256x256", "256x128", "128x256", "128x128", "64x64"]


def _cfg(tile, stages=0, pipeline="ring"):
    import tiled_bf16_gemm_amd as tbg
    return None if tile == "auto" else tbg.gemm_config(tile, stages, pipeline)


@gpu
@pytest.mark.parametrize("tile", TILES)
def test_every_tile(ops, orc, tile):
    """Each workgroup tile the library can pick, forced through tbg_gemm_configured: ragged shapes
    against the oracle (both B layouts, both output types, a padded ldc), and small-integer
    operands bit for bit."""
    cfg = _cfg(tile)
    cases = [(700, 520, 300, "kn", "f32"), (333, 190, 200, "nk", "bf16"), (130, 70, 1, "kn", "bf16"),
             (64, 64, 64, "nk", "f32")]
    for i, (M, N, K, bl, out) in enumerate(cases):
        A = workloads.matrix(M, K, K, ("normal", 1.0), 300 + i)
        B = workloads.matrix(K, N, N, ("normal", 1.0), 400 + i) if bl == "kn" else \
            workloads.matrix(N, K, K, ("normal", 1.0), 400 + i)
        ldc = N + 3
        _say(f"tile {tile}: gemm M={M} N={N} K={K} {bl} {out} ldc={ldc}")
        Cbuf = _run(ops, A, B, M, N, K, bl, out, ldc=ldc, config=cfg)
        ref = orc.gemm(workloads.bits(A), workloads.bits(B), M, N, K, K, B.shape[1], bl)
        got = _to_f32(Cbuf)
        _check(got[:, :N], ref, f"tile {tile} case {i}")
        assert np.all(np.isnan(got[:, N:])), "columns past N were written"
    for M, N, K, bl in [(300, 257, 136, "kn"), (300, 257, 136, "nk")]:
        rng = np.random.default_rng(M + N + K)
        Ai = torch.from_numpy(rng.integers(-8, 9, (M, K)).astype(np.float32)).to(torch.bfloat16)
        shape_b = (K, N) if bl == "kn" else (N, K)
        Bi = torch.from_numpy(rng.integers(-8, 9, shape_b).astype(np.float32)).to(torch.bfloat16)
        _say(f"tile {tile}: integer gemm M={M} N={N} K={K} {bl}")
        got = _to_f32(_run(ops, Ai, Bi, M, N, K, bl, "f32", config=cfg))
        ref = orc.gemm(workloads.bits(Ai), workloads.bits(Bi), M, N, K, K, shape_b[1], bl)
        assert np.array_equal(got, ref), f"{int((got != ref).sum())} entries differ"


# Every built (pipeline, tile, stages) configuration, as include/tbg.h lists them.
CONFIGS = ([("ring", "256x256", 2)] + [("ring", t, s) for t in ("256x128", "128x256") for s in (2, 3)]
           + [("ring", "128x128", s) for s in (2, 3, 4, 5)] + [("ring", "64x64", s) for s in range(2, 7)]
           + [("producer", t, s) for t in ("256x128", "128x256") for s in (2, 3)]
           + [("producer", "128x128", s) for s in (2, 3, 4)] + [("producer", "64x64", s) for s in range(2, 7)])

# (M, N, K, B layout, C type): ragged edges everywhere; K from one partial tile (fewer K tiles
# than stages) to 16 tiles (the ring wraps several times).
CONFIG_CASES = [(700, 520, 1000, "kn", "f32"), (333, 190, 200, "nk", "bf16"), (130, 70, 1, "kn", "bf16"),
                (257, 300, 64, "nk", "f32"), (300, 257, 520, "kn", "bf16")]
_config_refs = {}


def _config_case(orc, i):
    """Inputs, oracle result and the default configuration's bits for case i (computed once)."""
    if i not in _config_refs:
        M, N, K, bl, out = CONFIG_CASES[i]
        A = workloads.matrix(M, K, K, ("normal", 1.0), 800 + i)
        B = workloads.matrix(K, N, N, ("normal", 1.0), 900 + i) if bl == "kn" else \
            workloads.matrix(N, K, K, ("normal", 1.0), 900 + i)
        ref = orc.gemm(workloads.bits(A), workloads.bits(B), M, N, K, K, B.shape[1], bl)
        _config_refs[i] = (A, B, ref, None)
    return _config_refs[i]


@gpu
@pytest.mark.parametrize("pipeline,tile,stages", CONFIGS)
def test_every_configuration(ops, orc, pipeline, tile, stages):
    """Each built pipeline × tile × stage count: ragged shapes against the oracle, bit-identical to
    the default configuration (every configuration adds the same products in the same order),
    columns past N untouched, and small-integer operands bit for bit."""
    cfg = _cfg(tile, stages, pipeline)
    for i, (M, N, K, bl, out) in enumerate(CONFIG_CASES):
        A, B, ref, base = _config_case(orc, i)
        ldc = N + 3
        _say(f"{pipeline} {tile}/{stages}: gemm M={M} N={N} K={K} {bl} {out}")
        Cbuf = _run(ops, A, B, M, N, K, bl, out, ldc=ldc, config=cfg)
        got = _to_f32(Cbuf)
        _check(got[:, :N], ref, f"{pipeline} {tile}/{stages} case {i}")
        assert np.all(np.isnan(got[:, N:])), "columns past N were written"
        if base is None:
            base = _to_f32(_run(ops, A, B, M, N, K, bl, out, ldc=ldc))
            _config_refs[i] = (A, B, ref, base)
        assert np.array_equal(got[:, :N], base[:, :N]), \
            f"{int((got[:, :N] != base[:, :N]).sum())} entries differ from the default configuration"
    M, N, K = 300, 257, 392
    for bl in ("kn", "nk"):
        rng = np.random.default_rng(4242)
        Ai = torch.from_numpy(rng.integers(-8, 9, (M, K)).astype(np.float32)).to(torch.bfloat16)
        shape_b = (K, N) if bl == "kn" else (N, K)
        Bi = torch.from_numpy(rng.integers(-8, 9, shape_b).astype(np.float32)).to(torch.bfloat16)
        _say(f"{pipeline} {tile}/{stages}: integer gemm M={M} N={N} K={K} {bl}")
        got = _to_f32(_run(ops, Ai, Bi, M, N, K, bl, "f32", config=cfg))
        ref = orc.gemm(workloads.bits(Ai), workloads.bits(Bi), M, N, K, K, shape_b[1], bl)
        assert np.array_equal(got, ref), f"{int((got != ref).sum())} entries differ"


_remainder_cache = {}


@gpu
@pytest.mark.parametrize("pipeline,tile,stages", [c for c in CONFIGS if c[2] >= 3])
def test_stage_remainders(ops, orc, pipeline, tile, stages):
    """The K loop runs S tiles per iteration (one per stage) and the last ktiles mod S tiles
    through guarded copies of the same bodies: every residue 0..S-1, each with the main loop
    taken at least once (ktiles = S + r, K ragged), both B layouts, against the oracle and
    bit-identical to the default configuration."""
    cfg = _cfg(tile, stages, pipeline)
    M, N = 150, 130
    for r in range(stages):
        K = 64 * (stages + r) - 13
        bl = "kn" if r % 2 == 0 else "nk"
        key = (K, bl)
        if key not in _remainder_cache:
            A = workloads.matrix(M, K, K, ("normal", 1.0), 1900 + K)
            B = workloads.matrix(K, N, N, ("normal", 1.0), 2900 + K) if bl == "kn" else \
                workloads.matrix(N, K, K, ("normal", 1.0), 2900 + K)
            ref = orc.gemm(workloads.bits(A), workloads.bits(B), M, N, K, K, B.shape[1], bl)
            base = _to_f32(_run(ops, A, B, M, N, K, bl, "f32"))
            _remainder_cache[key] = (A, B, ref, base)
        A, B, ref, base = _remainder_cache[key]
        _say(f"{pipeline} {tile}/{stages}: K={K} ({stages + r} K tiles, residue {r}) {bl}")
        got = _to_f32(_run(ops, A, B, M, N, K, bl, "f32", config=cfg))
        _check(got, ref, f"{pipeline} {tile}/{stages} K={K}")
        assert np.array_equal(got, base), f"{int((got != base).sum())} entries differ from the default configuration"


@gpu
@pytest.mark.parametrize("tile,stages", [(c[1], c[2]) for c in CONFIGS if c[0] == "ring"])
def test_ring_interior_boundary(ops, orc, tile, stages):
    """The ring's K loop runs unmasked iterations while every copy they issue is of a tile before
    the last one, then masked iterations and the guarded remainder.  K tiles 2S .. 3S cover every
    hand-over between the two, ragged K, M and N (rows, K chunks and the columns past N masked),
    with B stored K×N at its dense pitch (the last row's straddling chunk at the end of B) and
    stored N×K."""
    cfg = _cfg(tile, stages, "ring")
    M, N = 150, 130
    for r in range(stages + 1):
        K = 64 * (2 * stages + r) - 13
        for bl in ("kn", "nk"):
            A = workloads.matrix(M, K, K, ("normal", 1.0), 3900 + K)
            B = workloads.matrix(K, N, N, ("normal", 1.0), 4900 + K) if bl == "kn" else \
                workloads.matrix(N, K, K, ("normal", 1.0), 4900 + K)
            ref = orc.gemm(workloads.bits(A), workloads.bits(B), M, N, K, K, B.shape[1], bl)
            _say(f"ring {tile}/{stages}: K={K} ({2 * stages + r} K tiles) {bl}")
            got = _to_f32(_run(ops, A, B, M, N, K, bl, "f32", config=cfg))
            _check(got, ref, f"ring {tile}/{stages} K={K} {bl}")


def _run_ex(ops, A_cpu, B_cpu, M, N, K, b_layout, out_dtype, alpha, beta, C_old, config=None):
    """C_old: (M, ldc) CPU tensor of the output type; returns the GPU result buffer."""
    A = A_cpu.cuda()[:, :K]
    B = B_cpu.cuda()
    B = B[:, :N] if b_layout == "kn" else B[:, :K]
    Cbuf = C_old.clone().cuda()
    ops.gemm(A, B, b_layout, out_dtype, out=Cbuf[:, :N], alpha=alpha, beta=beta, config=config)
    torch.cuda.synchronize()
    return Cbuf


@gpu
@pytest.mark.parametrize("pipeline,tile", [("ring", "auto"), ("ring", "256x256"), ("ring", "128x128"),
                                           ("ring", "64x64"), ("ring", "256x128"), ("producer", "128x128"),
                                           ("producer", "64x64")])
def test_gemm_alpha_beta(ops, orc, pipeline, tile):
    """C <- alpha·A·B + beta·C against the oracle: both layouts and output types, beta = 0 with NaN
    in C (C not read), alpha = 0 (the product skipped), and exact small-integer cases."""
    cfg = _cfg(tile, 0, pipeline)
    cases = [(700, 520, 300, "kn", "f32", 1.5, -0.75), (333, 190, 200, "nk", "bf16", 0.5, 2.0),
             (257, 129, 64, "kn", "bf16", -1.25, 0.0), (96, 80, 40, "nk", "f32", 0.0, 0.5),
             (64, 64, 0, "kn", "f32", 3.0, -2.0)]
    for i, (M, N, K, bl, out, alpha, beta) in enumerate(cases):
        A = workloads.matrix(M, K, K, ("normal", 1.0), 500 + i)
        B = workloads.matrix(K, N, N, ("normal", 1.0), 600 + i) if bl == "kn" else \
            workloads.matrix(N, K, K, ("normal", 1.0), 600 + i)
        tdt = torch.float32 if out == "f32" else torch.bfloat16
        ldc = N + 5
        if beta == 0.0:
            C_old = torch.full((M, ldc), float("nan"), dtype=tdt)
        else:
            C_old = torch.from_numpy(np.random.default_rng(700 + i).normal(size=(M, ldc)).astype(np.float32)).to(tdt)
        _say(f"gemm_ex {pipeline} {tile}: M={M} N={N} K={K} {bl} {out} alpha={alpha} beta={beta}")
        Cbuf = _run_ex(ops, A, B, M, N, K, bl, out, alpha, beta, C_old, config=cfg)
        ref = orc.gemm_ex(workloads.bits(A), workloads.bits(B), M, N, K, K, B.shape[1], bl, alpha, beta,
                          C_old[:, :N].float().numpy())
        got = _to_f32(Cbuf)
        _check(got[:, :N], ref, f"gemm_ex case {i}")
        assert np.array_equal(got[:, N:], C_old[:, N:].float().numpy(), equal_nan=True), "columns past N changed"
        if alpha == 0.0:
            want = (C_old[:, :N].float() * beta).to(tdt).float().numpy()
            assert np.array_equal(got[:, :N], want), "alpha = 0 must give beta·C exactly"
    # small integers: alpha·S + beta·C is exact in binary32, so the bits must match
    M, N, K = 300, 257, 136
    rng = np.random.default_rng(77)
    Ai = torch.from_numpy(rng.integers(-8, 9, (M, K)).astype(np.float32)).to(torch.bfloat16)
    Bi = torch.from_numpy(rng.integers(-8, 9, (N, K)).astype(np.float32)).to(torch.bfloat16)
    Ci = torch.from_numpy(rng.integers(-100, 101, (M, N)).astype(np.float32))
    Cbuf = _run_ex(ops, Ai, Bi, M, N, K, "nk", "f32", 2.0, -3.0, Ci, config=cfg)
    ref = orc.gemm_ex(workloads.bits(Ai), workloads.bits(Bi), M, N, K, K, K, "nk", 2.0, -3.0, Ci.numpy())
    assert np.array_equal(_to_f32(Cbuf), ref)


F16_CONFIGS = [("ring", "256x256", 2), ("ring", "256x128", 2), ("ring", "128x256", 2), ("ring", "128x128", 2),
               ("ring", "64x64", 2), ("ring", "64x64", 3), ("producer", "256x128", 2), ("producer", "128x256", 2), ("producer", "128x128", 3),
               ("producer", "64x64", 3)]


def _f16_matrix(rows, cols, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((rows, cols), generator=g) * scale).to(torch.float16)


@gpu
@pytest.mark.parametrize("pipeline,tile,stages", [(None, None, 0)] + F16_CONFIGS)
def test_fp16_inputs(ops, orc, pipeline, tile, stages):
    """fp16 A and B (tbg_gemm_typed) against the oracle's binary16 decoding: ragged shapes, both B
    layouts, both output types, the automatic choice and every fp16 configuration, bit-identical
    across configurations; small integers bit for bit."""
    import tiled_bf16_gemm_amd as tbg
    cfg = None if pipeline is None else tbg.gemm_config(tile, stages, pipeline)
    cases = [(700, 520, 1000, "kn", "f32"), (333, 190, 200, "nk", "bf16"), (130, 70, 1, "kn", "bf16"),
             (257, 300, 64, "nk", "f32")]
    for i, (M, N, K, bl, out) in enumerate(cases):
        A = _f16_matrix(M, K, 1100 + i)
        B = _f16_matrix(K, N, 1200 + i) if bl == "kn" else _f16_matrix(N, K, 1200 + i)
        _say(f"fp16 {pipeline} {tile}/{stages}: gemm M={M} N={N} K={K} {bl} {out}")
        tdt = torch.float32 if out == "f32" else torch.bfloat16
        Cbuf = torch.full((M, N + 3), float("nan"), dtype=tdt, device="cuda")
        ops.gemm(A.cuda(), B.cuda(), bl, out, out=Cbuf[:, :N], config=cfg)
        torch.cuda.synchronize()
        got = _to_f32(Cbuf)
        ref = orc.gemm(A.view(torch.int16).numpy().view(np.uint16), B.view(torch.int16).numpy().view(np.uint16),
                       M, N, K, K, B.shape[1], bl, ab="f16")
        _check(got[:, :N], ref, f"fp16 case {i}")
        assert np.all(np.isnan(got[:, N:])), "columns past N were written"
        if cfg is not None:
            Cd = torch.empty((M, N), dtype=tdt, device="cuda")
            ops.gemm(A.cuda(), B.cuda(), bl, out, out=Cd)
            torch.cuda.synchronize()
            assert np.array_equal(got[:, :N], _to_f32(Cd)), "differs from the automatic configuration"
    M, N, K = 300, 257, 392
    rng = np.random.default_rng(88)
    for bl in ("kn", "nk"):
        Ai = torch.from_numpy(rng.integers(-16, 17, (M, K)).astype(np.float32)).to(torch.float16)
        shape_b = (K, N) if bl == "kn" else (N, K)
        Bi = torch.from_numpy(rng.integers(-16, 17, shape_b).astype(np.float32)).to(torch.float16)
        _say(f"fp16 {pipeline} {tile}/{stages}: integer gemm {bl}")
        C = ops.gemm(Ai.cuda(), Bi.cuda(), bl, "f32", config=cfg)
        torch.cuda.synchronize()
        ref = orc.gemm(Ai.view(torch.int16).numpy().view(np.uint16), Bi.view(torch.int16).numpy().view(np.uint16),
                       M, N, K, K, shape_b[1], bl, ab="f16")
        assert np.array_equal(_to_f32(C), ref)


def _f8(rows, cols, seed, fmt, scale=1.0):
    """A (rows, cols) matrix of 8-bit floats drawn N(0, scale): (uint8 bits, float32 values)."""
    g = torch.Generator().manual_seed(seed)
    tdt = torch.float8_e4m3fn if fmt == "f8e4m3" else torch.float8_e5m2
    t = (torch.randn((rows, cols), generator=g) * scale).to(tdt)
    return t.view(torch.uint8).contiguous(), t.float()


def _check_f8(got, ref, A_vals, B_vals, what):
    """oracle.gemm_check_f8: the usual rule widened by the 8-bit instruction's own dot-product
    error (oracle.F8_DOT_BOUND · Σ|a·b|, grounded by test_fp8_instruction_error)."""
    r = oracle.gemm_check_f8(got, ref, A_vals, B_vals)
    _say(f"  {what}: n={r['n']} max_abs={r['max_abs_err']:.3g} max(err/sum|ab|)={r['max_err_over_abs_dot']:.3g} "
         f"fail={r['n_fail']}")
    assert r["pass"], what


def _run_f8(M, N, K, A8, B8, fmt, out, cfg=None, lda=None, ldb=None, alpha=1.0, beta=0.0, C_old=None, ldc_pad=3):
    import tiled_bf16_gemm_amd as tbg
    lda = lda or A8.shape[1]
    ldb = ldb or B8.shape[1]
    Ad, Bd = A8.cuda(), B8.cuda()
    tdt = torch.float32 if out == "f32" else torch.bfloat16
    ldc = N + ldc_pad
    Cbuf = torch.full((M, ldc), float("nan"), dtype=tdt, device="cuda") if C_old is None else C_old.clone().cuda()
    ws = torch.empty(((M + N) * ((K + 15) // 16 * 16) + 1024), dtype=torch.uint8, device="cuda")
    tbg.gemm_typed(M, N, K, alpha, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, "nk", fmt, beta, Cbuf.data_ptr(), ldc, out,
                   cfg, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return _to_f32(Cbuf)


@gpu
@pytest.mark.parametrize("fmt", ["f8e4m3", "f8e5m2"])
def test_fp8_inputs(ops, orc, fmt):
    """OCP 8-bit inputs (tbg_gemm_typed) against the oracle, within the usual rule plus the matrix
    instruction's own dot-product error (F8_DOT_BOUND): ragged shapes (K not a multiple of 16
    bytes: repack path; an odd number of 128-wide K tiles), padded leading dimensions, both output
    types, every fp8 tile, bit-identical across tiles; small integers bit for bit; alpha/beta."""
    import tiled_bf16_gemm_amd as tbg
    ofmt = "e4m3" if fmt == "f8e4m3" else "e5m2"
    cases = [(700, 520, 1000, "f32"), (333, 190, 200, "bf16"), (130, 70, 1, "bf16"), (257, 300, 128, "f32"),
             (64, 64, 3000, "f32")]
    for i, (M, N, K, out) in enumerate(cases):
        A8, Av = _f8(M, K, 1300 + i, fmt)
        B8, Bv = _f8(N, K, 1400 + i, fmt)
        ref = orc.gemm_f8(A8.numpy(), B8.numpy(), M, N, K, K, K, ofmt)
        base = None
        for tile in (None, "256x256", "128x128", "64x64"):
            cfg = None if tile is None else tbg.gemm_config(tile, 2, "ring")
            _say(f"{fmt} gemm M={M} N={N} K={K} {out} tile {tile or 'auto'}")
            got = _run_f8(M, N, K, A8, B8, fmt, out, cfg)
            _check_f8(got[:, :N], ref, Av.numpy(), Bv.numpy(), f"{fmt} case {i} tile {tile}")
            assert np.all(np.isnan(got[:, N:])), "columns past N were written"
            if base is None:
                base = got
            else:
                assert np.array_equal(got[:, :N], base[:, :N]), "tiles disagree"
    # padded leading dimensions (multiples of 16: no repack) and a misaligned start (repack)
    M, N, K = 300, 257, 384
    A8, Av = _f8(M, K + 32, 1500, fmt)
    B8, Bv = _f8(N, K + 16, 1501, fmt)
    ref = orc.gemm_f8(A8.numpy(), B8.numpy(), M, N, K, K + 32, K + 16, ofmt)
    _say(f"{fmt} gemm padded leading dimensions")
    _check_f8(_run_f8(M, N, K, A8, B8, fmt, "f32")[:, :N], ref, Av[:, :K].numpy(), Bv[:, :K].numpy(), f"{fmt} padded")
    # small integers: every product and every partial sum of one instruction (at most 128 · 16)
    # is an integer well inside the instruction's precision, so the result is exact
    lim = 4
    rng = np.random.default_rng(91)
    Ai = rng.integers(-lim, lim + 1, (M, K)).astype(np.float32)
    Bi = rng.integers(-lim, lim + 1, (N, K)).astype(np.float32)
    tdt = torch.float8_e4m3fn if fmt == "f8e4m3" else torch.float8_e5m2
    A8 = torch.from_numpy(Ai).to(tdt).view(torch.uint8)
    B8 = torch.from_numpy(Bi).to(tdt).view(torch.uint8)
    _say(f"{fmt} integer gemm")
    got = _run_f8(M, N, K, A8, B8, fmt, "f32")
    assert np.array_equal(got[:, :N], (Ai.astype(np.float64) @ Bi.T.astype(np.float64)).astype(np.float32))
    # alpha/beta
    C_old = torch.from_numpy(rng.standard_normal((M, N + 3)).astype(np.float32))
    _say(f"{fmt} gemm alpha=2 beta=-1")
    got = _run_f8(M, N, K, A8, B8, fmt, "f32", alpha=2.0, beta=-1.0, C_old=C_old)
    want = (2.0 * (Ai.astype(np.float64) @ Bi.T.astype(np.float64)) - C_old[:, :N].double().numpy()).astype(np.float32)
    assert np.array_equal(got[:, :N], want)
    assert np.array_equal(got[:, N:], C_old[:, N:].numpy())


@gpu
@pytest.mark.parametrize("tile", ["256x256", "128x128", "64x64"])
def test_fp8_interior_boundary(ops, orc, tile):
    """K-tile counts 1..9 (128 values each), whole and ragged last tiles: the fp8 loop takes its
    pairs of tiles without masking while both tiles they copy lie before the last one, masked
    after; small integers make every result exact, so each case is compared bit for bit."""
    import tiled_bf16_gemm_amd as tbg
    cfg = tbg.gemm_config(tile, 2, "ring")
    rng = np.random.default_rng(77)
    M, N = 300, 200
    for t in range(1, 10):
        for K in (128 * t, 128 * t - 48):
            Ai = rng.integers(-4, 5, (M, K)).astype(np.float32)
            Bi = rng.integers(-4, 5, (N, K)).astype(np.float32)
            A8 = torch.from_numpy(Ai).to(torch.float8_e4m3fn).view(torch.uint8)
            B8 = torch.from_numpy(Bi).to(torch.float8_e4m3fn).view(torch.uint8)
            _say(f"fp8 interior boundary: tile {tile} K={K} ({t} K tiles)")
            got = _run_f8(M, N, K, A8, B8, "f8e4m3", "f32", cfg)
            want = (Ai.astype(np.float64) @ Bi.T.astype(np.float64)).astype(np.float32)
            assert np.array_equal(got[:, :N], want), f"K={K}: {int((got[:, :N] != want).sum())} entries differ"


@gpu
def test_fp8_torch_ops(ops, orc):
    """torch_ops.gemm on float8 tensors: the same bits as tbg_gemm_typed, for dense rows and for
    rows that the library repacks (K = 200, not a multiple of 16 bytes; a row view with pitch 210)."""
    for fmt, tdt in (("f8e4m3", torch.float8_e4m3fn), ("f8e5m2", torch.float8_e5m2)):
        for M, N, K, pitch in ((300, 260, 512, 512), (130, 90, 200, 210)):
            A8, Av = _f8(M, pitch, 1700, fmt)
            B8, Bv = _f8(N, pitch, 1701, fmt)
            _say(f"torch_ops {fmt} M={M} N={N} K={K} pitch {pitch}")
            want = _run_f8(M, N, K, A8, B8, fmt, "f32", lda=pitch, ldb=pitch)[:, :N]
            At, Bt = A8.cuda().view(tdt)[:, :K], B8.cuda().view(tdt)[:, :K]
            got = ops.gemm(At, Bt, "nk", "f32")
            torch.cuda.synchronize()
            assert np.array_equal(got.cpu().numpy(), want), (fmt, M, N, K)
            ref = orc.gemm_f8(A8.numpy(), B8.numpy(), M, N, K, pitch, pitch, "e4m3" if fmt == "f8e4m3" else "e5m2")
            _check_f8(want, ref, Av[:, :K].numpy(), Bv[:, :K].numpy(), f"{fmt} torch_ops")
        with pytest.raises(Exception):
            ops.gemm(At, Bt.t(), "kn", "f32")


@gpu
def test_fp8_large_sampled(ops, orc):
    """The 16384×14336×4096 product (the MLP workload's shape) with E4M3 inputs: sampled rows
    against the oracle, finite everywhere, deterministic."""
    M, N, K = 16384, 14336, 4096
    A8, Av = _f8(M, K, 1600, "f8e4m3")
    B8, Bv = _f8(N, K, 1601, "f8e4m3", 0.05)
    _say("fp8 16384x14336x4096")
    got = _run_f8(M, N, K, A8, B8, "f8e4m3", "bf16", ldc_pad=0)
    again = _run_f8(M, N, K, A8, B8, "f8e4m3", "bf16", ldc_pad=0)
    assert np.isfinite(got).all()
    assert np.array_equal(got, again), "not deterministic"
    for m0 in (0, 7777, M - 64):
        ref = orc.gemm_f8(A8.numpy(), B8.numpy(), M, N, K, K, K, "e4m3", rows=(m0, m0 + 64))
        _check_f8(got[m0:m0 + 64], ref, Av[m0:m0 + 64].numpy(), Bv.numpy(), f"fp8 rows {m0}..{m0 + 64}")


@gpu
def test_graph_capture(ops, orc):
    """The GEMM under HIP graph capture (torch.cuda.graph): three products (plain, the repack
    path of a leading dimension off 16 bytes, and C <- alpha·A·B + beta·C) are captured once and
    replayed three times, with eager work between the replays; every replay equals the eager
    result bit for bit."""
    rng = np.random.default_rng(77)
    cases = [(512, 384, 256, "kn", 256), (300, 257, 777, "kn", 777), (256, 256, 512, "nk", 512)]
    ins, outs, eager = [], [], []
    for M, N, K, bl, lda in cases:
        A = torch.from_numpy(rng.standard_normal((M, lda)).astype(np.float32)).to(torch.bfloat16).cuda()[:, :K]
        B = torch.from_numpy(rng.standard_normal((K, N) if bl == "kn" else (N, K)).astype(np.float32)).to(
            torch.bfloat16).cuda()
        C0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).cuda()
        ins.append((A, B, bl, C0))
    # eager results; the third case as C <- 1.5 AB - 0.5 C0
    for i, (A, B, bl, C0) in enumerate(ins):
        C = C0.clone()
        if i == 2:
            ops.gemm(A, B, bl, "f32", out=C, alpha=1.5, beta=-0.5)
        else:
            ops.gemm(A, B, bl, "f32", out=C)
        eager.append(C)
    torch.cuda.synchronize()
    # the workspace the repack case uses is allocated before capture
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    outs = [C0.clone() for (_, _, _, C0) in ins]
    starts = [C0.clone() for (_, _, _, C0) in ins]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm-up on the capture stream
        for i, (A, B, bl, _) in enumerate(ins):
            if i == 2:
                ops.gemm(A, B, bl, "f32", out=outs[i], workspace=ws, alpha=1.5, beta=-0.5)
            else:
                ops.gemm(A, B, bl, "f32", out=outs[i], workspace=ws)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i, (A, B, bl, _) in enumerate(ins):
            if i == 2:
                ops.gemm(A, B, bl, "f32", out=outs[i], workspace=ws, alpha=1.5, beta=-0.5)
            else:
                ops.gemm(A, B, bl, "f32", out=outs[i], workspace=ws)
    for rep in range(3):
        for i in range(3):
            outs[i].copy_(starts[i])  # C holds the old C again for the alpha/beta case
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"graph replay {rep}")
        for i in range(3):
            assert torch.equal(outs[i], eager[i]), f"replay {rep} case {i} differs from the eager result"
        # eager work between replays
        x = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        del x
    del g


@gpu
@pytest.mark.parametrize("pipeline,tile,stages", CONFIGS)
def test_permutation_products(ops, pipeline, tile, stages):
    """Closed forms that pin the product's row and column placement without the oracle: for a
    selection matrix P (each row a single 1, at a random column), P·B is B's rows picked out in
    P's order and Bᵀ·Pᵀ (Pᵀ given as P stored N×K) the same columns, exactly; and I·B = B.
    Ragged sizes, both B layouts, fp32 out; random bf16 values, so any entry landing in the wrong
    place shows."""
    cfg = _cfg(tile, stages, pipeline)
    rng = np.random.default_rng(4242)
    M, K, N = 300, 257, 193
    for case in ("select", "identity"):
        perm = rng.integers(0, K, M) if case == "select" else np.arange(K)
        P = np.zeros((len(perm), K), np.float32)
        P[np.arange(len(perm)), perm] = 1.0
        Bkn = torch.randn((K, N), generator=torch.Generator().manual_seed(int(rng.integers(1 << 30)))).to(torch.bfloat16)
        want = Bkn.float().numpy()[perm]  # (rows of P) × N
        Pt = torch.from_numpy(P).to(torch.bfloat16)
        _say(f"{pipeline} {tile}/{stages}: {case} · B (K×N and N×K)")
        got = ops.gemm(Pt.cuda(), Bkn.cuda(), "kn", "f32", config=cfg)
        got_nk = ops.gemm(Pt.cuda(), Bkn.t().contiguous().cuda(), "nk", "f32", config=cfg)
        # B' · Pᵀ with B' = Bᵀ (N×K row-major A operand) and Pᵀ given as P stored N×K
        got_cols = ops.gemm(Bkn.t().contiguous().cuda(), Pt.cuda(), "nk", "f32", config=cfg)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), want), f"{case}: P·B (K×N) misplaced entries"
        assert np.array_equal(got_nk.cpu().numpy(), want), f"{case}: P·B (N×K) misplaced entries"
        assert np.array_equal(got_cols.cpu().numpy(), want.T), f"{case}: Bᵀ·Pᵀ misplaced entries"
