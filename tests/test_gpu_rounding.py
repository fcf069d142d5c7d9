"""GPU unit checks of the numeric steps below the GEMM's tolerance: the epilogue's fp32 → bf16
rounding, bit for bit, and the 8-bit matrix instruction's own summation error.

The epilogue rounds the binary32 sum to bf16 to nearest, ties to even (the pages fix bf16 inputs
with fp32 accumulation; the conversion's rounding is the IEEE default).  With small-integer
operands every product and partial sum is an integer below 2^24, so the kernel's binary32 sum
is the exact product whatever the order of its additions; the sums exceed bf16's 8 significant
bits, so the bf16 result is exactly the oracle's round-to-nearest-even of its binary32 result.
Every built configuration is run, with the plain and the alpha/beta epilogue, and a K = 2 case
whose entries are built to fall exactly halfway between two bf16 values (both tie directions).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.test_gpu_gemm import CONFIGS, _cfg, _say, gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tiled_bf16_gemm_amd import torch_ops
    return torch_ops


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _int_case(M, N, K, bl, seed, lim=8):
    rng = np.random.default_rng(seed)
    A = torch.from_numpy(rng.integers(-lim, lim + 1, (M, K)).astype(np.float32)).to(torch.bfloat16)
    shape_b = (K, N) if bl == "kn" else (N, K)
    B = torch.from_numpy(rng.integers(-lim, lim + 1, shape_b).astype(np.float32)).to(torch.bfloat16)
    return A, B, shape_b[1]


def _tie_case():
    """K = 2 products whose exact value lies halfway between two bf16 numbers in many entries:
    C[m, n] = s_m + t_m·u_n with s_m a power of two and t_m = q_m·s_m/256, so C = s_m·(1 +
    q_m·u_n/256); bf16 spaces values s_m/128 apart in [s_m, 2·s_m), so every odd q_m·u_n is a tie
    (rounded down when the lower neighbour's last significand bit is 0, up otherwise)."""
    M, N = 128, 96
    scales = np.array([256.0, 512.0, 1024.0, 4096.0, 2.0 ** 20, 0.5, 2.0 ** -10, 65536.0])
    rng = np.random.default_rng(2024)
    q = rng.integers(-16, 17, M).astype(np.float64)
    u = rng.integers(-16, 17, N).astype(np.float64)
    s = scales[np.arange(M) % len(scales)]
    A = np.stack([s, q * s / 256.0], axis=1).astype(np.float32)        # exact in bf16: ≤ 5 significant bits
    Bkn = np.stack([np.ones(N), u], axis=0).astype(np.float32)
    exact = s[:, None] + (q * s / 256.0)[:, None] * u[None, :]
    # a binary32 value is a bf16 tie when its low 16 bits are exactly half a bf16 unit
    ties = (exact.astype(np.float32).view(np.uint32) & 0xFFFF) == 0x8000
    return (torch.from_numpy(A).to(torch.bfloat16), torch.from_numpy(Bkn).to(torch.bfloat16), exact, ties)


@gpu
@pytest.mark.parametrize("pipeline,tile,stages", CONFIGS)
def test_bf16_output_rounding_every_configuration(ops, orc, pipeline, tile, stages):
    """Dense integer operands in [-8, 8] with K = 777 and K = 1000 (|C| up to 8000, well past
    bf16's 256, while every binary32 partial sum stays exact): the bf16 output equals
    oracle.f32_to_bf16 of the exact binary32 product, bit for bit, for the plain epilogue and the
    alpha/beta one (alpha = 1.5, beta = -0.5 on an integer C: alpha·S + beta·C is exact in
    binary32 and rounded once)."""
    cfg = _cfg(tile, stages, pipeline)
    for i, (M, N, K, bl) in enumerate([(300, 257, 777, "kn"), (257, 300, 1000, "nk")]):
        A, B, ldb = _int_case(M, N, K, bl, 31 + i)
        ref32 = orc.gemm(workloads.bits(A), workloads.bits(B), M, N, K, K, ldb, bl)
        want = orc.f32_to_bf16(ref32)
        assert np.abs(ref32).max() > 256, "the sums must exceed bf16's significand"
        assert not np.array_equal(want.astype(np.uint32) << 16, ref32.view(np.uint32)), "rounding must occur"
        _say(f"{pipeline} {tile}/{stages}: bf16 out, integer gemm M={M} N={N} K={K} {bl}")
        got = ops.gemm(A.cuda(), B.cuda(), bl, "bf16", config=cfg)
        torch.cuda.synchronize()
        g = _bf16_bits(got)
        assert np.array_equal(g, want), f"{int((g != want).sum())} bf16 entries differ from RNE of the exact sum"
        # alpha/beta epilogue on the same product
        rng = np.random.default_rng(77 + i)
        C_old = torch.from_numpy(rng.integers(-64, 65, (M, N)).astype(np.float32)).to(torch.bfloat16)
        ref_ex = orc.gemm_ex(workloads.bits(A), workloads.bits(B), M, N, K, K, ldb, bl, 1.5, -0.5,
                             C_old.float().numpy())
        want_ex = orc.f32_to_bf16(ref_ex)
        out = C_old.clone().cuda()
        _say(f"{pipeline} {tile}/{stages}: bf16 out, alpha/beta")
        ops.gemm(A.cuda(), B.cuda(), bl, "bf16", out=out, alpha=1.5, beta=-0.5, config=cfg)
        torch.cuda.synchronize()
        g = _bf16_bits(out)
        assert np.array_equal(g, want_ex), f"{int((g != want_ex).sum())} alpha/beta entries differ"


@gpu
@pytest.mark.parametrize("tile", ["auto", "256x256", "128x128", "64x64"])
def test_bf16_output_exact_ties(ops, orc, tile):
    """K = 2 entries built to lie exactly halfway between two bf16 values: each must round to the
    neighbour with an even last significand bit, as the oracle's rounding does."""
    A, Bkn, exact, ties = _tie_case()
    M, N = exact.shape
    assert ties.sum() >= 1000, "the case must hold many exact ties"
    ref32 = orc.gemm(workloads.bits(A), workloads.bits(Bkn), M, N, 2, 2, N, "kn")
    assert np.array_equal(ref32.astype(np.float64), exact), "the exact sums are binary32 values"
    want = orc.f32_to_bf16(ref32)
    # both directions occur among the ties
    up = (want.astype(np.uint32) << 16).view(np.float32).astype(np.float64) > exact
    assert (up & ties).any() and (~up & ties).any()
    cfg = _cfg(tile, 0, "ring")
    for bl, Bop in (("kn", Bkn), ("nk", Bkn.t().contiguous())):
        _say(f"ties: tile {tile} {bl}")
        got = ops.gemm(A.cuda(), Bop.cuda(), bl, "bf16", config=cfg)
        torch.cuda.synchronize()
        g = _bf16_bits(got)
        assert np.array_equal(g, want), f"{int((g != want).sum())} of {int(ties.sum())} ties rounded differently"


@gpu
@pytest.mark.parametrize("fmt", ["f8e4m3", "f8e5m2"])
def test_fp8_instruction_error(ops, orc, fmt):
    """A hardware characterisation, kept as the basis of oracle.F8_DOT_BOUND: with K = 128 every
    output of the fp8 GEMM is one 16×16×128 8-bit matrix instruction adding 128 exact products.
    On random inputs its error against the exact sum (binary64 oracle) stays within
    2^-15 · Σ_k |a_k·b_k|; the comparator allows four times that."""
    import tiled_bf16_gemm_amd as tbg
    M, N, K = 2048, 1024, 128
    tdt = torch.float8_e4m3fn if fmt == "f8e4m3" else torch.float8_e5m2
    g = torch.Generator().manual_seed(5150)
    A8 = torch.randn((M, K), generator=g).to(tdt)
    B8 = torch.randn((N, K), generator=g).to(tdt)
    a, b = A8.float().numpy().astype(np.float64), B8.float().numpy().astype(np.float64)
    _, ref64 = orc.gemm_f8(A8.view(torch.uint8).numpy(), B8.view(torch.uint8).numpy(), M, N, K, K, K,
                           "e4m3" if fmt == "f8e4m3" else "e5m2", want64=True)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Ad, Bd = A8.view(torch.uint8).cuda(), B8.view(torch.uint8).cuda()
    tbg.gemm_typed(M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), K, "nk", fmt, 0.0, C.data_ptr(), N, "f32", None,
                   0, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    err = np.abs(C.cpu().numpy().astype(np.float64) - ref64)
    absum = np.abs(a) @ np.abs(b).T
    ratio = float((err / np.maximum(absum, 1e-300)).max())
    _say(f"{fmt}: {M * N} outputs, max |err| / sum|ab| = 2^{np.log2(max(ratio, 1e-300)):.2f}")
    assert ratio <= 2.0 ** -15
    assert oracle.F8_DOT_BOUND == 4 * 2.0 ** -15
