"""The C ABI from a plain C99 program (tests/c_client/tbg_client.c): the header compiles as C with
warnings as errors, the program links libtbg.so, and its host-side checks pass; on a GPU it runs
one product through tbg_gemm with device memory from the HIP runtime, compared with the oracle
bit for bit (small integer operands: every partial sum is exact in binary32)."""
import os
import subprocess

import numpy as np
import pytest
import torch

import tiled_bf16_gemm_amd as tbg
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_client", "tbg_client.c")


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("c_client") / "tbg_client")
    libdir = os.path.dirname(tbg.library_path())
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", SRC, "-o", exe, "-L", libdir, "-ltbg", "-Wl,-rpath," + libdir,
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_client_host_checks(client):
    r = subprocess.run([client, "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.gpu
def test_c_client_gemm(client, orc, tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M, N, K = 300, 264, 200
    rng = np.random.default_rng(12)
    A = torch.from_numpy(rng.integers(-8, 9, (M, K)).astype(np.float32)).to(torch.bfloat16)
    B = torch.from_numpy(rng.integers(-8, 9, (K, N)).astype(np.float32)).to(torch.bfloat16)
    inp = str(tmp_path / "ab")
    workloads.bits(A).tofile(inp + ".a")
    workloads.bits(B).tofile(inp + ".b")
    out = str(tmp_path / "c.f32")
    print(f"C client gemm M={M} N={N} K={K}", flush=True)
    r = subprocess.run([client, "gemm", str(M), str(N), str(K), inp, out], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    got = np.fromfile(out, dtype=np.float32).reshape(M, N)
    ref = orc.gemm(workloads.bits(A), workloads.bits(B), M, N, K, K, N, "kn")
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} entries differ"
