"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only; device
code is not instrumented): csrc/api.hip is compiled with both sanitizers on its host side only,
linked with the library's other objects, and the plain C caller tests/c_client/tbg_client.c,
built with the same sanitizers, runs its host checks (descriptor encoding, every rejection,
GEMM argument checks) against it.  Any report fails the test."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_bf16_gemm_amd", "csrc")
OBJS = os.path.join(ROOT, "tiled_bf16_gemm_amd", "_build")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


def test_abi_host_code_under_sanitizers(tmp_path):
    others = [o for o in glob.glob(os.path.join(OBJS, "*.o")) if os.path.basename(o) != "api.o"]
    if not others or not os.path.exists(CLANG):
        pytest.skip("the library's objects (build() first) or ROCm's clang are missing")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    obj = str(tmp_path / "api_san.o")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", *san, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
                    os.path.join(CSRC, "api.hip"), "-o", obj], check=True, capture_output=True)
    lib = str(tmp_path / "libtbg.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san[:4], obj, *others, "-o", lib],
                   check=True, capture_output=True)
    exe = str(tmp_path / "tbg_client")
    subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "c_client", "tbg_client.c"), "-o", exe, "-L", str(tmp_path), "-ltbg",
                    "-Wl,-rpath," + str(tmp_path), "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                   check=True, capture_output=True)
    r = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-4000:]
