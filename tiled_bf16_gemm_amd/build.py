"""Build ``libtbg.so`` (the C-ABI library) from ``csrc/*.hip`` with hipcc, for gfx950 only.

Run ``python tiled_bf16_gemm_amd/build.py`` (or ``__graft_entry__.build()``).  The library is
built in-tree next to this file.  ``TBG_SAVE_ISA=<dir>`` also writes the device assembly there.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtbg.so")
# The benchmark's measurement aid (products alone, the power-limited ceiling): a library of its own,
# outside the C ABI of include/tbg.h.
DIAG_SRC = os.path.join(HERE, "diag", "mfma_rate.hip")
DIAG_LIB = os.path.join(HERE, "diag", "libtbg_diag.so")
# The hand-off checking build of the same sources (TBG_HANDOFF_CHECK=1: every stage hand-off
# drains all copies and LDS reads), with the same C ABI; only the tests load it.
CHECK_LIB = os.path.join(HERE, "diag", "libtbg_check.so")


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
        # no packed fp32 arithmetic anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIB, verbose: bool = False, check: bool = True) -> str:
    """Compile every csrc/*.hip to an object in parallel (one hipcc per file), then link; then the
    measurement library and (check=True) the hand-off checking build of the same sources."""
    build_library(out, verbose)
    tmp = DIAG_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *flags(), "-shared", DIAG_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {DIAG_SRC}:\n{r.stderr}")
    os.replace(tmp, DIAG_LIB)
    if check:
        build_library(CHECK_LIB, verbose, defines=["-DTBG_HANDOFF_CHECK=1"], objdir="_build_check")
    isa_dir = os.environ.get("TBG_SAVE_ISA")
    if isa_dir:
        save_isa(isa_dir)
    return out


def build_library(out: str, verbose: bool = False, defines=(), objdir: str = "_build") -> str:
    import concurrent.futures
    objdir = os.path.join(HERE, objdir)
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [hipcc(), *flags(), *defines, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if msg.strip() and verbose:
            print(msg, flush=True)
        return obj

    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def save_isa(out_dir: str) -> None:
    os.makedirs(out_dir, exist_ok=True)
    for src in sources():
        name = os.path.splitext(os.path.basename(src))[0]
        subprocess.run([hipcc(), *flags(), "--offload-device-only", "-S", src, "-o",
                        os.path.join(out_dir, name + ".s")], check=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
