"""Build ``liboracle.so`` from ``oracle.c`` with the host C compiler (test infrastructure only).

Floating-point contraction is off so every product and every addition rounds on its own, as the
source reads; the instruction set is the portable x86-64-v2 level so the library built here also
runs on other hosts.  ``extra_cflags`` lets a test build a deliberately broken copy (``-D`` flags)
into another path."""
from __future__ import annotations

import os
import subprocess
import sys
from typing import Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(out: str = OUT, extra_cflags: Sequence[str] = ()) -> str:
    cc = os.environ.get("CC", "gcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc, "-O2", "-march=x86-64-v2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra", *extra_cflags, SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(extra_cflags=sys.argv[1:]))
