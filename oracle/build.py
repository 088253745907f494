"""Build ``liboracle.so`` from ``oracle.c`` with gcc.

The oracle is plain C with OpenMP over tokens. It is compiled without
fast-math and without floating-point contraction so that every fp32 operation
rounds as written.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(src: str = SRC, out: str = OUT, extra=()) -> str:
    """Compile ``src`` into the shared library ``out``; returns ``out``."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:]))
