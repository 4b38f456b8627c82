"""Compile the C oracle (test infrastructure) with the host gcc.

No fast-math and no FMA contraction: the oracle evaluates each fp64
expression as written.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssd_oracle.c")
LIB = os.path.join(HERE, "libssd_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Werror"]


def compile_oracle(src: str = SRC, out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def ensure_built() -> str:
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        compile_oracle()
    return LIB


if __name__ == "__main__":
    print(compile_oracle(), file=sys.stderr)
