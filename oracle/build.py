"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: only the tests, the package smoke check and the
benchmark's CPU-baseline leg load the result.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "h2o_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No fast-math and no FMA contraction: every operation is the rounded IEEE
# fp64 operation the source spells out.
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    cmd = ["gcc", *CFLAGS, *extra, "-I", HERE, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
