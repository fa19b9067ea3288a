"""Compile the CPU oracle (plain C) into oracle/liboracle.so with gcc.

Test infrastructure: the product library never links this.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    lm = os.path.getmtime(LIB)
    return any(os.path.getmtime(os.path.join(HERE, f)) > lm
               for f in ("nvfp4_oracle.c", "nvfp4_oracle.h"))


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
