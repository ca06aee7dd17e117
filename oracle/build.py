"""Compile the oracle's C source into a shared library with gcc.

Test infrastructure only (see ``conv_fprop_oracle.c``).  Plain ``-O2``: no
intrinsics, no vectorisation flags, OpenMP for the (batch, channel) split.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "conv_fprop_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "liboracle_conv.so")


def compile_oracle(src: str = SRC, out: str = LIB, extra=()) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(compile_oracle(*sys.argv[1:2]))
