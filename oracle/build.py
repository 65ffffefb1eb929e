"""Compile the C oracle into oracle/libgboracle.so with gcc.

Test infrastructure: the flags keep binary32 arithmetic plain IEEE
(no fast-math, no fused multiply-add contraction).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libgboracle.so")
SRC = os.path.join(HERE, "gb_oracle.c")

CFLAGS = ["-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
          "-fexcess-precision=standard", "-fPIC", "-Wall", "-Wextra", "-Werror"]


def build(verbose=False):
    """Build the oracle library unconditionally; return its path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-shared", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
