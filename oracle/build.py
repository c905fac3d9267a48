"""Build the CPU oracle (``liboracle_rkv.so``) with gcc -- TEST INFRASTRUCTURE.

The flags keep the arithmetic as written: no contraction into FMA, no fast
math, IEEE semantics.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rkv_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle_rkv.so")
CFLAGS = ["-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Werror"]


def build(src: str = SRC, out: str = LIB_PATH) -> str:
    cmd = ["gcc", *CFLAGS, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:]))
