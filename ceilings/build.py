"""Build ``libceilings.so`` (the measurement kernels bench.py times beside the
library) for gfx950 with hipcc, in-tree, with the library's compiler flags."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rkv_ceilings.hip")
LIB_PATH = os.path.join(HERE, "libceilings.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-kernarg-preload-count=10",
         "-Wall", "-Wno-unused-command-line-argument"]


def build(out: str = LIB_PATH) -> str:
    subprocess.run([HIPCC, *FLAGS, "-o", out + ".tmp", SRC], check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:]))
