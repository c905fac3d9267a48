"""Build ``librkv.so`` (the HIP kernels and their C ABI) for gfx950 with hipcc.

The library is built in-tree, next to this file.  Packed-FP32 instructions
are disabled for all device code (``-packed-fp32-ops``); the host pass of
hipcc warns that it does not know that feature, which is harmless.  The
kernels take the values a wave needs first as leading scalar arguments, and
the build asks for them to be preloaded into SGPRs at wave start.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "librkv.so")
SOURCES = [os.path.join(CSRC, f) for f in ("rkv_abi.hip", "rkv_kernels.hip",
                                            "rkv_kernels_fp8.hip", "rkv_kernels_norm.hip",
                                            "rkv_kernels_norm_fp8.hip", "rkv_meta.hip")]
OBJ_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Kernel-argument preloading: the leading scalar arguments of every kernel
# (up to 14 dwords) are written into SGPRs when a wave starts.
PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=10"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *PRELOAD,
         "-Wall", "-Wno-unused-command-line-argument"]


def build(out: str = LIB_PATH, extra=()) -> str:
    """Compile every source to an object (in parallel), then link."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = os.path.basename(out).replace(".so", "")

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, f"{tag}_{os.path.basename(src)}.o")
        subprocess.run([HIPCC, *FLAGS, *extra, "-c", "-o", obj, src], check=True)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", out + ".tmp",
                    *objs], check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
