"""Compile libafx.so (HIP for gfx950 plus its host half) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libafx.so")
SOURCES = [os.path.join(CSRC, "afx_host.cpp"), os.path.join(CSRC, "afx_io.cpp"),
           os.path.join(CSRC, "afx_host_decode.cpp"), os.path.join(CSRC, "afx_decode.hip"),
           os.path.join(CSRC, "afx_gemv.hip"), os.path.join(CSRC, "afx_gemm.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 instructions are kept out of every device build.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    cmd = [HIPCC, *DEVICE_FLAGS, "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", LIB + ".tmp", *(extra_flags or [])]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
