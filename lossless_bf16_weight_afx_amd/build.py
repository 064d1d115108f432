"""Compile libafx.so (HIP for gfx950 plus its host half) in-tree with hipcc."""
from __future__ import annotations

import functools
import hashlib
import os
import subprocess
import sys
import tempfile

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


@functools.lru_cache(maxsize=None)
def device_code_sha(source: str) -> str:
    """A hash of the gfx950 code that one kernel source compiles to: the
    device assembly hipcc makes from csrc/<source> with the library's flags,
    without comments, debug lines and the compiler's per-unit id. A profile
    records it: edits that leave the code unchanged (comments, host-side
    code) keep a profile valid, any change to the generated code makes it
    stale."""
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        subprocess.run([HIPCC, *DEVICE_FLAGS, "-O3", "-std=c++17", "--cuda-device-only", "-S",
                        "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, source), "-o", out],
                       check=True, capture_output=True)
        h = hashlib.sha256()
        with open(out) as f:
            for line in f:
                t = line.split(";", 1)[0].strip()
                if not t or t.startswith((".loc", ".file", ".ident")) or "__hip_cuid_" in t:
                    continue
                h.update(t.encode() + b"\n")
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
