"""The library's host-side code and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/native/host_check.cpp drives the encoder, blob validation, the host
unpack, the file reader and the oracle's encoder and decoders, including on
damaged blobs; here it is built with g++/gcc with both sanitizers (host code
only: no HIP source is part of that program) and must finish cleanly.
"""
import os
import subprocess

from conftest import ROOT

CSRC = os.path.join(ROOT, "lossless_bf16_weight_afx_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]


def test_host_code_clean_under_sanitizers(tmp_path):
    objs = []
    for src in ("afx_host.cpp", "afx_io.cpp", "afx_host_decode.cpp"):
        o = tmp_path / (src + ".o")
        subprocess.run(["g++", "-std=c++17", "-pthread", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(CSRC, src), "-o", str(o)], check=True, capture_output=True, text=True)
        objs.append(str(o))
    o = tmp_path / "afx_oracle.o"
    subprocess.run(["gcc", "-std=c11", "-pthread", *SAN, "-c", os.path.join(ROOT, "oracle", "afx_oracle.c"), "-o",
                    str(o)], check=True, capture_output=True, text=True)
    objs.append(str(o))
    exe = tmp_path / "host_check"
    subprocess.run(["g++", "-std=c++17", "-pthread", *SAN, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "native", "host_check.cpp"), *objs, "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=900, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failures" in r.stdout
