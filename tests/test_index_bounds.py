"""A corrupt device blob decodes to wrong bits, never out of bounds (CPU).

The restore kernels form every index that depends on blob contents (chunk
bases, gaps, code lengths, code words) with the constexpr functions of
csrc/afx_index.h. tests/native/index_check.cpp drives those same functions
the way the kernels compose them, on random and wild inputs, and checks
every LDS slot and global word index against its buffer. It is built here
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer (a shift or
overflow that is undefined fails too). A planted mistake in a copy of the
header (a clamp removed) must make it fail.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "lossless_bf16_weight_afx_amd", "csrc")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def build(tmp_path, csrc=CSRC):
    exe = tmp_path / "index_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", *SANITIZE, "-I", csrc,
                    os.path.join(ROOT, "tests", "native", "index_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    return exe


def test_every_index_in_range(tmp_path):
    exe = build(tmp_path)
    r = subprocess.run([str(exe), "300000", "7"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 out of range" in r.stdout


@pytest.mark.parametrize("what,old,new", [
    ("chain start unclamped", "return 32 * kRev - umin32(rel + gap, kMaxStart) + kLead;",
     "return 32 * kRev - (rel + gap) + kLead;"),
    ("stream words unclamped", "constexpr uint64_t word4_index(uint64_t g, uint64_t last4) { return umin64(g, last4); }",
     "constexpr uint64_t word4_index(uint64_t g, uint64_t last4) { return g; }"),
    ("staged word count unclamped", "g.nwords = (uint32_t)umin64(want, kStageWords);", "g.nwords = (uint32_t)want;"),
    ("gap slot unclamped", "constexpr uint32_t gap_slot(uint32_t g, uint32_t ng) { return umin32(g, ng - 1); }",
     "constexpr uint32_t gap_slot(uint32_t g, uint32_t ng) { return g; }"),
    ("segment chain start unclamped", "return 32 * kSegRev - (uint32_t)umin64(p - 32 * wa, kSegMaxStart);",
     "return 32 * kSegRev - (uint32_t)(p - 32 * wa);"),
    ("launch order's token block off by a factor", "constexpr uint32_t gemm_block_token(uint32_t b, uint32_t nt) { return (b / 8) % nt; }",
     "constexpr uint32_t gemm_block_token(uint32_t b, uint32_t nt) { return b % nt; }"),
])
def test_check_catches_a_removed_clamp(tmp_path, what, old, new):
    """Control: the check is able to fail (each clamp it relies on matters)."""
    # a copy of the sources laid out as in the package: csrc/../../include/afx.h
    d = tmp_path / "pkg" / "csrc"
    shutil.copytree(CSRC, d)
    os.makedirs(tmp_path / "include")
    shutil.copy(os.path.join(ROOT, "include", "afx.h"), tmp_path / "include" / "afx.h")
    text = (d / "afx_index.h").read_text()
    assert text.count(old) == 1, what
    (d / "afx_index.h").write_text(text.replace(old, new))
    exe = build(tmp_path, str(d))
    r = subprocess.run([str(exe), "50000", "7"], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"{what}: the check did not notice\n{r.stdout}"
