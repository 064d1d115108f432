"""The restore's division of a launch's grid among its tensors (CPU).

tests/native/split_check.cpp drives csrc/afx_split.h, the function the
restore's launch code calls: every tensor's workgroup range inside the grid,
every chunk assigned once under the kernel's rotation, no idle workgroup,
never a busier workgroup than the proportional split, the fewest possible
chunks on the busiest workgroup wherever brute force over all allocations
can tell, and a decoder layer on the full grid launched exactly as the
proportional split. Built under AddressSanitizer and UndefinedBehaviorSanitizer.
A planted mistake in a copy of the header must make it fail.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "lossless_bf16_weight_afx_amd", "csrc")


def build(tmp_path, csrc=CSRC):
    exe = tmp_path / "split_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", csrc, os.path.join(ROOT, "tests", "native", "split_check.cpp"),
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    return exe


def test_grid_split(tmp_path):
    r = subprocess.run([str(build(tmp_path))], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "split ok" in r.stdout


@pytest.mark.parametrize("what,old,new", [
    ("second candidate always taken", "if (min_max >= prop_max) return grid;", "if (false) return grid;"),
    ("workgroups counted with floor division", "for (uint32_t t = 0; t < n_big; ++t) k += (chunks[t] + L - 1) / L;",
     "for (uint32_t t = 0; t < n_big; ++t) k += chunks[t] / L;"),
    ("bisection stops one short", "            L_lo = mid + 1;", "            L_lo = mid + 2;"),
])
def test_check_catches_a_planted_mistake(tmp_path, what, old, new):
    d = tmp_path / "csrc"
    d.mkdir()
    text = open(os.path.join(CSRC, "afx_split.h")).read()
    assert text.count(old) == 1, what
    (d / "afx_split.h").write_text(text.replace(old, new))
    r = subprocess.run([str(build(tmp_path, str(d)))], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"{what}: the check did not notice\n{r.stdout}"
