"""The committed rocprofv3 summaries describe the kernel sources as they are.

Each summary records a hash of its kernel's generated gfx950 code (the
device assembly of its source, comments aside); bench.py reports a
profile's HBM traffic only while that hash matches. A summary whose hash no
longer matches was taken on other code and must be retaken, not kept.
"""
import glob
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt")))


def _fields(path):
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = (t.strip() for t in line.split("=", 1))
            kv[k] = v
    return kv


def test_every_kernel_has_a_timed_summary():
    names = {os.path.basename(p) for p in SUMMARIES}
    for kernel in bench.KERNEL_SRCS:
        assert any(n.startswith(kernel + "_") and n.endswith("_pmc.txt") for n in names), kernel


@pytest.mark.parametrize("path", SUMMARIES, ids=os.path.basename)
def test_summary_matches_current_sources(path):
    kv = _fields(path)
    kernel = kv.get("kernel")
    assert kernel in bench.KERNEL_SRCS, f"{path}: unknown kernel {kernel}"
    assert os.path.basename(path).startswith(kernel + "_")
    assert kv.get("kernel_sha") == bench.kernel_sha(kernel), f"{path} was taken on other sources of {kernel}"
    if path.endswith("_pmc.txt"):
        # the trace's average launch and the HBM bytes it reports
        assert float(kv["avg_duration_ns"]) > 0
        traffic = float(kv["hbm_bytes_per_launch"])
        algorithmic = float(kv["algorithmic_bytes_per_launch"])
        assert 0.95 < traffic / algorithmic < 1.25
