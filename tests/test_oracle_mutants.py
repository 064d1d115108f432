"""The pins of the oracle catch plausible mistakes in it (CPU only).

Each case plants one mistake in a copy of oracle/afx_oracle.c (a dropped or
misplaced term, a wrong index, a flipped order), builds that copy, and runs
the oracle's pins (tests/test_oracle_pins.py) against it in a child process
that loads it instead of the real oracle. Every planted mistake must make at
least one pin fail; none of these pins consults the GPU library, so each
mutant is caught by what the pages and the mathematics fix (closed forms,
brute force, textbook cases, round trips), not by a second implementation.
"""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "afx_oracle.c")

# (what the mistake is, text in afx_oracle.c, replacement)
MUTANTS = [
    ("package-merge takes 2m-1 items instead of 2m-2",
     "int take = 2 * m - 2;", "int take = 2 * m - 1;"),
    ("package-merge sorts by descending frequency",
     "(freq[sym[j]] > freq[s] || (freq[sym[j]] == freq[s] && sym[j] > s))",
     "(freq[sym[j]] < freq[s] || (freq[sym[j]] == freq[s] && sym[j] > s))"),
    ("canonical codes step by two",
     "c = (c + 1) << (len[order[i]] - len[order[i - 1]]);",
     "c = (c + 2) << (len[order[i]] - len[order[i - 1]]);"),
    ("code bits written LSB first inside each word",
     "uint64_t w = *pos / 32, k = 31 - (*pos % 32);", "uint64_t w = *pos / 32, k = *pos % 32;"),
    ("gaps recorded as absolute positions",
     "uint64_t g = i / OR_GROUP, d = pos - cbase;", "uint64_t g = i / OR_GROUP, d = pos;"),
    ("one mantissa bit dropped from the raw byte",
     "sm_p[i] = (uint8_t)(((h >> 8) & 0x80) | (h & 0x7F));", "sm_p[i] = (uint8_t)(((h >> 8) & 0x80) | (h & 0x3F));"),
    ("the exponent taken one bit too high",
     "uint32_t e = (h >> 7) & 0xFF;", "uint32_t e = (h >> 8) & 0xFF;"),
    ("decoder's first code per length uses the wrong count",
     "code = (code + (uint32_t)d->count[l - 1]) << 1;", "code = (code + (uint32_t)d->count[l]) << 1;"),
    ("sign/mantissa section one byte too late",
     "off[4] = align_up(off[3] + n);", "off[4] = align_up(off[3] + n + 1);"),
    ("two pad words after the stream instead of four",
     "#define OR_PAD_WORDS 4u", "#define OR_PAD_WORDS 2u"),
    ("decoded element puts the exponent one bit too low",
     "out[i] = (uint16_t)(((b & 0x80) << 8) | ((uint32_t)e << 7) | (b & 0x7F));",
     "out[i] = (uint16_t)(((b & 0x80) << 8) | ((uint32_t)e << 6) | (b & 0x7F));"),
]


def test_every_mutation_applies_once():
    text = open(SRC).read()
    for what, old, _ in MUTANTS:
        assert text.count(old) == 1, what


def run_pins(tmp_path, text):
    """Build `text` as the oracle and run the pins against it in a child."""
    src = tmp_path / "afx_oracle_copy.c"
    src.write_text(text)
    lib = tmp_path / "liboracle_copy.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", str(src), "-o", str(lib)],
                   check=True, capture_output=True)
    env = dict(os.environ, AFX_ORACLE_LIB=str(lib))
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x",
                           "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def test_unchanged_copy_passes_the_pins(tmp_path):
    """The control: the same route with the oracle unchanged passes."""
    r = run_pins(tmp_path, open(SRC).read())
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, what, old, new):
    r = run_pins(tmp_path, open(SRC).read().replace(old, new))
    assert r.returncode == 1, f"no pin fails when {what} (exit {r.returncode}):\n{r.stdout[-2000:]}"
    assert " failed" in r.stdout, r.stdout[-2000:]
