"""Damaged copies of a blob, as a stale or corrupted device copy might
hold them, for the GPU tests of the promise that such a copy decodes to wrong
bits and never reads or writes out of bounds (the index arithmetic behind it
is checked on the CPU by test_index_bounds.py). Only the oracle's section
layout is used; no arithmetic of the method."""
import numpy as np

import oracle

KINDS = ("bases", "gaps", "words", "lengths", "all")


def damage(blob: np.ndarray, what: str, rng) -> np.ndarray:
    """A copy of blob with one section damaged as a stale or corrupted
    device copy might be: random bit flips (high bits included) in the chunk
    bases, random gaps, random code words, random code lengths (0..255), or
    all of them at once."""
    s = oracle.sections(blob)["offsets"]
    n_chunks = -(-int(oracle.sections(blob)["header"]["n"]) // 4096)
    c = blob.copy()

    def flip(lo, hi, k):
        idx = rng.integers(lo, hi, k)
        c[idx] ^= (np.uint8(1) << rng.integers(0, 8, k).astype(np.uint8))

    if what in ("bases", "all"):
        flip(s["chunk_base"], s["chunk_base"] + 8 * (n_chunks + 1), max(4, n_chunks))
    if what in ("gaps", "all"):
        lo, hi = s["gap"], s["signmant"]
        c[lo:hi] = rng.integers(0, 256, hi - lo, dtype=np.uint8)
    if what in ("words", "all"):
        lo, hi = s["exp"], s["blob_bytes"]
        c[lo:hi] = rng.integers(0, 256, hi - lo, dtype=np.uint8)
    if what in ("lengths", "all"):
        c[s["code_len"]:s["code_len"] + 256] = rng.integers(0, 256, 256, dtype=np.uint8)
    return c
