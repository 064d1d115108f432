"""Python handle on the plain C oracle (``afx_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does. It shares no code with the GPU library.

The oracle restates the lossless exponent coding of "Why Weight Offloading
Slows Inference" (section "Lossless compression: fewer bytes to read, more
work to unpack"; Huffman's minimum-redundancy code is that page's reference
[2]). See ``afx_oracle.c`` for the readings it takes where the pages are
silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "afx_oracle.c")
# AFX_ORACLE_LIB names another build of afx_oracle.c to load instead (the
# mutation check of the pins loads deliberately broken copies this way)
_LIB = os.environ.get("AFX_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

LMAX = 12
CHUNK = 4096
GROUP = 32

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u64p = ctypes.POINTER(ctypes.c_uint64)


def build() -> str:
    """Compile the oracle with gcc (plain C11, pthreads)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
           _SRC, "-o", _LIB + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            if "AFX_ORACLE_LIB" in os.environ:
                raise OSError(f"AFX_ORACLE_LIB names {_LIB}, which does not exist")
            build()
        L = ctypes.CDLL(_LIB)
        L.afx_oracle_layout.argtypes = [ctypes.c_uint64, ctypes.c_uint64, _u64p]
        L.afx_oracle_blob_bytes.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.afx_oracle_blob_bytes.restype = ctypes.c_uint64
        L.afx_oracle_code_lengths.argtypes = [_u64p, ctypes.c_int, ctypes.c_int, _u8p]
        L.afx_oracle_plan.argtypes = [_u16p, ctypes.c_uint64, ctypes.c_int, _u8p, _u64p]
        L.afx_oracle_encode.argtypes = [_u16p, ctypes.c_uint64, ctypes.c_uint32, _u64p, _u8p,
                                        ctypes.c_uint64, _u8p, ctypes.c_uint64]
        L.afx_oracle_decode.argtypes = [_u8p, ctypes.c_uint64, _u16p, ctypes.c_uint64, ctypes.c_int]
        L.afx_oracle_decode_chunks.argtypes = [_u8p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                               _u16p, ctypes.c_uint64, ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what} failed with status {rc}")


def code_lengths(freq, lmax: int = LMAX) -> np.ndarray:
    """Optimal length-limited prefix-code lengths by package-merge."""
    f = np.ascontiguousarray(freq, dtype=np.uint64)
    out = np.zeros(f.size, np.uint8)
    _check(lib().afx_oracle_code_lengths(_ptr(f, _u64p), f.size, lmax, _ptr(out, _u8p)), "code_lengths")
    return out


def canonical_codes(lengths) -> np.ndarray:
    """Canonical code of each symbol: (length, value) order, consecutive codes.

    Pure Python restatement used by the pins (the C encoder has its own).
    """
    lengths = [int(v) for v in lengths]
    order = sorted((l, s) for s, l in enumerate(lengths) if l > 0)
    codes = np.zeros(len(lengths), np.uint32)
    c = 0
    for i, (l, s) in enumerate(order):
        if i:
            c = (c + 1) << (l - order[i - 1][0])
        codes[s] = c
    return codes


def layout(n: int, total_bits: int) -> dict:
    off = np.zeros(6, np.uint64)
    lib().afx_oracle_layout(n, total_bits, _ptr(off, _u64p))
    keys = ("code_len", "chunk_base", "gap", "signmant", "exp", "blob_bytes")
    return {k: int(v) for k, v in zip(keys, off)}


def plan(x: np.ndarray, lmax: int = LMAX):
    """Code lengths (256) and total stream bits for the tensor's exponents."""
    x = np.ascontiguousarray(x, dtype=np.uint16).ravel()
    lens = np.zeros(256, np.uint8)
    bits = np.zeros(1, np.uint64)
    _check(lib().afx_oracle_plan(_ptr(x, _u16p), x.size, lmax, _ptr(lens, _u8p), _ptr(bits, _u64p)), "plan")
    return lens, int(bits[0])


def encode(x: np.ndarray, shape=None, lmax: int = LMAX, out: np.ndarray | None = None) -> np.ndarray:
    """Encode BF16 bit patterns (uint16) into a blob (uint8 array)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if shape is None:
        shape = x.shape if x.ndim else (1,)
    x = x.ravel()
    shp = np.array(list(shape) + [0] * (4 - len(shape)), np.uint64)
    lens, bits = plan(x, lmax)
    nbytes = int(lib().afx_oracle_blob_bytes(x.size, bits))
    if out is None:
        out = np.empty(nbytes, np.uint8)
    assert out.dtype == np.uint8 and out.size >= nbytes
    rc = lib().afx_oracle_encode(_ptr(x, _u16p), x.size, len(shape), _ptr(shp, _u64p), _ptr(lens, _u8p),
                                 bits, _ptr(out, _u8p), nbytes)
    _check(rc, "encode")
    return out[:nbytes]


def decode(blob: np.ndarray, threads: int = 1) -> np.ndarray:
    """Restore the BF16 bit patterns (flat uint16) from a blob.

    threads <= 1: one sequential pass over the whole stream; otherwise each
    chunk is decoded independently from its recorded start, chunks spread
    over ``threads`` POSIX threads.
    """
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    n = int(header(blob)["n"])
    out = np.empty(n, np.uint16)
    _check(lib().afx_oracle_decode(_ptr(blob, _u8p), blob.size, _ptr(out, _u16p), n, threads), "decode")
    return out


def decode_chunks(blob: np.ndarray, c0: int, c1: int, out: np.ndarray | None = None, threads: int = 1) -> np.ndarray:
    """Restore the elements of chunks [c0, c1) only."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    n = int(header(blob)["n"])
    e0, e1 = c0 * CHUNK, min(c1 * CHUNK, n)
    if out is None:
        out = np.empty(max(e1 - e0, 0), np.uint16)
    _check(lib().afx_oracle_decode_chunks(_ptr(blob, _u8p), blob.size, c0, c1, _ptr(out, _u16p),
                                          out.size, threads), "decode_chunks")
    return out


def header(blob: np.ndarray) -> dict:
    """Header fields of a blob, read with plain little-endian views."""
    b = np.ascontiguousarray(blob[:256], dtype=np.uint8)
    u32 = b[:64].view("<u4")
    u64 = b[:96].view("<u8")
    ndim = int(u32[8])
    return {
        "magic": bytes(b[:4]),
        "version": int(u32[1]),
        "n": int(u64[1]),
        "total_bits": int(u64[2]),
        "exp_words": int(u64[3]),
        "ndim": ndim,
        "chunk": int(u32[9]),
        "group": int(u32[10]),
        "lmax": int(u32[11]),
        "n_symbols": int(u32[12]),
        "shape": tuple(int(v) for v in u64[8:8 + ndim]),
    }


def sections(blob: np.ndarray) -> dict:
    """Views of every blob section (for pins that inspect the layout)."""
    h = header(blob)
    n, bits = h["n"], h["total_bits"]
    off = layout(n, bits)
    n_chunks = -(-n // CHUNK)
    n_groups = -(-n // GROUP)
    return {
        "code_len": blob[off["code_len"]:off["code_len"] + 256],
        "chunk_base": blob[off["chunk_base"]:off["chunk_base"] + 8 * (n_chunks + 1)].view("<u8"),
        "gap": blob[off["gap"]:off["gap"] + 2 * n_groups].view("<u2"),
        "signmant": blob[off["signmant"]:off["signmant"] + n],
        "exp": blob[off["exp"]:off["exp"] + 4 * h["exp_words"]].view("<u4"),
        "offsets": off,
        "header": h,
    }


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns as float64 values (a BF16 value is the float32 whose
    upper 16 bits are its pattern)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def restore_gemv(blob: np.ndarray, rows: int, cols: int, x_bits: np.ndarray, threads: int = 1, y0=None):
    """y = y0 + W x in float64 for the matrix W that the blob restores
    (row-major [rows, cols]), BF16 activations x [m, cols] and a starting y0
    [m, rows] (zero when None); also the bound that FP32 summation of those
    terms in any order stays within. Summing k values in floating point with
    unit roundoff u, in any order, errs by at most gamma_(k-1) times the sum of
    their magnitudes, gamma_j = j u / (1 - j u) (the classical error bound of
    recursive and pairwise summation); here u = 2^-24, the products of two
    BF16 values are exact in FP32, and k = cols (+ 1 with y0). The restore is
    this module's decoder; the product is numpy's.
    Returns (y [m, rows], bound [m, rows])."""
    w = bf16_to_f64(decode(blob, threads=threads)).reshape(rows, cols)
    x = bf16_to_f64(x_bits).reshape(-1, cols)
    y = x @ w.T
    mag = np.abs(x) @ np.abs(w).T
    k = cols
    if y0 is not None:
        y0 = np.asarray(y0, dtype=np.float64).reshape(y.shape)
        y = y + y0
        mag = mag + np.abs(y0)
        k += 1
    j = (k - 1) * 2.0 ** -24
    bound = j / (1.0 - j) * mag
    return y, bound
