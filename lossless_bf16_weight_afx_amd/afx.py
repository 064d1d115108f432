"""Thin ctypes binding of libafx (``include/afx.h``), same names as the C ABI.

Argument marshalling only: every step of the restore runs in the library's
HIP kernels. PyTorch supplies device buffers and streams. If ``libafx.so`` has
not been built, loading raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libafx.so")

AFX_OK = 0
AFX_E_INVALID_ARG = -1
AFX_E_BAD_MAGIC = -2
AFX_E_BAD_VERSION = -3
AFX_E_CORRUPT = -4
AFX_E_BUFFER_TOO_SMALL = -5
AFX_E_MISALIGNED = -6
AFX_E_HIP = -7
AFX_E_UNSUPPORTED = -8
AFX_E_IO = -9
AFX_E_HOST_MEMORY = -10
MAX_JOBS_PER_LAUNCH = 32
AFX_READ_DIRECT = 1

# Every symbol include/afx.h declares.
EXPORTS = ("afx_query", "afx_decode_tensor", "afx_decode_layer_async", "afx_decode_layer_grid_async",
           "afx_status_str",
           "afx_encode_plan", "afx_encode", "afx_file_read", "afx_decode_host",
           "afx_restore_gemv_async", "afx_restore_gemv_batch_async", "afx_restore_gemm_async",
           "afx_restore_gemm_batch_async")


class AfxError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


class afx_info(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32),
        ("format_version", ctypes.c_uint32),
        ("n_elems", ctypes.c_uint64),
        ("decoded_bytes", ctypes.c_uint64),
        ("blob_bytes", ctypes.c_uint64),
        ("total_bits", ctypes.c_uint64),
        ("exp_words", ctypes.c_uint64),
        ("n_chunks", ctypes.c_uint64),
        ("n_groups", ctypes.c_uint64),
        ("ndim", ctypes.c_uint32),
        ("n_symbols", ctypes.c_uint32),
        ("shape", ctypes.c_uint64 * 4),
        ("chunk_elems", ctypes.c_uint32),
        ("group_elems", ctypes.c_uint32),
        ("max_code_len", ctypes.c_uint32),
        ("longest_code", ctypes.c_uint32),
        ("off_code_len", ctypes.c_uint64),
        ("off_chunk_base", ctypes.c_uint64),
        ("off_gap", ctypes.c_uint64),
        ("off_signmant", ctypes.c_uint64),
        ("off_exp", ctypes.c_uint64),
    ]


class afx_gemv_job(ctypes.Structure):
    _fields_ = [
        ("info", ctypes.POINTER(afx_info)),
        ("blob_dev", ctypes.c_void_p),
        ("rows", ctypes.c_uint64),
        ("cols", ctypes.c_uint64),
        ("x_dev", ctypes.c_void_p),
        ("y_dev", ctypes.c_void_p),
    ]


class afx_job(ctypes.Structure):
    _fields_ = [
        ("info", ctypes.POINTER(afx_info)),
        ("blob_dev", ctypes.c_void_p),
        ("out_dev", ctypes.c_void_p),
        ("out_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libafx.so (raises OSError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise OSError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "or python -m lossless_bf16_weight_afx_amd.build")
        L = ctypes.CDLL(_LIB_PATH)
        u8p, u16p, u64p = (ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_uint16),
                           ctypes.POINTER(ctypes.c_uint64))
        L.afx_query.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(afx_info)]
        L.afx_query.restype = ctypes.c_int
        L.afx_decode_tensor.argtypes = [ctypes.POINTER(afx_info), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
        L.afx_decode_tensor.restype = ctypes.c_int
        L.afx_decode_layer_async.argtypes = [ctypes.POINTER(afx_job), ctypes.c_size_t, ctypes.c_void_p]
        L.afx_decode_layer_async.restype = ctypes.c_int
        L.afx_decode_layer_grid_async.argtypes = [ctypes.POINTER(afx_job), ctypes.c_size_t, ctypes.c_uint32,
                                                  ctypes.c_void_p]
        L.afx_decode_layer_grid_async.restype = ctypes.c_int
        L.afx_status_str.argtypes = [ctypes.c_int]
        L.afx_status_str.restype = ctypes.c_char_p
        L.afx_encode_plan.argtypes = [u16p, ctypes.c_uint64, ctypes.c_int, u8p, u64p, u64p]
        L.afx_encode_plan.restype = ctypes.c_int
        L.afx_encode.argtypes = [u16p, ctypes.c_uint64, ctypes.c_uint32, u64p, u8p, ctypes.c_uint64,
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        L.afx_encode.restype = ctypes.c_int
        L.afx_file_read.argtypes = [ctypes.c_char_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_uint]
        L.afx_file_read.restype = ctypes.c_int
        L.afx_decode_host.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        L.afx_decode_host.restype = ctypes.c_int
        L.afx_restore_gemv_async.argtypes = [ctypes.POINTER(afx_info), ctypes.c_void_p, ctypes.c_uint64,
                                             ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p,
                                             ctypes.c_void_p]
        L.afx_restore_gemv_async.restype = ctypes.c_int
        L.afx_restore_gemv_batch_async.argtypes = [ctypes.POINTER(afx_gemv_job), ctypes.c_size_t, ctypes.c_uint32,
                                                   ctypes.c_void_p]
        L.afx_restore_gemv_batch_async.restype = ctypes.c_int
        L.afx_restore_gemm_async.argtypes = L.afx_restore_gemv_async.argtypes
        L.afx_restore_gemm_async.restype = ctypes.c_int
        L.afx_restore_gemm_batch_async.argtypes = L.afx_restore_gemv_batch_async.argtypes
        L.afx_restore_gemm_batch_async.restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().afx_status_str(status).decode()


def _host_bytes(a: np.ndarray, nbytes: int | None) -> tuple[int, int]:
    """Address and size of a blob held in a numpy array; a size given with
    the array may not exceed it (the library would read past its end)."""
    if a.dtype != np.uint8 or not a.flags.c_contiguous:
        raise ValueError("a blob must be a contiguous uint8 array")
    if nbytes is None:
        return a.ctypes.data, a.size
    if not 0 <= int(nbytes) <= a.size:
        raise ValueError(f"blob size {nbytes} outside the array's {a.size} bytes")
    return a.ctypes.data, int(nbytes)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """BF16 bit patterns as a contiguous uint16 array. Only 16-bit integer
    arrays hold them; a cast from any other type would change the bits."""
    x = np.asarray(x)
    if x.dtype not in (np.uint16, np.int16):
        raise TypeError(f"BF16 bit patterns must be uint16 or int16, not {x.dtype}")
    return np.ascontiguousarray(x).view(np.uint16)


def _check(rc: int, what: str) -> None:
    if rc != AFX_OK:
        raise AfxError(rc, what)


# ---------------------------------------------------------------------------
# C entry points
# ---------------------------------------------------------------------------
def afx_query(blob_host, blob_bytes: int | None = None) -> afx_info:
    """Validate a host blob (numpy uint8 array, or an address with a size)."""
    info = afx_info()
    if isinstance(blob_host, np.ndarray):
        ptr, size = _host_bytes(blob_host, blob_bytes)
    else:
        ptr, size = int(blob_host), int(blob_bytes)
    _check(lib().afx_query(ctypes.c_void_p(ptr), size, ctypes.byref(info)), "afx_query")
    return info


def afx_decode_tensor(info: afx_info, blob_dev: int, out_dev: int, out_bytes: int, stream: int = 0) -> None:
    """Restore one tensor; blocks until the stream has finished it."""
    _check(lib().afx_decode_tensor(ctypes.byref(info), ctypes.c_void_p(blob_dev), ctypes.c_void_p(out_dev),
                                   out_bytes, ctypes.c_void_p(stream)), "afx_decode_tensor")


def make_jobs(jobs) -> ctypes.Array:
    """Pack (info, blob_dev, out_dev, out_bytes) tuples into an afx_job array.

    The returned array refers to the afx_info objects; keep them alive.
    """
    arr = (afx_job * len(jobs))()
    for i, (info, blob_dev, out_dev, out_bytes) in enumerate(jobs):
        arr[i].info = ctypes.pointer(info)
        arr[i].blob_dev = blob_dev
        arr[i].out_dev = out_dev
        arr[i].out_bytes = out_bytes
    return arr


def afx_decode_layer_async(jobs, stream: int = 0) -> None:
    """Enqueue the restore of a batch of tensors on `stream`; returns at once.

    ``jobs`` is an afx_job array from make_jobs, or a list of tuples.
    """
    arr = jobs if isinstance(jobs, ctypes.Array) else make_jobs(jobs)
    _check(lib().afx_decode_layer_async(arr, len(arr), ctypes.c_void_p(stream)), "afx_decode_layer_async")


def afx_decode_layer_grid_async(jobs, max_workgroups: int, stream: int = 0) -> None:
    """afx_decode_layer_async on at most ``max_workgroups`` workgroups (CUs)."""
    if not 0 <= int(max_workgroups) < 2 ** 32:
        raise ValueError(f"max_workgroups {max_workgroups} is not a 32-bit unsigned count")
    arr = jobs if isinstance(jobs, ctypes.Array) else make_jobs(jobs)
    _check(lib().afx_decode_layer_grid_async(arr, len(arr), ctypes.c_uint32(max_workgroups), ctypes.c_void_p(stream)),
           "afx_decode_layer_grid_async")


def afx_encode_plan(x: np.ndarray, threads: int = 0):
    """Code lengths (256 u8), stream bits and blob size for BF16 bits x."""
    x = _bf16_bits(x).ravel()
    lens = np.zeros(256, np.uint8)
    bits = ctypes.c_uint64()
    nbytes = ctypes.c_uint64()
    _check(lib().afx_encode_plan(x.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), x.size, threads,
                                 lens.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), ctypes.byref(bits),
                                 ctypes.byref(nbytes)), "afx_encode_plan")
    return lens, bits.value, nbytes.value


def afx_encode(x: np.ndarray, shape=None, threads: int = 0, out=None, plan=None) -> np.ndarray:
    """Encode BF16 bits x into a blob.

    ``out`` may be a numpy uint8 array, or an (address, capacity) pair of
    host memory (e.g. pinned) with room for the planned size; the blob bytes
    are returned as a numpy view when out is an array or None, else the size
    is returned. ``plan`` is a result of afx_encode_plan for the same x.
    """
    x = _bf16_bits(x)
    if shape is None:
        shape = x.shape if x.ndim else (1,)
    x = x.ravel()
    lens, bits, nbytes = plan if plan is not None else afx_encode_plan(x, threads)
    shp = (ctypes.c_uint64 * 4)(*(list(shape) + [0] * (4 - len(shape))))
    if out is None:
        out = np.empty(nbytes, np.uint8)
    if isinstance(out, np.ndarray):
        if out.dtype != np.uint8 or not out.flags.c_contiguous:
            raise ValueError("out must be a contiguous uint8 array")
        addr, cap = out.ctypes.data, out.size
    else:
        addr, cap = int(out[0]), int(out[1])
    _check(lib().afx_encode(x.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), x.size, len(shape), shp,
                            lens.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), bits, ctypes.c_void_p(addr),
                            cap, threads), "afx_encode")
    return out[:nbytes] if isinstance(out, np.ndarray) else nbytes


def afx_restore_gemv_async(info: afx_info, blob_dev: int, rows: int, cols: int, x_dev: int, m: int, y_dev: int,
                           stream: int = 0) -> None:
    """y += W x with W restored on the fly from its device blob (see afx.h)."""
    _check(lib().afx_restore_gemv_async(ctypes.byref(info), ctypes.c_void_p(blob_dev), rows, cols,
                                        ctypes.c_void_p(x_dev), m, ctypes.c_void_p(y_dev), ctypes.c_void_p(stream)),
           "afx_restore_gemv_async")


def make_gemv_jobs(jobs) -> ctypes.Array:
    """Pack (info, blob_dev, rows, cols, x_dev, y_dev) tuples into an
    afx_gemv_job array (which refers to the afx_info objects: keep them)."""
    arr = (afx_gemv_job * len(jobs))()
    for i, (info, blob_dev, rows, cols, x_dev, y_dev) in enumerate(jobs):
        arr[i].info = ctypes.pointer(info)
        arr[i].blob_dev, arr[i].rows, arr[i].cols = blob_dev, rows, cols
        arr[i].x_dev, arr[i].y_dev = x_dev, y_dev
    return arr


def afx_restore_gemv_batch_async(jobs, m: int, stream: int = 0) -> None:
    """y += W x for every job of a batch (array from make_gemv_jobs, or tuples)."""
    arr = jobs if isinstance(jobs, ctypes.Array) else make_gemv_jobs(jobs)
    _check(lib().afx_restore_gemv_batch_async(arr, len(arr), m, ctypes.c_void_p(stream)),
           "afx_restore_gemv_batch_async")


def afx_restore_gemm_async(info: afx_info, blob_dev: int, rows: int, cols: int, x_dev: int, m: int, y_dev: int,
                           stream: int = 0) -> None:
    """y += x W^T with 64-row tiles of W restored into LDS for the matrix
    cores (see afx.h)."""
    _check(lib().afx_restore_gemm_async(ctypes.byref(info), ctypes.c_void_p(blob_dev), rows, cols,
                                        ctypes.c_void_p(x_dev), m, ctypes.c_void_p(y_dev), ctypes.c_void_p(stream)),
           "afx_restore_gemm_async")


def afx_restore_gemm_batch_async(jobs, m: int, stream: int = 0) -> None:
    """afx_restore_gemm_async for every job of a batch (array from
    make_gemv_jobs, or tuples)."""
    arr = jobs if isinstance(jobs, ctypes.Array) else make_gemv_jobs(jobs)
    _check(lib().afx_restore_gemm_batch_async(arr, len(arr), m, ctypes.c_void_p(stream)),
           "afx_restore_gemm_batch_async")


def afx_decode_host(blob, blob_bytes: int | None = None, out=None, threads: int = 0):
    """Restore a host blob on the host (the pages' placement of the unpack).

    ``blob`` is a numpy uint8 array or an address (with blob_bytes); ``out``
    a numpy uint16 array, an (address, capacity) pair, or None (allocated).
    Returns the uint16 array, or None when out is an address pair."""
    if isinstance(blob, np.ndarray):
        addr, size = _host_bytes(blob, blob_bytes)
    else:
        addr, size = int(blob), int(blob_bytes)
    if out is None:
        out = np.empty(int(afx_query(addr, size).n_elems), np.uint16)
    if isinstance(out, np.ndarray):
        if out.dtype != np.uint16 or not out.flags.c_contiguous:
            raise ValueError("out must be a contiguous uint16 array")
        oaddr, cap = out.ctypes.data, 2 * out.size
    else:
        oaddr, cap = int(out[0]), int(out[1])
    _check(lib().afx_decode_host(ctypes.c_void_p(addr), size, ctypes.c_void_p(oaddr), cap, threads), "afx_decode_host")
    return out if isinstance(out, np.ndarray) else None


def afx_file_read(path: str, offset: int, nbytes: int, dst: int, threads: int = 0, direct: bool = True) -> None:
    """Read nbytes at offset of the file into host memory at address dst."""
    _check(lib().afx_file_read(os.fsencode(path), offset, nbytes, ctypes.c_void_p(dst), threads,
                               AFX_READ_DIRECT if direct else 0), "afx_file_read")


# ---------------------------------------------------------------------------
# torch conveniences (buffers and streams only)
# ---------------------------------------------------------------------------
def to_device(blob: np.ndarray, device="cuda"):
    """Copy a host blob into a fresh uint8 device tensor (256-byte aligned)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(blob)).to(device)


def decode(info: afx_info, blob_dev, out=None, stream=None):
    """Restore into a torch int16 device tensor (bit patterns of BF16)."""
    import torch

    if out is None:
        out = torch.empty(int(info.n_elems), dtype=torch.int16, device=blob_dev.device)
    s = stream if stream is not None else torch.cuda.current_stream(blob_dev.device)
    afx_decode_tensor(info, blob_dev.data_ptr(), out.data_ptr(), out.numel() * out.element_size(), s.cuda_stream)
    return out
