"""The storage step on the CPU: the store file, the native reader, and the
oracle restoring what was read back.

Expected values are the generated weights themselves; the oracle decoder
(pinned in test_oracle_pins.py) restores them from the bytes afx_file_read
returns. Nothing here needs a GPU.
"""
import os

import numpy as np
import pytest

import oracle
from lossless_bf16_weight_afx_amd import afx, store, synth

T = synth.TensorSpec


def small_units():
    return [
        [T("u0.w", (300, 517), "normal", 31), T("u0.norm", (5120,), "normal", 32, 1.0, 0.05)],
        [T("u1.w", (64, 4096), "t4", 33)],
        [T("u2.a", (77, 33), "normal", 34), T("u2.b", (4097,), "normal", 35), T("u2.c", (128,), "normal", 36, 1.0, 0.05)],
    ]


def aligned(nbytes):
    raw = np.zeros(nbytes + store.PAGE, np.uint8)
    off = (-raw.ctypes.data) % store.PAGE
    return raw[off:off + nbytes]


def direct_supported(path):
    try:
        fd = os.open(path, os.O_RDONLY | os.O_DIRECT)
    except OSError:
        return False
    os.close(fd)
    return True


@pytest.fixture(scope="module")
def written(tmp_path_factory):
    afx.lib()
    path = str(tmp_path_factory.mktemp("store") / "model.afxs")
    st = store.write_store(path, small_units(), threads=4)
    return path, st


def test_layout(written):
    path, st = written
    again = store.open_store(path)
    assert again.units == st.units
    assert again.file_bytes == os.path.getsize(path)
    prev_end = store.PAGE
    for u, specs in zip(again.units, small_units()):
        assert u.offset == prev_end and u.offset % store.PAGE == 0 and u.bytes % store.PAGE == 0
        assert [t.name for t in u.tensors] == [sp.name for sp in specs]
        assert [t.shape for t in u.tensors] == [tuple(sp.shape) for sp in specs]
        for t in u.tensors:
            assert t.offset % store.BLOB_ALIGN == 0 and t.offset + t.bytes <= u.bytes
        prev_end = u.offset + u.bytes


@pytest.mark.parametrize("direct", [False, True])
def test_read_back_and_restore(written, direct):
    path, st = written
    if direct and not direct_supported(path):
        pytest.skip("file system refuses O_DIRECT")
    for u, specs in zip(st.units, small_units()):
        buf = aligned(u.bytes)
        afx.afx_file_read(path, u.offset, u.bytes, buf.ctypes.data, threads=3, direct=direct)
        for t, sp in zip(u.tensors, specs):
            blob = np.ascontiguousarray(buf[t.offset:t.offset + t.bytes])
            info = afx.afx_query(blob)
            assert int(info.n_elems) == int(np.prod(sp.shape))
            assert np.array_equal(oracle.decode(blob, threads=2), synth.generate(sp).ravel()), t.name


def test_reader_pieces_and_threads(tmp_path):
    data = np.random.default_rng(5).integers(0, 256, (9 << 20) + 4096 * 3, dtype=np.uint8)
    p = str(tmp_path / "f.bin")
    data.tofile(p)
    for threads in (1, 2, 7):
        buf = aligned(data.size - 4096)
        afx.afx_file_read(p, 4096, buf.size, buf.ctypes.data, threads=threads, direct=False)
        assert np.array_equal(buf, data[4096:])


def test_reader_unaligned_ranges(tmp_path):
    """Any offset, size and destination, direct or not: the bytes asked for
    and nothing around them."""
    data = np.random.default_rng(6).integers(0, 256, (9 << 20) + 12345, dtype=np.uint8)
    p = str(tmp_path / "g.bin")
    data.tofile(p)
    modes = [False, True] if direct_supported(p) else [False]
    for direct in modes:
        for off, n in [(0, 1), (1, 4095), (4095, 2), (4097, (4 << 20) + 3), (12345, data.size - 12345),
                       (data.size - 7, 7), ((4 << 20) - 1, (4 << 20) + 2)]:
            buf = np.full(n + 16, 0xAB, np.uint8)
            afx.afx_file_read(p, off, n, buf.ctypes.data + 5, threads=3, direct=direct)
            assert np.array_equal(buf[5:5 + n], data[off:off + n]), (direct, off, n)
            assert np.all(buf[:5] == 0xAB) and np.all(buf[5 + n:] == 0xAB), (direct, off, n)


def test_reader_errors(tmp_path):
    p = str(tmp_path / "f.bin")
    np.zeros(3 * 4096, np.uint8).tofile(p)
    buf = aligned(4 * 4096)
    with pytest.raises(afx.AfxError) as e:
        afx.afx_file_read(p + ".missing", 0, 4096, buf.ctypes.data, direct=False)
    assert e.value.status == afx.AFX_E_IO
    with pytest.raises(afx.AfxError) as e:
        afx.afx_file_read(p, 2 * 4096, 2 * 4096, buf.ctypes.data, direct=False)  # past the end
    assert e.value.status == afx.AFX_E_IO
    if direct_supported(p):
        with pytest.raises(afx.AfxError) as e:
            afx.afx_file_read(p, 2 * 4096 + 100, 4096, buf.ctypes.data, direct=True)  # past the end
        assert e.value.status == afx.AFX_E_IO
    rc = afx.lib().afx_file_read(p.encode(), 0, 4096, buf.ctypes.data, 1, 6)
    assert rc == afx.AFX_E_INVALID_ARG
    rc = afx.lib().afx_file_read(None, 0, 4096, buf.ctypes.data, 1, 0)
    assert rc == afx.AFX_E_INVALID_ARG
    afx.afx_file_read(p, 0, 0, buf.ctypes.data, direct=True)  # empty range: nothing to do


def test_bad_store_files(written, tmp_path):
    path, st = written
    raw = open(path, "rb").read()
    bad = tmp_path / "bad.afxs"
    bad.write_bytes(b"XXXX" + raw[4:])
    with pytest.raises(ValueError):
        store.open_store(str(bad))
    bad.write_bytes(raw[:-10])
    with pytest.raises(ValueError):
        store.open_store(str(bad))
