"""The C ABI on the CPU: symbols, blob validation, argument errors, encoder.

No GPU here: only calls that fail before any HIP call, and host-side code.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from conftest import ROOT
from lossless_bf16_weight_afx_amd import afx, synth


@pytest.fixture(scope="module")
def L():
    return afx.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "afx.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(afx_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol(L):
    declared = header_functions()
    assert set(declared) == set(afx.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert afx.status_str(afx.AFX_E_CORRUPT).startswith("corrupt")


def c1_blob():
    x = synth.generate(synth.TensorSpec("t", (3 * 4096 + 100,), "normal", 21))
    return x, oracle.encode(x)


def test_query_reports_layout(L):
    x, blob = c1_blob()
    info = afx.afx_query(blob)
    s = oracle.sections(blob)
    off = s["offsets"]
    assert info.n_elems == x.size and info.decoded_bytes == 2 * x.size
    assert info.blob_bytes == blob.size == off["blob_bytes"]
    assert (info.off_code_len, info.off_chunk_base, info.off_gap, info.off_signmant, info.off_exp) == (
        off["code_len"], off["chunk_base"], off["gap"], off["signmant"], off["exp"])
    assert info.n_chunks == 4 and info.n_groups == -(-x.size // 32)
    assert info.total_bits == s["header"]["total_bits"] and info.exp_words == s["header"]["exp_words"]
    assert info.max_code_len == 12 and info.longest_code == s["code_len"].max()
    assert info.ndim == 1 and info.shape[0] == x.size


def expect(status, blob, size=None):
    with pytest.raises(afx.AfxError) as e:
        afx.afx_query(blob, size)
    assert e.value.status == status


def test_query_rejects_bad_blobs(L):
    _, blob = c1_blob()
    assert L.afx_query(None, 0, None) == afx.AFX_E_INVALID_ARG
    expect(afx.AFX_E_BUFFER_TOO_SMALL, blob[:300].copy())
    expect(afx.AFX_E_BUFFER_TOO_SMALL, blob[:-256].copy())
    b = blob.copy(); b[0] = ord("B"); expect(afx.AFX_E_BAD_MAGIC, b)
    b = blob.copy(); b[4] = 2; expect(afx.AFX_E_BAD_VERSION, b)
    b = blob.copy(); b[44] = 16; expect(afx.AFX_E_BAD_VERSION, b)
    s = oracle.sections(blob)
    lens = s["code_len"]
    # a code length above the limit
    b = blob.copy(); b[256 + int(np.argmax(lens))] = 13; expect(afx.AFX_E_CORRUPT, b)
    # break Kraft equality: shorten the longest code by one bit
    b = blob.copy(); i = int(np.argmax(lens)); b[256 + i] = lens[i] - 1; expect(afx.AFX_E_CORRUPT, b)
    # a gap that does not start its chunk at 0
    b = blob.copy(); g = oracle.sections(b)["gap"]; g[128] = 3; expect(afx.AFX_E_CORRUPT, b)
    # gaps that go backwards
    b = blob.copy(); g = oracle.sections(b)["gap"]; g[5] = g[4] - 1; expect(afx.AFX_E_CORRUPT, b)
    # chunk bases that do not end at total_bits
    b = blob.copy(); cb = oracle.sections(b)["chunk_base"]; cb[-1] += 1; expect(afx.AFX_E_CORRUPT, b)
    # n that disagrees with the shape
    b = blob.copy(); b[64] ^= 1; expect(afx.AFX_E_CORRUPT, b)


def test_query_accepts_edge_blobs(L):
    for x in (np.zeros(0, np.uint16), np.zeros(1, np.uint16), np.full(4097, 0x3F80, np.uint16),
              np.arange(65536, dtype=np.uint16)):
        info = afx.afx_query(oracle.encode(x))
        assert info.n_elems == x.size


def test_decode_argument_errors_before_any_hip_call(L):
    _, blob = c1_blob()
    info = afx.afx_query(blob)
    fake_dev = 0x10000  # never dereferenced: every case fails validation first
    n = info.n_elems
    assert L.afx_decode_tensor(None, fake_dev, fake_dev * 4, 2 * n, None) == afx.AFX_E_INVALID_ARG
    assert L.afx_decode_tensor(ctypes.byref(info), None, fake_dev * 4, 2 * n, None) == afx.AFX_E_INVALID_ARG
    assert L.afx_decode_tensor(ctypes.byref(info), fake_dev, None, 2 * n, None) == afx.AFX_E_INVALID_ARG
    assert L.afx_decode_tensor(ctypes.byref(info), fake_dev, fake_dev * 4, 2 * n - 1, None) == \
        afx.AFX_E_BUFFER_TOO_SMALL
    assert L.afx_decode_tensor(ctypes.byref(info), fake_dev + 8, fake_dev * 4, 2 * n, None) == afx.AFX_E_MISALIGNED
    assert L.afx_decode_tensor(ctypes.byref(info), fake_dev, fake_dev * 4 + 2, 2 * n, None) == afx.AFX_E_MISALIGNED
    # output overlapping the blob
    assert L.afx_decode_tensor(ctypes.byref(info), fake_dev, fake_dev + 256, 2 * n, None) == afx.AFX_E_INVALID_ARG
    # an afx_info that was tampered with
    bad = afx.afx_info.from_buffer_copy(info); bad.off_exp += 256
    assert L.afx_decode_tensor(ctypes.byref(bad), fake_dev, fake_dev * 4, 2 * n, None) == afx.AFX_E_CORRUPT
    bad = afx.afx_info.from_buffer_copy(info); bad.abi_version = 99
    assert L.afx_decode_tensor(ctypes.byref(bad), fake_dev, fake_dev * 4, 2 * n, None) == afx.AFX_E_BAD_VERSION
    # batches: one bad job rejects the whole batch before anything is enqueued
    jobs = afx.make_jobs([(info, fake_dev, fake_dev * 4, 2 * n), (info, fake_dev, fake_dev * 8 + 2, 2 * n)])
    assert L.afx_decode_layer_async(jobs, 2, None) == afx.AFX_E_MISALIGNED
    assert L.afx_decode_layer_async(None, 3, None) == afx.AFX_E_INVALID_ARG
    assert L.afx_decode_layer_async(None, 0, None) == afx.AFX_OK
    # jobs of one call run in one launch: an output may share no byte with
    # another job's output or blob
    out_b = fake_dev * 8
    jobs = afx.make_jobs([(info, fake_dev, fake_dev * 4, 2 * n), (info, fake_dev * 4 + 4096, out_b, 2 * n)])
    assert L.afx_decode_layer_async(jobs, 2, None) == afx.AFX_E_INVALID_ARG  # job 0 writes job 1's blob
    jobs = afx.make_jobs([(info, fake_dev, fake_dev * 4, 2 * n), (info, fake_dev, fake_dev * 4 + 4096, 2 * n)])
    assert L.afx_decode_layer_async(jobs, 2, None) == afx.AFX_E_INVALID_ARG  # outputs overlap
    jobs = afx.make_jobs([(info, fake_dev, fake_dev * 8, 2 * n), (info, fake_dev, fake_dev * 12, 2 * n),
                          (info, fake_dev * 12, fake_dev * 16, 2 * n)])
    assert L.afx_decode_layer_async(jobs, 3, None) == afx.AFX_E_INVALID_ARG  # job 2's blob is job 1's output
    # the grid-capped batch: a zero cap, then the same checks as the batch call
    assert L.afx_decode_layer_grid_async(None, 0, 0, None) == afx.AFX_E_INVALID_ARG
    assert L.afx_decode_layer_grid_async(None, 0, 1, None) == afx.AFX_OK
    assert L.afx_decode_layer_grid_async(jobs, 3, 8, None) == afx.AFX_E_INVALID_ARG
    jobs = afx.make_jobs([(info, fake_dev, fake_dev * 4, 2 * n), (info, fake_dev, fake_dev * 8 + 2, 2 * n)])
    assert L.afx_decode_layer_grid_async(jobs, 2, 64, None) == afx.AFX_E_MISALIGNED
    with pytest.raises(ValueError):  # the binding refuses a cap that is no 32-bit count
        afx.afx_decode_layer_grid_async(jobs, -1)
    with pytest.raises(afx.AfxError) as e:
        afx.afx_decode_layer_grid_async(jobs, 0)
    assert e.value.status == afx.AFX_E_INVALID_ARG



def test_batch_overlap_check_matches_brute_force(L):
    """Random batches of up to 40 jobs over a small address range: the
    library rejects a batch exactly when some output shares a byte with
    another output or with any blob. A batch that passes the check goes on to
    the launch, which fails here for want of a GPU (never a device access:
    the test is skipped where a GPU is present, since the addresses are
    made up)."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("made-up device addresses must not reach a launch")
    x, blob = c1_blob()
    info = afx.afx_query(blob)
    n, nb = int(info.n_elems), int(info.blob_bytes)
    rng = np.random.default_rng(5)
    base, unit = 1 << 40, 4096
    seen = {True: 0, False: 0}
    for trial in range(400):
        k = int(rng.integers(2, 41))
        span = int(rng.integers(4, 12)) * k  # address slots of `unit` bytes
        blobs = [base + unit * int(rng.integers(0, span)) for _ in range(k)]
        outs = [base + unit * int(rng.integers(0, span)) for _ in range(k)]
        if trial % 2 == 0:  # disjoint outputs far from the blobs, or one planted overlap
            outs = [base + (1 << 36) + i * 2 * (2 * n + unit) for i in range(k)]
            if trial % 4 == 0:
                outs[int(rng.integers(k))] = blobs[int(rng.integers(k))] + 16 * int(rng.integers(0, 4))
        def hit(a0, a1, b0, b1):
            return a0 < b1 and b0 < a1
        want = any(hit(outs[i], outs[i] + 2 * n, outs[j], outs[j] + 2 * n) for i in range(k) for j in range(i))
        want |= any(hit(outs[i], outs[i] + 2 * n, blobs[j], blobs[j] + nb) for i in range(k) for j in range(k))
        jobs = afx.make_jobs([(info, b, o, 2 * n) for b, o in zip(blobs, outs)])
        rc = L.afx_decode_layer_async(jobs, k, None)
        assert (rc == afx.AFX_E_INVALID_ARG) == want, (trial, rc)
        seen[want] += 1
    assert min(seen.values()) > 80, seen
    # past 1024 jobs the ranges go to the heap: same answers
    k = 1100
    blobs = [base + i * 2 * (nb + unit) for i in range(k)]
    outs = [base + (1 << 36) + i * 2 * (2 * n + unit) for i in range(k)]
    jobs = afx.make_jobs([(info, b, o, 2 * n) for b, o in zip(blobs, outs)])
    assert L.afx_decode_layer_async(jobs, k, None) != afx.AFX_E_INVALID_ARG
    outs[k - 1] = blobs[3] + 16
    jobs = afx.make_jobs([(info, b, o, 2 * n) for b, o in zip(blobs, outs)])
    assert L.afx_decode_layer_async(jobs, k, None) == afx.AFX_E_INVALID_ARG

# ---------------------------------------------------------------------------
# The library's own encoder: its blobs must satisfy the oracle decoder and
# its code must be as short as the oracle's optimum.
# ---------------------------------------------------------------------------
ENC_CASES = [
    ("normal", (1000, 33)), ("normal", (4096,)), ("normal", (1,)), ("t4", (257, 4096)),
    ("normal", (5, 4096 + 7)),
]


@pytest.mark.parametrize("dist,shape", ENC_CASES)
def test_encoder_blob_decodes_with_oracle(dist, shape):
    spec = synth.TensorSpec("t", shape, dist, 31)
    x = synth.generate(spec)
    blob1 = afx.afx_encode(x, shape, threads=1)
    blob8 = afx.afx_encode(x, shape, threads=8)
    assert np.array_equal(blob1, blob8)
    assert np.array_equal(oracle.decode(blob1), x)
    assert np.array_equal(oracle.decode(blob1, threads=4), x)
    ob = oracle.encode(x, shape)
    lo, hi = oracle.sections(ob), oracle.sections(blob1)
    # equal total code length: both are optimal under the 12-bit limit
    assert lo["header"]["total_bits"] == hi["header"]["total_bits"]
    if np.array_equal(lo["code_len"], hi["code_len"]):
        assert np.array_equal(ob, blob1)
    info = afx.afx_query(blob1)
    assert info.n_elems == x.size


def test_encoder_special_tensors():
    for x in (np.zeros(77, np.uint16), np.arange(65536, dtype=np.uint16),
              np.array([0x7FC1, 0xFF80, 0x0001, 0x8000] * 1000, np.uint16)):
        b = afx.afx_encode(x)
        assert np.array_equal(oracle.decode(b), x)
        assert np.array_equal(b, oracle.encode(x))  # the optimum is unique here


def test_encoder_lengths_match_oracle_optimum_on_random_histograms():
    rng = np.random.default_rng(5)
    for _ in range(20):
        m = int(rng.integers(2, 60))
        syms = rng.choice(256, size=m, replace=False)
        counts = (rng.pareto(0.6, size=m) * 50 + 1).astype(np.int64)
        x = np.repeat(syms.astype(np.uint16) << 7, counts)
        rng.shuffle(x)
        lo = oracle.sections(oracle.encode(x))["header"]["total_bits"]
        hi = oracle.sections(afx.afx_encode(x))["header"]["total_bits"]
        assert lo == hi


def test_encoder_rejects_bad_plans():
    """afx_encode refuses lengths that are not a complete prefix code, a
    shape whose product is not n (also when the product wraps), a wrong
    stream length and a buffer below the blob size; every refusal is an
    error status, never a blob that afx_query would reject."""
    rng = np.random.default_rng(8)
    x = rng.integers(0, 1 << 16, size=5000, dtype=np.uint16)
    lens, bits, nbytes = afx.afx_encode_plan(x)

    def status(lens=lens, bits=bits, shape=(5000,), cap=nbytes):
        with pytest.raises(afx.AfxError) as e:
            afx.afx_encode(x, shape, out=np.empty(cap, np.uint8), plan=(lens, bits, nbytes))
        return e.value.status

    short = lens.copy()
    short[np.flatnonzero(short)[0]] += 1  # Kraft sum below 1: not complete
    assert status(lens=short) == afx.AFX_E_INVALID_ARG
    over = lens.copy()
    k = np.flatnonzero(over == over.max())[0]
    over[k] -= 1  # Kraft sum above 1: not a prefix code
    assert status(lens=over) == afx.AFX_E_INVALID_ARG
    missing = lens.copy()
    missing[(int(x[0]) >> 7) & 0xFF] = 0  # an exponent of x without a code
    assert status(lens=missing) == afx.AFX_E_INVALID_ARG
    assert status(bits=bits + 1) == afx.AFX_E_INVALID_ARG
    assert status(shape=(50, 101)) == afx.AFX_E_INVALID_ARG
    assert status(shape=((1 << 62) + 1250, 4)) == afx.AFX_E_INVALID_ARG  # 2^64 + 5000 wraps to 5000
    assert status(cap=nbytes - 1) == afx.AFX_E_BUFFER_TOO_SMALL
    one = np.zeros(256, np.uint8)
    one[3] = 2  # a single symbol must take length 1
    y = np.full(10, 3 << 7, np.uint16)
    with pytest.raises(afx.AfxError) as e:
        afx.afx_encode(y, plan=(one, 20, 1 << 12))
    assert e.value.status == afx.AFX_E_INVALID_ARG
    assert np.array_equal(oracle.decode(afx.afx_encode(x, (50, 100))), x)  # the plan itself is fine


def test_binding_refuses_sizes_past_the_array():
    """A size given with a numpy blob may not exceed the array: the library
    would read past its end. Wrong dtypes are refused too."""
    x, blob = c1_blob()
    with pytest.raises(ValueError):
        afx.afx_query(blob, blob.size + 1)
    with pytest.raises(ValueError):
        afx.afx_query(blob.view(np.int8))
    with pytest.raises(ValueError):
        afx.afx_decode_host(blob, blob.size + 64)
    with pytest.raises(ValueError):
        afx.afx_decode_host(blob, out=np.empty(x.size, np.int16))
    assert afx.afx_query(blob, blob.size).n_elems == x.size


def test_encoder_takes_only_16_bit_patterns():
    """The encoder's input is BF16 bit patterns: uint16 or int16 (same bits);
    any other type is refused rather than cast."""
    x = synth.generate(synth.TensorSpec("t", (5000,), "normal", 4))
    assert np.array_equal(afx.afx_encode(x.view(np.int16)), afx.afx_encode(x))
    with pytest.raises(TypeError):
        afx.afx_encode(x.astype(np.float32))
    with pytest.raises(TypeError):
        afx.afx_encode_plan(x.astype(np.int32))


def test_every_status_has_its_own_text(tmp_path):
    codes = [v for k, v in vars(afx).items() if k.startswith("AFX_E_")]
    assert afx.AFX_E_HOST_MEMORY in codes
    texts = [afx.status_str(c) for c in codes]
    assert "unknown status" not in texts and len(set(texts)) == len(codes)
    # a byte range whose end does not fit a file offset is refused before any read
    p = tmp_path / "f.bin"
    p.write_bytes(b"x" * 64)
    dst = np.empty(16, np.uint8)
    for off, n in (((1 << 63) - 8, 16), (1 << 63, 1), (8, (1 << 64) - 4)):
        with pytest.raises(afx.AfxError) as e:
            afx.afx_file_read(str(p), off, n, dst.ctypes.data, direct=False)
        assert e.value.status == afx.AFX_E_INVALID_ARG
