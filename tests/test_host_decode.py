"""The host-placed unpack (afx_decode_host) against the original bits and the
oracle decoder. CPU only."""
import numpy as np
import pytest

import oracle
from lossless_bf16_weight_afx_amd import afx, synth


@pytest.fixture(scope="module", autouse=True)
def lib():
    return afx.lib()


@pytest.mark.parametrize("n", [1, 31, 32, 33, 255, 256, 257, 4095, 4096, 4097, 5120, 3 * 4096 + 17])
def test_sizes(n):
    rng = np.random.default_rng(100 + n)
    x = synth.f32_to_bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    blob = oracle.encode(x)
    for threads in (1, 3):
        assert np.array_equal(afx.afx_decode_host(blob, threads=threads), x)


def test_special_patterns_and_one_value():
    for x in (np.arange(65536, dtype=np.uint16), np.zeros(10000, np.uint16), np.full(4097, 0x3F80, np.uint16),
              np.tile(np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x807F], np.uint16), 777)):
        assert np.array_equal(afx.afx_decode_host(oracle.encode(x), threads=2), x)


def test_twelve_bit_codes():
    fib = [1, 1]
    while len(fib) < 30:
        fib.append(fib[-1] + fib[-2])
    x = np.repeat((np.arange(30, dtype=np.uint16) + 100) << 7, np.array(fib) * 3)
    np.random.default_rng(2).shuffle(x)
    x = x[:200_000] | np.uint16(0x8055)
    blob = oracle.encode(x)
    assert oracle.sections(blob)["code_len"].max() == 12
    assert np.array_equal(afx.afx_decode_host(blob, threads=4), x)


def test_matches_oracle_on_heavy_tails_and_library_blobs():
    x = synth.generate(synth.TensorSpec("t", (300, 4096), "t4", 8))
    blob = oracle.encode(x)
    assert np.array_equal(afx.afx_decode_host(blob, threads=4), oracle.decode(blob, threads=4))
    y = synth.generate(synth.TensorSpec("u", (777, 5120), "normal", 9))
    assert np.array_equal(afx.afx_decode_host(afx.afx_encode(y, (777, 5120)), threads=4), y.ravel())


def test_empty_and_errors():
    blob = oracle.encode(np.zeros(0, np.uint16))
    assert afx.afx_decode_host(blob).size == 0
    x = synth.generate(synth.TensorSpec("t", (4096,), "normal", 3))
    blob = oracle.encode(x)
    small = np.zeros(x.size - 1, np.uint16)
    with pytest.raises(afx.AfxError) as e:
        afx.afx_decode_host(blob, out=small)
    assert e.value.status == afx.AFX_E_BUFFER_TOO_SMALL
    bad = blob.copy()
    bad[:4] = np.frombuffer(b"XXXX", np.uint8)
    with pytest.raises(afx.AfxError) as e:
        afx.afx_decode_host(bad)
    assert e.value.status == afx.AFX_E_BAD_MAGIC
