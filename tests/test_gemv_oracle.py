"""Pins of the oracle's restore-and-multiply reference (CPU): products the
arithmetic fixes in closed form, and the argument checks of the fused entry
point that come before any HIP call."""
import numpy as np
import pytest

import oracle
from lossless_bf16_weight_afx_amd import afx, synth


def bf16(values) -> np.ndarray:
    return synth.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


def test_all_ones_times_ramp():
    rows, cols = 3, 64
    w = np.full(rows * cols, 0x3F80, np.uint16)  # 1.0
    x = bf16(np.arange(1, cols + 1))  # small integers are exact in BF16
    y, bound = oracle.restore_gemv(oracle.encode(w), rows, cols, x)
    assert y.shape == (1, rows)
    assert np.all(y == cols * (cols + 1) / 2)
    assert np.all(bound > 0)


def test_identity_returns_x():
    n = 32
    w = np.zeros((n, n), np.uint16)
    w[np.arange(n), np.arange(n)] = 0x3F80
    x = bf16(np.random.default_rng(1).standard_normal((2, n)))
    y, _ = oracle.restore_gemv(oracle.encode(w.ravel()), n, n, x)
    assert np.array_equal(y, oracle.bf16_to_f64(x).reshape(2, n))


def test_orientation_rows_times_first_column():
    # W[r, 0] = r + 1, every other entry 0: y[r] = (r + 1) * x[0]; a transposed
    # W would give y[0] = sum_r (r + 1) x[r] instead
    rows, cols = 5, 40
    w = np.zeros((rows, cols), np.float32)
    w[:, 0] = np.arange(1, rows + 1)
    x = bf16(np.linspace(0.5, 3.0, cols))
    y, _ = oracle.restore_gemv(oracle.encode(bf16(w.ravel())), rows, cols, x)
    x0 = oracle.bf16_to_f64(x)[0]
    assert np.array_equal(y[0], np.arange(1, rows + 1) * x0)


def test_bound_scale_against_a_sum_that_loses_every_small_term():
    # 1 + (cols - 1) * 2^-25 summed left to right in FP32: each 2^-25 is
    # below half an ulp of 1 and rounds away, so the sum stays 1 and errs by
    # (cols - 1) * 2^-25, about half the bound; a bound missing its factor
    # (cols - 1) or off by an order of magnitude fails one of the two checks
    rows, cols = 2, 4096
    w = np.full(rows * cols, 0x3F80, np.uint16)  # 1.0
    x = np.full(cols, 0x3300, np.uint16)  # 2^-25
    x[0] = 0x3F80
    y, bound = oracle.restore_gemv(oracle.encode(w), rows, cols, x)
    assert np.all(y == 1 + (cols - 1) * 2.0 ** -25)
    s = np.float32(0)
    for v in oracle.bf16_to_f64(x).astype(np.float32):
        s = np.float32(s + v)
    assert s == np.float32(1.0)
    err = abs(float(s) - y[0, 0])
    assert err <= bound[0, 0] <= 2.5 * err


def test_bound_with_a_starting_y():
    rows, cols = 3, 64
    w = np.full(rows * cols, 0x3F80, np.uint16)
    x = bf16(np.ones(cols))
    y0 = np.array([[1e6, -2.0, 0.0]])
    y, bound = oracle.restore_gemv(oracle.encode(w), rows, cols, x, y0=y0)
    assert np.array_equal(y, y0 + cols)
    mag = np.abs(y0) + cols  # every term's magnitude, the start included
    assert np.all(bound > mag * cols * 2.0 ** -24) and np.all(bound < mag * (cols + 1) * 2.0 ** -24)


def test_bf16_to_f64_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x3E80, 0x7F80], np.uint16)
    v = oracle.bf16_to_f64(bits)
    assert list(v[:6]) == [1.0, -1.0, 2.0, 0.0, -0.0, 0.25] and np.isinf(v[6])


def test_entry_point_argument_errors():
    afx.lib()
    x = synth.generate(synth.TensorSpec("t", (64, 4096), "normal", 3))
    info = afx.afx_query(oracle.encode(x, (64, 4096)))
    fake = 1 << 40  # never dereferenced: every check below precedes any HIP call
    def rc(rows, cols, m=1, blob=fake, xp=fake, y=fake):
        try:
            afx.afx_restore_gemv_async(info, blob, rows, cols, xp, m, y, 0)
        except afx.AfxError as e:
            return e.status
        return afx.AFX_OK
    assert rc(64, 4095) == afx.AFX_E_INVALID_ARG
    assert rc(65, 4096) == afx.AFX_E_INVALID_ARG
    assert rc(0, 4096) == afx.AFX_E_INVALID_ARG
    assert rc(64, 0) == afx.AFX_E_INVALID_ARG
    assert rc(64 * 4096 // 4, 4) == afx.AFX_E_UNSUPPORTED  # cols not a multiple of 8
    assert rc(64, 4096, m=3) == afx.AFX_E_UNSUPPORTED
    assert rc(64, 4096, m=8) == afx.AFX_E_UNSUPPORTED
    assert rc(64, 4096, blob=0) == afx.AFX_E_INVALID_ARG
    assert rc(64, 4096, xp=0) == afx.AFX_E_INVALID_ARG
    assert rc(64, 4096, y=0) == afx.AFX_E_INVALID_ARG
    assert rc(64, 4096, xp=fake + 8) == afx.AFX_E_MISALIGNED
    assert rc(64, 4096, y=fake + 2) == afx.AFX_E_MISALIGNED
    assert rc(64, 4096, blob=fake + 4) == afx.AFX_E_MISALIGNED


def test_gemm_entry_point_argument_errors():
    afx.lib()
    x = synth.generate(synth.TensorSpec("t", (128, 512), "normal", 4))
    info = afx.afx_query(oracle.encode(x, (128, 512)))
    fake = 1 << 40  # never dereferenced: every check below precedes any HIP call
    def rc(rows, cols, m=1, blob=fake, xp=fake, y=fake):
        try:
            afx.afx_restore_gemm_async(info, blob, rows, cols, xp, m, y, 0)
        except afx.AfxError as e:
            return e.status
        return afx.AFX_OK
    assert rc(128, 511) == afx.AFX_E_INVALID_ARG
    assert rc(0, 512) == afx.AFX_E_INVALID_ARG
    assert rc(512, 128) == afx.AFX_E_UNSUPPORTED  # cols not a multiple of 256
    assert rc(32, 2048) == afx.AFX_E_UNSUPPORTED  # rows not a multiple of 64
    assert rc(128, 512, m=0) == afx.AFX_E_UNSUPPORTED
    assert rc(128, 512, blob=0) == afx.AFX_E_INVALID_ARG
    assert rc(128, 512, xp=0) == afx.AFX_E_INVALID_ARG
    assert rc(128, 512, y=0) == afx.AFX_E_INVALID_ARG
    assert rc(128, 512, xp=fake + 8) == afx.AFX_E_MISALIGNED
    assert rc(128, 512, y=fake + 2) == afx.AFX_E_MISALIGNED
    assert rc(128, 512, blob=fake + 4) == afx.AFX_E_MISALIGNED


def test_fused_outputs_must_not_overlap_inputs():
    """y sharing a byte with a blob or an x of the batch is refused before
    any HIP call (fake, never dereferenced addresses)."""
    afx.lib()
    x = synth.generate(synth.TensorSpec("t", (128, 512), "normal", 5))
    info = afx.afx_query(oracle.encode(x, (128, 512)))
    blob, xp = 1 << 40, 1 << 41
    for call, m in [(afx.afx_restore_gemv_batch_async, 4), (afx.afx_restore_gemm_batch_async, 8)]:
        for y in (blob + 256, xp + 64, blob + int(info.blob_bytes) - 4):
            with pytest.raises(afx.AfxError) as e:
                call([(info, blob, 128, 512, xp, y)], m, 0)
            assert e.value.status == afx.AFX_E_INVALID_ARG
        # another job's blob and x count too
        with pytest.raises(afx.AfxError) as e:
            call([(info, blob, 128, 512, xp, 1 << 42), (info, 1 << 43, 128, 512, xp, blob + 16)], m, 0)
        assert e.value.status == afx.AFX_E_INVALID_ARG
