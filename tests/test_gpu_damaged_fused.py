"""The fused products read a damaged device blob without leaving bounds.

A device blob that differs from the host copy afx_query validated makes the
fused products compute with wrong weights, never read or write outside their
buffers: both kernels take every index that depends on blob contents from the
clamped functions of csrc/afx_index.h (checked on the CPU by
test_index_bounds.py). Here each kind of damage goes through the
matrix-vector kernel (m = 1, 4) and the MFMA kernel (m = 16, 64, 300) in a
batch call beside an undamaged matrix: the call succeeds, guard words before
and after both outputs stay untouched, and the undamaged matrix's product is
still exact (small integers keep every FP32 partial sum exact, so the oracle's
float64 product is the exact answer).
"""
import sys

import numpy as np
import pytest

import oracle
from blob_damage import KINDS, damage
from lossless_bf16_weight_afx_amd import afx, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GUARD = 64  # float32 guard words before and after each output
SENTINEL = 1234.5


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    afx.lib()


def small_ints(rng, shape, lo, hi):
    return synth.f32_to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


def guarded_y(m, rows):
    y = torch.full((m * rows + 2 * GUARD,), SENTINEL, dtype=torch.float32, device="cuda")
    y[GUARD:GUARD + m * rows] = 0
    return y


def guards_intact(y, m, rows):
    a = y.cpu().numpy()
    return bool(np.all(a[:GUARD] == SENTINEL) and np.all(a[GUARD + m * rows:] == SENTINEL))


@pytest.mark.parametrize("what", KINDS)
@pytest.mark.parametrize("kind,m", [("gemv", 1), ("gemv", 4), ("gemm", 16), ("gemm", 64), ("gemm", 300)])
def test_damaged_blob_stays_in_bounds(what, kind, m):
    say(f"[gpu] case damaged blob through the {kind} product: {what}, m={m}")
    rng = np.random.default_rng([KINDS.index(what), m, 7])
    rows, cols = 128, 1024  # a multiple of 64 rows and 256 columns: both kernels take it
    grows, gcols = 64, 512
    w = small_ints(rng, rows * cols, -3, 3)
    gw = small_ints(rng, grows * gcols, -3, 3)
    blob = oracle.encode(w, (rows, cols))
    gblob = oracle.encode(gw, (grows, gcols))
    info, ginfo = afx.afx_query(blob), afx.afx_query(gblob)  # the undamaged host copies
    bad = afx.to_device(damage(blob, what, rng))
    good = afx.to_device(gblob)
    x = torch.from_numpy(small_ints(rng, (m, cols), -2, 2).view(np.int16)).to("cuda")
    gx_bits = small_ints(rng, (m, gcols), -2, 2)
    gx = torch.from_numpy(gx_bits.view(np.int16)).to("cuda")
    y, gy = guarded_y(m, rows), guarded_y(m, grows)
    jobs = [(info, bad.data_ptr(), rows, cols, x.data_ptr(), y.data_ptr() + 4 * GUARD),
            (ginfo, good.data_ptr(), grows, gcols, gx.data_ptr(), gy.data_ptr() + 4 * GUARD)]
    call = afx.afx_restore_gemv_batch_async if kind == "gemv" else afx.afx_restore_gemm_batch_async
    call(jobs, m, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert guards_intact(y, m, rows), "wrote outside the damaged matrix's output"
    assert guards_intact(gy, m, grows), "wrote outside the undamaged matrix's output"
    got = gy[GUARD:GUARD + m * grows].cpu().numpy().astype(np.float64).reshape(m, grows)
    ref, _ = oracle.restore_gemv(gblob, grows, gcols, gx_bits, threads=4)
    assert np.abs(ref).max() < 2 ** 24
    assert np.array_equal(got, ref), "the undamaged matrix of the batch came out wrong"
