"""GPU parity of the restore fused into a matrix product on the matrix cores:
y += x W^T with 64-row tiles of W restored into LDS, against the oracle's
float64 product of the restored matrix.

Small-integer weights and activations keep every partial sum exact in FP32,
so there the result must equal the oracle's exactly, whatever the order of
the sums: any indexing mistake (a transposed tile, a wrong slab, a lane
layout) shows. Other data are checked within the classical bound of FP32
summation, gamma_(k-1) * sum |terms|. The matrix instruction's internal
rounding is not documented; test_one_matrix_instruction_rounding measures
it through this product: one instruction (16 products added to an FP32
value) errs by at most a few units u * sum |terms|, inside gamma_16 of an
FP32 sum of its 17 terms in any order, so a product over k columns made of
k/16 such steps stays inside gamma_(k-1) * sum |terms|. Each test reports
its worst error / bound."""
import sys

import numpy as np
import pytest

import oracle
from lossless_bf16_weight_afx_amd import afx, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    afx.lib()


def gemm(blob, rows, cols, x_bits, m, y0=None):
    info = afx.afx_query(blob)
    db = afx.to_device(blob)
    xd = torch.from_numpy(x_bits.view(np.int16)).to("cuda")
    y = torch.zeros((m, rows), dtype=torch.float32, device="cuda") if y0 is None else y0.clone()
    afx.afx_restore_gemm_async(info, db.data_ptr(), rows, cols, xd.data_ptr(), m, y.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def small_ints(rng, shape, lo, hi):
    return synth.f32_to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


@pytest.mark.parametrize("rows,cols,m", [
    (64, 256, 1),       # one tile, one slab, one token
    (128, 768, 37),     # two row tiles, three slabs, a partial token block
    (192, 2816, 130),   # two column ranges (2560 + 256), two token blocks
    (64, 17408, 64),    # down_proj-shaped rows: seven column ranges
    (128, 512, 300),    # two token blocks per wave, two token tiles, the last one partial
    (128, 2816, 48),    # two waves share each token block (partial second block), two column ranges
    (64, 1024, 100),    # one block per wave, the fourth partial
    (64, 768, 20),      # four waves share one partial token block
    (64, 17408, 300),   # two token blocks per wave over 5120-column ranges (3 + a 2048 remainder)
    (128, 5376, 200),   # two token blocks per wave, a 5120-column range and a 256-column one
])
def test_integer_data_exact(rows, cols, m):
    say(f"[gpu] case gemm integers {rows}x{cols} m={m}")
    rng = np.random.default_rng(rows + cols + m)
    w = small_ints(rng, rows * cols, -3, 3)
    x = small_ints(rng, (m, cols), -2, 2)
    blob = oracle.encode(w, (rows, cols))
    got = gemm(blob, rows, cols, x, m)
    ref, _ = oracle.restore_gemv(blob, rows, cols, x, threads=4)
    assert np.abs(ref).max() < 2 ** 24  # every partial sum is exact in FP32
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("m", [31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513])
def test_token_counts_at_every_variant_boundary(m):
    """Exact at the token counts where the kernel variant (four, two or one
    waves per 32-token block, two blocks per wave) or the number of 256-token
    blocks per tile changes; 513 tokens make three blocks per tile, dispatched
    together on one XCD."""
    say(f"[gpu] case gemm integers 128x1024 m={m}")
    rng = np.random.default_rng(5000 + m)
    rows, cols = 128, 1024
    w = small_ints(rng, rows * cols, -3, 3)
    x = small_ints(rng, (m, cols), -2, 2)
    blob = oracle.encode(w, (rows, cols))
    got = gemm(blob, rows, cols, x, m)
    ref, _ = oracle.restore_gemv(blob, rows, cols, x, threads=4)
    assert np.abs(ref).max() < 2 ** 24
    assert np.array_equal(got, ref)


def check(blob, rows, cols, x, m, y0=None):
    got = gemm(blob, rows, cols, x, m, y0)
    ref, bound = oracle.restore_gemv(blob, rows, cols, x, threads=4,
                                     y0=None if y0 is None else y0.cpu().numpy())
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    say(f"[gpu]   worst error / bound = {worst:.3g}")
    assert np.all(err <= bound), f"error above the bound: worst ratio {worst}"
    return worst


def test_one_matrix_instruction_rounding():
    """The rounding of one v_mfma_f32_32x32x16_bf16 step, measured through the
    product: only the first 16 columns of W are nonzero, so every y[t, r] is
    y0[t, r] plus one instruction's 16 products (the later steps add exact
    zeros). Values span 2^-10..2^10 with random signs and y0 is as large as
    the sums, so the sums cancel. The error of each output must stay within
    gamma_16 * (sum |products| + |y0|), the bound of FP32 summation of its 17
    terms in any order (products of two BF16 values are exact in FP32)."""
    rows, cols, m = 128, 256, 256
    rng = np.random.default_rng(5)
    w = np.zeros((rows, cols), np.float32)
    w[:, :16] = rng.standard_normal((rows, 16)) * np.exp2(rng.integers(-10, 10, (rows, 16)))
    wb = synth.f32_to_bf16_bits(w.ravel())
    x = synth.f32_to_bf16_bits((rng.standard_normal((m, cols)) * np.exp2(rng.integers(-10, 10, (m, cols))))
                               .astype(np.float32))
    y0 = torch.from_numpy((rng.standard_normal((m, rows)) * 1e3).astype(np.float32)).to("cuda")
    blob = oracle.encode(wb, (rows, cols))
    say("[gpu] case one matrix instruction's rounding")
    got = gemm(blob, rows, cols, x, m, y0)
    wf = synth.bf16_bits_to_f32(wb).astype(np.float64).reshape(rows, cols)[:, :16]
    xf = synth.bf16_bits_to_f32(x).astype(np.float64).reshape(m, cols)[:, :16]
    c = y0.cpu().numpy().astype(np.float64)
    exact = xf @ wf.T + c  # float64: the 16 exact products and y0, up to float64 rounding
    terms = np.abs(xf) @ np.abs(wf).T + np.abs(c)
    u = 2.0 ** -24
    ratio = np.abs(got - exact) / (u * terms)
    one_rounding = np.mean(got == exact.astype(np.float32).astype(np.float64))
    say(f"[gpu]   max error / (u * sum |terms|) = {ratio.max():.3g} (gamma_16 = 16); equal to one rounding of "
        f"the exact sum in {one_rounding:.3f} of {ratio.size} outputs")
    assert ratio.max() <= 16 / (1 - 16 * u)


@pytest.mark.parametrize("rows,cols,m,dist", [
    (64, 5120, 128, "normal"),     # a q_proj-shaped row tile, one full token block
    (320, 5120, 200, "normal"),
    (128, 17408, 16, "normal"),
    (256, 5120, 33, "t4"),         # heavy tails: longer codes
])
def test_random_data_within_bound(rows, cols, m, dist):
    say(f"[gpu] case gemm {dist} {rows}x{cols} m={m}")
    w = synth.generate(synth.TensorSpec("w", (rows, cols), dist, rows + cols + m))
    x = synth.f32_to_bf16_bits(np.random.default_rng(m).standard_normal((m, cols)).astype(np.float32))
    check(oracle.encode(w, (rows, cols)), rows, cols, x, m)


def test_twelve_bit_codes_and_a_starting_y():
    """Exponents spread over all 256 values: codes up to the 12-bit limit and
    the longest staged row segments; y starts from nonzero values."""
    say("[gpu] case gemm 256 exponent values, y accumulated onto existing values")
    rows, cols, m = 128, 1024, 40
    rng = np.random.default_rng(12)
    e = np.minimum(rng.geometric(0.02, size=rows * cols), 255).astype(np.uint16)
    w = (rng.integers(0, 2, rows * cols).astype(np.uint16) << 15) | (e << 7) | rng.integers(0, 128, rows * cols).astype(np.uint16)
    w[(e == 255)] &= 0x807F  # keep them finite: no Inf or NaN in the products
    w[(e == 255)] |= 254 << 7
    blob = oracle.encode(w, (rows, cols))
    assert afx.afx_query(blob).longest_code == 12
    x = synth.f32_to_bf16_bits((rng.standard_normal((m, cols)) * 1e-30).astype(np.float32))
    y0 = torch.randn((m, rows), dtype=torch.float32, device="cuda")
    check(blob, rows, cols, x, m, y0)


def test_incompressible_exponents():
    """Uniformly random exponent bytes (8-bit codes, nothing to compress):
    every row's code words for a 256-column slab are the longest the data can
    make, 2048 bits plus alignment."""
    say("[gpu] case gemm uniform exponents")
    rows, cols, m = 64, 512, 8
    rng = np.random.default_rng(21)
    e = rng.integers(1, 255, rows * cols).astype(np.uint16)  # no Inf/NaN
    w = (rng.integers(0, 2, rows * cols).astype(np.uint16) << 15) | (e << 7) | rng.integers(0, 128, rows * cols).astype(np.uint16)
    blob = oracle.encode(w, (rows, cols))
    x = synth.f32_to_bf16_bits((rng.standard_normal((m, cols)) * 1e-30).astype(np.float32))
    check(blob, rows, cols, x, m)


def test_layer_batch_one_launch():
    """The seven matrices of one Qwen3-14B-shaped decoder layer in one batch
    call at m = 16; every product within its bound."""
    m = 16
    specs = [s for s in synth.decoder_layer(0) if len(s.shape) == 2]
    rng = np.random.default_rng(41)
    jobs, keep = [], []
    for sp in specs:
        rows, cols = sp.shape
        blob = afx.afx_encode(synth.generate(sp, threads=16), sp.shape, threads=16)
        info = afx.afx_query(blob)
        db = afx.to_device(blob)
        x = synth.f32_to_bf16_bits(rng.standard_normal((m, cols)).astype(np.float32))
        xd = torch.from_numpy(x.view(np.int16)).to("cuda")
        y = torch.zeros((m, rows), dtype=torch.float32, device="cuda")
        keep.append((blob, x, y, db, xd, info))
        jobs.append((info, db.data_ptr(), rows, cols, xd.data_ptr(), y.data_ptr()))
    say("[gpu] case gemm batch of a layer's 7 matrices, m=16")
    afx.afx_restore_gemm_batch_async(jobs, m, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for (blob, x, y, _, _, _), sp in zip(keep, specs):
        ref, bound = oracle.restore_gemv(blob, sp.shape[0], sp.shape[1], x, threads=16)
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        say(f"[gpu]   {sp.name}: worst error / bound = {float(np.max(err / np.maximum(bound, 1e-300))):.3g}")
        assert np.all(err <= bound), sp.name


def test_batches_over_sixteen_matrices():
    """Eighteen matrices in one batch call of each fused entry point: two
    launches each (16 + 2); every product within its bound."""
    rng = np.random.default_rng(77)
    mats = []
    for t in range(18):
        rows, cols = 64 * (1 + t % 3), 256 * (1 + t % 4)
        w = synth.generate(synth.TensorSpec(f"b{t}", (rows, cols), "normal", 800 + t))
        blob = oracle.encode(w, (rows, cols))
        mats.append((blob, rows, cols, afx.afx_query(blob), afx.to_device(blob)))
    for name, m, call, tol in [("gemv", 4, afx.afx_restore_gemv_batch_async, 1.0),
                               ("gemm", 5, afx.afx_restore_gemm_batch_async, 1.0)]:
        say(f"[gpu] case {name} batch of 18 matrices, m={m}")
        jobs, keep = [], []
        for blob, rows, cols, info, db in mats:
            x = synth.f32_to_bf16_bits(rng.standard_normal((m, cols)).astype(np.float32))
            xd = torch.from_numpy(x.view(np.int16)).to("cuda")
            y = torch.zeros((m, rows), dtype=torch.float32, device="cuda")
            keep.append((x, xd, y))
            jobs.append((info, db.data_ptr(), rows, cols, xd.data_ptr(), y.data_ptr()))
        call(jobs, m, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for (blob, rows, cols, _, _), (x, _, y) in zip(mats, keep):
            ref, bound = oracle.restore_gemv(blob, rows, cols, x)
            err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
            assert np.all(err <= tol * bound), (name, rows, cols)


def test_graph_replays_exact():
    """The MFMA product captured in a HIP graph (through torch.cuda.graph)
    after a fill kernel that clears y, replayed three times with eager work
    in between; on integer data every replay equals the oracle exactly."""
    rows, cols, m = 128, 2816, 40
    rng = np.random.default_rng(77)
    w = small_ints(rng, rows * cols, -3, 3)
    x = small_ints(rng, (m, cols), -2, 2)
    blob = oracle.encode(w, (rows, cols))
    info = afx.afx_query(blob)
    db = afx.to_device(blob)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    y = torch.zeros((m, rows), dtype=torch.float32, device="cuda")
    ref, _ = oracle.restore_gemv(blob, rows, cols, x, threads=4)
    say("[gpu] case graph capture of an MFMA product")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        y.zero_()
        afx.afx_restore_gemm_async(info, db.data_ptr(), rows, cols, xd.data_ptr(), m, y.data_ptr(), side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y.zero_()  # a fill kernel, not a memset node
        afx.afx_restore_gemm_async(info, db.data_ptr(), rows, cols, xd.data_ptr(), m, y.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        y.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().astype(np.float64), ref), f"replay {rep}"


def test_fused_products_past_2_32_weights():
    """One matrix of 1,048,640 x 4096 weights (more than 2^32): element
    offsets, sign/mantissa byte offsets and row indices pass 32 bits. The
    integer weights repeat with a period of 2^24 + 4099, prime to the chunk
    size and the row length. Both fused products, the matrix-vector one
    (m = 1) and the MFMA one (m = 8), must equal y = W x exactly (integer
    sums below 2^24 are exact in FP32). The blob comes from the library's
    encoder; the oracle decoder checks it on chunks at the start, around
    element 2^32 and at the end."""
    rows, cols = 1_048_640, 4096
    n = rows * cols
    period = (1 << 24) + 4099
    rng = np.random.default_rng(99)
    vals = rng.integers(-3, 4, size=period).astype(np.int8)
    pat = synth.f32_to_bf16_bits(vals.astype(np.float32))
    say("[gpu] generate 2^32+ integer weights")
    w = np.empty(n, np.uint16)
    for o in range(0, n, period):
        k = min(period, n - o)
        w[o:o + k] = pat[:k]
    say("[gpu] encode 2^32+ weights")
    blob = afx.afx_encode(w, (rows, cols))
    info = afx.afx_query(blob)
    c_mid, c_hi = (1 << 32) // 4096, int(info.n_chunks)
    for c0, c1 in ((0, 3), (c_mid - 2, c_mid + 2), (c_hi - 2, c_hi)):
        assert np.array_equal(oracle.decode_chunks(blob, c0, c1), w[c0 * 4096:min(c1 * 4096, n)])
    del w
    dev = afx.to_device(blob)
    del blob
    x8 = rng.integers(-2, 3, size=(8, cols)).astype(np.float32)
    say("[gpu] reference y = W x in blocks of rows")
    ref = np.empty((8, rows), np.float32)
    blk = 1 << 16  # rows per block; a block's weights are a slice of the repeated pattern
    reps = np.tile(vals, (blk * cols) // period + 2)
    for r0 in range(0, rows, blk):
        nr = min(blk, rows - r0)
        o = (r0 * cols) % period
        wb = reps[o:o + nr * cols].reshape(nr, cols).astype(np.float32)
        ref[:, r0:r0 + nr] = (wb @ x8.T).T
    del reps, wb
    xd = torch.from_numpy(synth.f32_to_bf16_bits(x8).view(np.int16)).to("cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for m, name in ((1, "matrix-vector"), (8, "MFMA")):
        y = torch.zeros((m, rows), dtype=torch.float32, device="cuda")
        say(f"[gpu] case {name} product, {rows}x{cols}, m={m}")
        if m == 1:
            afx.afx_restore_gemv_async(info, dev.data_ptr(), rows, cols, xd.data_ptr(), m, y.data_ptr(), stream)
        else:
            afx.afx_restore_gemm_async(info, dev.data_ptr(), rows, cols, xd.data_ptr(), m, y.data_ptr(), stream)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), ref[:m]), name
