"""GPU parity of the restore fused into a matrix-vector product: y += W x with
W restored on the fly, against the oracle's float64 product of the restored
matrix, within the bound that FP32 summation in any order keeps:
gamma_(cols-1) * sum |w x| per output, gamma_j = j u / (1 - j u), u = 2^-24."""
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


def run(w_bits, rows, cols, m, seed, y0=None, dist="normal"):
    blob = oracle.encode(w_bits, (rows, cols))
    info = afx.afx_query(blob)
    dev_blob = afx.to_device(blob)
    x = synth.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((m, cols)).astype(np.float32))
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    y = torch.zeros((m, rows), dtype=torch.float32, device="cuda") if y0 is None else y0.clone()
    afx.afx_restore_gemv_async(info, dev_blob.data_ptr(), rows, cols, xd.data_ptr(), m, y.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref, bound = oracle.restore_gemv(blob, rows, cols, x, threads=4,
                                     y0=None if y0 is None else y0.cpu().numpy())
    got = y.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    assert np.all(err <= bound), f"error above the bound: worst ratio {worst}"
    return worst


@pytest.mark.parametrize("rows,cols,m", [
    (64, 4096, 1),      # one chunk per row
    (640, 5120, 1),     # rows cross chunk boundaries (q_proj-shaped rows)
    (640, 5120, 2),
    (640, 5120, 4),
    (96, 17408, 4),     # down_proj-shaped rows
    (40, 10240, 2),     # x fills the 40 KB activation stage exactly
    (50, 10248, 2),     # x 16 bytes over the stage: read from L2
    (333, 1000, 2),     # several rows per chunk, short last chunk
    (129, 32, 1),       # 128 rows in a chunk
    (7, 8, 4),          # one tiny chunk
])
def test_shapes(rows, cols, m):
    say(f"[gpu] case gemv {rows}x{cols} m={m}")
    w = synth.generate(synth.TensorSpec("w", (rows, cols), "normal", rows + cols))
    worst = run(w, rows, cols, m, seed=rows * 7 + m)
    say(f"[gpu]   worst error / bound = {worst:.3g}")


def test_heavy_tails_and_accumulation():
    say("[gpu] case gemv t4 weights, y accumulated onto existing values")
    rows, cols = 300, 5120
    w = synth.generate(synth.TensorSpec("w", (rows, cols), "t4", 77))
    y0 = torch.randn((2, rows), dtype=torch.float32, device="cuda")
    run(w, rows, cols, 2, seed=5, y0=y0)


def test_q_proj_full_size():
    say("[gpu] case gemv 5120x5120 m=1")
    spec = synth.single_tensor(5120, 5120, 2)[0]
    run(synth.generate(spec), 5120, 5120, 1, seed=9)


def test_batch_of_mixed_matrices_one_launch():
    """Seven matrices of mixed shapes (a decoder layer's, scaled down) in one
    batch call, m = 4; every product within its bound."""
    shapes = [(640, 640), (128, 640), (128, 640), (640, 640), (2176, 640), (2176, 640), (640, 2176)]
    m = 4
    rng = np.random.default_rng(31)
    jobs, keep, refs = [], [], []
    for t, (rows, cols) in enumerate(shapes):
        w = synth.generate(synth.TensorSpec(f"w{t}", (rows, cols), "t4" if t == 6 else "normal", 700 + t))
        blob = oracle.encode(w, (rows, cols))
        info = afx.afx_query(blob)
        db = afx.to_device(blob)
        x = synth.f32_to_bf16_bits(rng.standard_normal((m, cols)).astype(np.float32))
        xd = torch.from_numpy(x.view(np.int16)).to("cuda")
        y = torch.zeros((m, rows), dtype=torch.float32, device="cuda")
        keep.append((info, db, xd, y))
        jobs.append((info, db.data_ptr(), rows, cols, xd.data_ptr(), y.data_ptr()))
        refs.append(oracle.restore_gemv(blob, rows, cols, x, threads=4))
    say("[gpu] case gemv batch of 7 matrices, m=4")
    afx.afx_restore_gemv_batch_async(jobs, m, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for (info, db, xd, y), (ref, bound), shape in zip(keep, refs, shapes):
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= bound), shape


@pytest.mark.parametrize("m", [2, 4])
def test_batch_of_long_rows(m):
    """A batch whose matrices all have rows of a chunk or longer (the two-
    accumulator kernel): rows that wrap at odd columns (8200), a last chunk
    of 104 elements (a partial round), rows of exactly one chunk and
    down_proj-length rows; every product within its bound."""
    shapes = [(40, 5120), (9, 4096), (13, 8200), (3, 17408)]
    rng = np.random.default_rng(47 + m)
    jobs, keep, refs = [], [], []
    for t, (rows, cols) in enumerate(shapes):
        w = synth.generate(synth.TensorSpec(f"l{t}", (rows, cols), "t4" if t == 2 else "normal", 900 + t))
        blob = oracle.encode(w, (rows, cols))
        info = afx.afx_query(blob)
        db = afx.to_device(blob)
        x = synth.f32_to_bf16_bits(rng.standard_normal((m, cols)).astype(np.float32))
        xd = torch.from_numpy(x.view(np.int16)).to("cuda")
        y = torch.zeros((m, rows), dtype=torch.float32, device="cuda")
        keep.append((info, db, xd, y))
        jobs.append((info, db.data_ptr(), rows, cols, xd.data_ptr(), y.data_ptr()))
        refs.append(oracle.restore_gemv(blob, rows, cols, x, threads=4))
    say(f"[gpu] case gemv batch of 4 long-row matrices, m={m}")
    afx.afx_restore_gemv_batch_async(jobs, m, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for (info, db, xd, y), (ref, bound), shape in zip(keep, refs, shapes):
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= bound), shape


@pytest.mark.parametrize("m", [2, 4])
@pytest.mark.parametrize("rows_a,rows_d", [(64, 192), (128, 384)])
def test_long_activations_staged_as_a_chunk_window(m, rows_a, rows_d):
    """Rows of 17,408 columns whose activations (m x 17,408 BF16) do not fit
    the activation stage: when the matrix's workgroup count is a multiple of
    17 (the period, in chunks, of a chunk's starting column), each workgroup
    stages just the 4,096 columns its chunks cover, in chunk order. On a
    256-CU GPU these batches take that path: D's share of the grid is 204
    workgroups as split (64, 192), or 234 trimmed to 221 (128, 384). Small
    integers keep every sum exact, so a wrong column shows."""
    shapes = [(rows_a, 5120), (rows_d, 17408)]
    rng = np.random.default_rng(60 + m + rows_a)
    jobs, keep, refs = [], [], []
    for rows, cols in shapes:
        w = synth.f32_to_bf16_bits(rng.integers(-3, 4, size=rows * cols).astype(np.float32))
        blob = oracle.encode(w, (rows, cols))
        info = afx.afx_query(blob)
        db = afx.to_device(blob)
        x = synth.f32_to_bf16_bits(rng.integers(-2, 3, size=(m, cols)).astype(np.float32))
        xd = torch.from_numpy(x.view(np.int16)).to("cuda")
        y = torch.zeros((m, rows), dtype=torch.float32, device="cuda")
        keep.append((info, db, xd, y))
        jobs.append((info, db.data_ptr(), rows, cols, xd.data_ptr(), y.data_ptr()))
        refs.append(oracle.restore_gemv(blob, rows, cols, x, threads=4)[0])
    say(f"[gpu] case gemv chunk-window activations {shapes}, m={m}")
    afx.afx_restore_gemv_batch_async(jobs, m, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for (info, db, xd, y), ref, shape in zip(keep, refs, shapes):
        assert np.abs(ref).max() < 2 ** 24
        assert np.array_equal(y.cpu().numpy().astype(np.float64), ref), shape


def test_graph_replays_within_bound():
    """A fused matrix-vector product captured in a HIP graph (through
    torch.cuda.graph) after a fill kernel that clears y, replayed three
    times with eager work in between; every replay within its bound."""
    rows, cols, m = 200, 4096, 2
    w = synth.generate(synth.TensorSpec("gw", (rows, cols), "normal", 4242))
    blob = oracle.encode(w, (rows, cols))
    info = afx.afx_query(blob)
    db = afx.to_device(blob)
    x = synth.f32_to_bf16_bits(np.random.default_rng(43).standard_normal((m, cols)).astype(np.float32))
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    y = torch.zeros((m, rows), dtype=torch.float32, device="cuda")
    ref, bound = oracle.restore_gemv(blob, rows, cols, x, threads=4)
    say("[gpu] case graph capture of a fused matrix-vector product")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        y.zero_()
        afx.afx_restore_gemv_async(info, db.data_ptr(), rows, cols, xd.data_ptr(), m, y.data_ptr(), side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y.zero_()  # a fill kernel, not a memset node
        afx.afx_restore_gemv_async(info, db.data_ptr(), rows, cols, xd.data_ptr(), m, y.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        y.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= bound), f"replay {rep}"
