"""GPU parity: the HIP restore against the original bits and the CPU oracle.

Blobs of the single-tensor tests come from the oracle's encoder. The test of
the library's encoder, the model paths (streamed, resident, stored, tiered:
they encode through the library, as a user would) and the tensor past 2^32
values (whose blob the oracle decoder checks on sampled chunks first) use the
library's encoder. The expected values are always the generated inputs
themselves, which the oracle decoder reproduces bit for bit (pinned in
test_oracle_pins.py). Every comparison is exact (integer bit patterns).
"""
import os
import sys

import numpy as np
import pytest

import oracle
from blob_damage import damage
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
    return torch.device("cuda:0")


def restore(blob: np.ndarray, guard: int = 64):
    """Decode on the GPU into a buffer with sentinel words after the output."""
    info = afx.afx_query(blob)
    dev = afx.to_device(blob)
    n = int(info.n_elems)
    out = torch.full((n + guard,), 0x5A5A, dtype=torch.int16, device="cuda")
    afx.afx_decode_tensor(info, dev.data_ptr(), out.data_ptr(), 2 * n, torch.cuda.current_stream().cuda_stream)
    tail = out[n:].cpu().numpy()
    assert np.all(tail == 0x5A5A), "wrote past the output"
    return out[:n].cpu().numpy().view(np.uint16)


def check(x: np.ndarray, name: str):
    say(f"[gpu] case {name}: n={x.size}")
    blob = oracle.encode(x)
    y = restore(blob)
    x = x.ravel()
    if not np.array_equal(y, x):
        bad = np.nonzero(y != x)[0]
        raise AssertionError(f"{name}: {bad.size} mismatches, first at {bad[:5]}: got {y[bad[:5]]} want {x[bad[:5]]}")


@pytest.mark.parametrize("n", [1, 31, 32, 33, 128, 4095, 4096, 4097, 5120, 3 * 4096 + 17, 64 * 4096 + 4000])
def test_sizes(n):
    rng = np.random.default_rng(n)
    x = synth.f32_to_bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    check(x, f"normal-n{n}")


def test_empty_tensor():
    blob = oracle.encode(np.zeros(0, np.uint16))
    info = afx.afx_query(blob)
    dev = afx.to_device(blob)
    afx.afx_decode_tensor(info, dev.data_ptr(), 0, 0, torch.cuda.current_stream().cuda_stream)


def test_special_patterns():
    check(np.arange(65536, dtype=np.uint16), "all-65536-patterns")
    check(np.zeros(10000, np.uint16), "all-zero")
    check(np.full(4097, 0x3F80, np.uint16), "constant")
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x807F, 0x7F7F], np.uint16)
    x = np.tile(specials, 5000)
    np.random.default_rng(1).shuffle(x)
    check(x, "nan-inf-zero-subnormal")


def test_longest_codes():
    # a Fibonacci histogram forces many 12-bit codes
    fib = [1, 1]
    while len(fib) < 30:
        fib.append(fib[-1] + fib[-2])
    counts = np.array(fib) * 3
    x = np.repeat((np.arange(30, dtype=np.uint16) + 100) << 7, counts)
    np.random.default_rng(2).shuffle(x)
    x = x[:200_000] | np.uint16(0x8055)
    blob = oracle.encode(x)
    assert oracle.sections(blob)["code_len"].max() == 12
    check(x, "fibonacci-12-bit-codes")


def test_c1_tensor():
    check(synth.generate(synth.single_tensor()[0]), "1024x1024")


def test_c2_q_proj():
    check(synth.generate(synth.single_tensor(5120, 5120, 2)[0]), "5120x5120")


def test_heavy_tail_slice():
    spec = synth.TensorSpec("t4", (4096, 5120), "t4", 4)
    check(synth.generate(spec), "t4-4096x5120")


def test_matches_oracle_decoder():
    x = synth.generate(synth.TensorSpec("t", (300, 4096), "t4", 8))
    blob = oracle.encode(x)
    assert np.array_equal(restore(blob), oracle.decode(blob, threads=4))


def test_library_encoder_blob():
    x = synth.generate(synth.TensorSpec("t", (777, 5120), "normal", 9))
    blob = afx.afx_encode(x, (777, 5120))
    say("[gpu] case library-encoder blob")
    assert np.array_equal(restore(blob), x)


def test_misaligned_output_rejected():
    x = synth.generate(synth.TensorSpec("t", (4096,), "normal", 3))
    blob = oracle.encode(x)
    info = afx.afx_query(blob)
    dev = afx.to_device(blob)
    out = torch.full((4096 + 8,), 7, dtype=torch.int16, device="cuda")
    with pytest.raises(afx.AfxError) as e:
        afx.afx_decode_tensor(info, dev.data_ptr(), out.data_ptr() + 2, 8192, 0)
    assert e.value.status == afx.AFX_E_MISALIGNED
    assert torch.all(out == 7).item()


@pytest.mark.parametrize("what", ["bases", "gaps", "words", "lengths", "all"])
def test_corrupt_device_blob_stays_in_bounds(what):
    """A device blob that differs from the host copy afx_query validated
    restores to wrong bits, never out of bounds: AFX_OK, the guard words
    before and after the output untouched, and a good tensor restored in the
    same launch still exact. (The index arithmetic behind this is checked
    on the CPU by test_index_bounds.py.)"""
    rng = np.random.default_rng(["bases", "gaps", "words", "lengths", "all"].index(what) + 90)
    xs = [synth.generate(synth.TensorSpec("c0", (3 * 4096 + 77,), "normal", 91)),
          synth.generate(synth.TensorSpec("c1", (256, 4096), "t4", 92))]
    good = synth.generate(synth.TensorSpec("good", (5000, 33), "normal", 93))
    guard = 128  # elements (256 bytes) of guard words before and after each output
    say(f"[gpu] case corrupt device blob: {what}")
    for x in xs:
        blob = oracle.encode(x)
        info = afx.afx_query(blob)  # the undamaged host copy
        bad = damage(blob, what, rng)
        dev = afx.to_device(bad)
        n = x.size
        out = torch.full((n + 2 * guard,), 0x5A5A, dtype=torch.int16, device="cuda")
        gblob = oracle.encode(good)
        ginfo = afx.afx_query(gblob)
        gdev = afx.to_device(gblob)
        gout = torch.full((good.size + 2 * guard,), 0x5A5A, dtype=torch.int16, device="cuda")
        jobs = afx.make_jobs([(info, dev.data_ptr(), out.data_ptr() + 2 * guard, 2 * n),
                              (ginfo, gdev.data_ptr(), gout.data_ptr() + 2 * guard, 2 * good.size)])
        afx.afx_decode_layer_async(jobs, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.all(o[:guard] == 0x5A5A) and np.all(o[guard + n:] == 0x5A5A), "wrote outside the output"
        g = gout.cpu().numpy()
        assert np.all(g[:guard] == 0x5A5A) and np.all(g[guard + good.size:] == 0x5A5A)
        assert np.array_equal(g[guard:guard + good.size].view(np.uint16), good), "good tensor of the batch damaged"
        # the same damaged blob through the blocking call
        afx.afx_decode_tensor(info, dev.data_ptr(), out.data_ptr() + 2 * guard, 2 * n,
                              torch.cuda.current_stream().cuda_stream)
        o = out.cpu().numpy()
        assert np.all(o[:guard] == 0x5A5A) and np.all(o[guard + n:] == 0x5A5A), "wrote outside the output"
        if what in ("words", "all"):
            assert not np.array_equal(o[guard:guard + n].view(np.uint16), x)  # it did decode something else


def layer_blobs(layer=0):
    specs = synth.decoder_layer(layer)
    xs, blobs = [], []
    for sp in specs:
        say(f"[gpu] encode {sp.name} {sp.shape}")
        x = synth.generate(sp)
        xs.append(x)
        blobs.append(oracle.encode(x, sp.shape))
    return specs, xs, blobs


def test_layer_batch_one_launch():
    """The 11 tensors of a Qwen3-14B-shaped layer restored by one enqueue."""
    specs, xs, blobs = layer_blobs(0)
    infos = [afx.afx_query(b) for b in blobs]
    devs = [afx.to_device(b) for b in blobs]
    outs = [torch.empty(x.size + 64, dtype=torch.int16, device="cuda").fill_(0x5A5A) for x in xs]
    jobs = afx.make_jobs([(i, d.data_ptr(), o.data_ptr(), 2 * x.size) for i, d, o, x in zip(infos, devs, outs, xs)])
    say("[gpu] case layer batch (11 tensors, one launch)")
    afx.afx_decode_layer_async(jobs, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for sp, x, o in zip(specs, xs, outs):
        y = o.cpu().numpy().view(np.uint16)
        assert np.all(y[x.size:] == 0x5A5A), sp.name
        assert np.array_equal(y[:x.size], x), sp.name
    # the same tensors one by one give the same bits
    for sp, x, i, d in zip(specs, xs, infos, devs):
        o = torch.empty(x.size, dtype=torch.int16, device="cuda")
        afx.afx_decode_tensor(i, d.data_ptr(), o.data_ptr(), 2 * x.size, 0)
        assert np.array_equal(o.cpu().numpy().view(np.uint16), x), sp.name


def test_many_small_tensors_split_over_launches():
    """More jobs than one launch holds: 40 tensors of mixed sizes."""
    rng = np.random.default_rng(4)
    xs = [synth.generate(synth.TensorSpec(f"t{i}", (int(rng.integers(1, 30000)),), "normal", 500 + i))
          for i in range(40)]
    blobs = [oracle.encode(x) for x in xs]
    infos = [afx.afx_query(b) for b in blobs]
    devs = [afx.to_device(b) for b in blobs]
    outs = [torch.empty(x.size, dtype=torch.int16, device="cuda") for x in xs]
    say("[gpu] case 40 small tensors")
    afx.afx_decode_layer_async([(i, d.data_ptr(), o.data_ptr(), 2 * x.size)
                                for i, d, o, x in zip(infos, devs, outs, xs)], 0)
    torch.cuda.synchronize()
    for x, o in zip(xs, outs):
        assert np.array_equal(o.cpu().numpy().view(np.uint16), x)


def restore_batch_exact(xs, name, max_workgroups=None, blobs=None):
    """Encode xs with the library (unless blobs are given), restore them with
    one batch call (on at most max_workgroups workgroups, if given) into
    outputs followed by guard words, and compare every output exactly."""
    if blobs is None:
        blobs = [afx.afx_encode(x, threads=8) for x in xs]
    infos = [afx.afx_query(b) for b in blobs]
    devs = [afx.to_device(b) for b in blobs]
    outs = [torch.full((x.size + 64,), 0x5A5A, dtype=torch.int16, device="cuda") for x in xs]
    say(f"[gpu] case {name}: {len(xs)} tensors, chunks {[int(i.n_chunks) for i in infos]}, "
        f"max_workgroups {max_workgroups}")
    jobs = [(i, d.data_ptr(), o.data_ptr(), 2 * x.size) for i, d, o, x in zip(infos, devs, outs, xs)]
    if max_workgroups is None:
        afx.afx_decode_layer_async(jobs, 0)
    else:
        afx.afx_decode_layer_grid_async(jobs, max_workgroups, 0)
    torch.cuda.synchronize()
    for k, (x, o) in enumerate(zip(xs, outs)):
        y = o.cpu().numpy().view(np.uint16)
        assert np.all(y[x.size:] == 0x5A5A), f"{name}: tensor {k} wrote past its output"
        assert np.array_equal(y[:x.size], x), f"{name}: tensor {k} differs"


def test_twelve_mid_size_tensors_one_launch():
    """Twelve tensors of 256-700 chunks with ragged ends, normal and
    heavy-tailed values, in one launch: the grid is split twelve ways, each
    workgroup restoring one tensor's share with that tensor's table."""
    rng = np.random.default_rng(12)
    xs = [synth.generate(synth.TensorSpec(f"w{i}", (int(rng.integers(256, 700)) * 4096 - int(rng.integers(0, 4000)),),
                                          "t4" if i % 3 == 0 else "normal", 700 + i))
          for i in range(12)]
    restore_batch_exact(xs, "12 mid-size tensors")


def test_workgroups_with_fewer_chunks_than_waves():
    """Three tensors (1000, 600 and 300 chunks) split over the grid leave
    each workgroup about eight chunks, fewer than its 16 waves: waves without
    a chunk of their own skip the tensor, the others restore it."""
    xs = [synth.generate(synth.TensorSpec(f"f{i}", (c * 4096 + 100 * i,), "normal", 800 + i))
          for i, c in enumerate((1000, 600, 300))]
    restore_batch_exact(xs, "few chunks per workgroup")


def test_full_launch_of_mixed_tensors():
    """32 tensors in one launch (the most one launch holds): eight of about
    300 chunks and 24 small ones down to one element, in a random order, with
    ragged ends; the small ones share workgroups."""
    rng = np.random.default_rng(32)
    xs = [synth.generate(synth.TensorSpec(f"m{i}", (300 * 4096 + int(rng.integers(0, 4096)),), "normal", 900 + i))
          for i in range(8)]
    xs += [synth.generate(synth.TensorSpec(f"s{i}", (int(rng.integers(1, 20000)),), "normal", 950 + i))
           for i in range(24)]
    order = rng.permutation(len(xs))
    restore_batch_exact([xs[i] for i in order], "32 mixed tensors")


_GRID_BATCH = {}


def grid_batch():
    """A large heavy-tailed tensor (2,000 chunks), three mid-size ones and
    four small ones, ragged ends, encoded once for every grid cap."""
    if not _GRID_BATCH:
        rng = np.random.default_rng(77)
        xs = [synth.generate(synth.TensorSpec("big", (2000 * 4096 - 123,), "t4", 1000))]
        xs += [synth.generate(synth.TensorSpec(f"mid{i}", (c * 4096 + 17 * i,), "normal", 1001 + i))
               for i, c in enumerate((300, 97, 33))]
        xs += [synth.generate(synth.TensorSpec(f"small{i}", (int(rng.integers(1, 20000)),), "normal", 1010 + i))
               for i in range(4)]
        _GRID_BATCH["xs"] = xs
        _GRID_BATCH["blobs"] = [afx.afx_encode(x, threads=8) for x in xs]
    return _GRID_BATCH["xs"], _GRID_BATCH["blobs"]


@pytest.mark.parametrize("cap", [1, 2, 3, 7, 9, 31, 100, 255, 257, 10**9])
def test_grid_caps_bit_exact(cap):
    """The same batch on at most 1 .. 257 workgroups (and a cap above any
    device): odd workgroup counts exercise the chunk rotation between a
    tensor's workgroups (ranks counted XCD by XCD), the waves' claiming of
    long per-workgroup lists, and workgroups that serve several tensors
    (fewer workgroups than tensors). Every output exact, guards intact."""
    xs, blobs = grid_batch()
    restore_batch_exact(xs, f"grid cap {cap}", max_workgroups=cap, blobs=blobs)


def test_embedding_full_size():
    """151936 x 5120 heavy-tailed tensor, bit-exact in full."""
    spec = synth.embedding()[0]
    say("[gpu] generate embedding")
    x = synth.generate(spec)
    say("[gpu] oracle-encode embedding")
    blob = oracle.encode(x, spec.shape)
    info = afx.afx_query(blob)
    dev = afx.to_device(blob)
    del blob
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    out = torch.empty_like(xd)
    say("[gpu] case embedding 151936x5120")
    afx.afx_decode_tensor(info, dev.data_ptr(), out.data_ptr(), 2 * x.size, torch.cuda.current_stream().cuda_stream)
    assert torch.equal(out, xd)


def test_more_than_2_32_values():
    """A tensor of 2^32 + 3 * 4096 + 77 values: element indices, sign/mantissa
    byte offsets and output byte offsets all pass 2^32, and the last chunk is
    ragged. The values repeat with a period of 2^24 + 4099, which shares no
    factor with the chunk size, so no two chunks hold the same values. The
    blob comes from the library's encoder (the oracle's bit-serial encoder
    takes minutes at this size); the oracle decoder checks it on the chunks
    at the start, around element 2^32 and at the end. The GPU restore must
    equal the input in full."""
    n = (1 << 32) + 3 * 4096 + 77
    period = (1 << 24) + 4099
    say("[gpu] generate 2^32+ values")
    rng = np.random.default_rng(42)
    base = (rng.standard_normal(period, dtype=np.float32) * 0.02).view(np.uint32)
    base = (base >> 16).astype(np.uint16)  # BF16 bits, truncated
    x = np.empty(n, np.uint16)
    for o in range(0, n, period):
        k = min(period, n - o)
        x[o:o + k] = base[:k]
    say("[gpu] encode 2^32+ values")
    blob = afx.afx_encode(x, (n,))
    info = afx.afx_query(blob)
    assert int(info.n_elems) == n
    c_mid, c_hi = (1 << 32) // 4096, int(info.n_chunks)
    for c0, c1 in ((0, 3), (c_mid - 2, c_mid + 2), (c_hi - 2, c_hi)):
        assert np.array_equal(oracle.decode_chunks(blob, c0, c1), x[c0 * 4096:min(c1 * 4096, n)])
    dev = afx.to_device(blob)
    del blob
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    del x
    out = torch.full((n + 64,), 0x5A5A, dtype=torch.int16, device="cuda")
    say(f"[gpu] case n={n}")
    afx.afx_decode_tensor(info, dev.data_ptr(), out.data_ptr(), 2 * n, torch.cuda.current_stream().cuda_stream)
    assert torch.equal(out[:n], xd)
    assert bool((out[n:] == 0x5A5A).all()), "wrote past the output"


def test_streamed_units_double_buffered():
    """Units copied from pinned host memory on a side stream while the
    previous unit is restored; every unit bit-exact."""
    from lossless_bf16_weight_afx_amd import stream

    T = synth.TensorSpec
    units_specs = [
        [T("u0.w", (2000, 517), "normal", 11), T("u0.norm", (5120,), "normal", 12, 1.0, 0.05)],
        [T("u1.w", (1024, 4096), "t4", 13)],
        [T("u2.a", (777, 33), "normal", 14), T("u2.b", (4096,), "normal", 15), T("u2.c", (128,), "normal", 16, 1.0, 0.05)],
        [T("u3.w", (3000, 1000), "normal", 17)],
        [T("u4.w", (50, 4096), "t4", 18)],
    ]
    say("[gpu] case streamed units: build store")
    units = stream.build_model(units_specs, threads=8, keep_raw=True)
    st = stream.Streamer(units)
    ok = []
    say("[gpu] case streamed units: checked pass")
    st.run(on_unit=lambda i, u, out: ok.append(stream.check_unit(u, out)))
    assert ok == [True] * len(units)
    say("[gpu] case streamed units: free-running pass, every unit copied aside")
    snaps = [torch.empty(stream.unit_slots(u), dtype=torch.int16, device="cuda") for u in units]
    res = st.run(snapshot=snaps)
    torch.cuda.synchronize()
    assert [stream.check_unit(u, sn) for u, sn in zip(units, snaps)] == [True] * len(units)
    # the last two units are still in their buffers after a free-running pass
    assert stream.check_unit(units[-1], st.out[(len(units) - 1) % 2])
    assert stream.check_unit(units[-2], st.out[(len(units) - 2) % 2])
    assert res["e2e_ms"] > 0 and len(res["decode_ms"]) == len(units)


def _box_threads() -> int:
    try:
        return max(1, int(os.environ.get("OMP_NUM_THREADS", "8")))
    except ValueError:
        return 8


def test_full_model_streamed_every_unit_bit_exact():
    """The whole 40-layer model at full size (42 units: the embedding, 40
    Qwen3-14B-shaped layers, the output head with the final norm; 29.5 GB
    restored from 20.5 GB compressed in pinned host memory), streamed with
    the copy of each unit overlapping the restore of the one before, running
    free. After each restore the unit's output is copied aside on the compute
    stream (no host wait), and every copy is compared with the unit's
    original bits, generated again unit by unit. The same model restored
    with its compressed bytes resident in HBM must equal those copies."""
    from lossless_bf16_weight_afx_amd import stream

    threads = _box_threads()
    say("[gpu] case full model: build the compressed store (42 units)")
    units = stream.build_model(synth.model_units(), threads=threads, progress=say)
    assert len(units) == 42
    assert 2 * sum(u.n_values for u in units) == 29_536_614_400
    st = stream.Streamer(units)
    snaps = [torch.empty(stream.unit_slots(u), dtype=torch.int16, device="cuda") for u in units]
    say("[gpu] case full model: free-running streamed pass with copies aside")
    res = st.run(snapshot=snaps)
    torch.cuda.synchronize()
    assert len(res["decode_ms"]) == 42
    del st
    bad = []
    for k, (u, sn) in enumerate(zip(units, snaps)):
        if not stream.check_unit_regen(u, sn, threads):
            bad.append((k, u.name))
        say(f"[gpu] case full model: unit {k} {u.name} checked")
    assert not bad, f"units restored wrong: {bad}"
    say("[gpu] case full model: resident pass against the streamed one")
    rres = stream.resident_decode(units, steps=1, check=True, reference=snaps)
    assert rres["bit_exact"] is True and rres["launches"] == 42


def test_resident_model_one_launch_per_unit():
    """Every unit's compressed bytes resident in HBM, one call per unit back
    to back, each unit into its own output region; every unit bit-exact."""
    from lossless_bf16_weight_afx_amd import stream

    T = synth.TensorSpec
    rng = np.random.default_rng(21)
    units_specs = []
    for u in range(12):
        units_specs.append([T(f"m{u}.a", (int(rng.integers(1, 700)), 512), "normal", 600 + 3 * u),
                            T(f"m{u}.b", (int(rng.integers(1, 9000)),), "t4", 601 + 3 * u),
                            T(f"m{u}.n", (128,), "normal", 602 + 3 * u, 1.0, 0.05)])
    say("[gpu] case resident model: build store (36 tensors)")
    units = stream.build_model(units_specs, threads=8, keep_raw=True)
    res = stream.resident_decode(units, steps=2, check=True)
    assert res["launches"] == 12
    assert res["bit_exact"] is True
    assert res["ms"] > 0


def test_disk_store_read_copy_restore(tmp_path):
    """Units read from a store file (O_DIRECT where the file system allows it)
    into pinned memory, copied and restored with the three steps overlapped;
    every unit bit-exact, staging and device buffers reused."""
    from lossless_bf16_weight_afx_amd import store

    T = synth.TensorSpec
    units_specs = [
        [T("d0.w", (1500, 640), "normal", 41), T("d0.norm", (5120,), "normal", 42, 1.0, 0.05)],
        [T("d1.w", (512, 4096), "t4", 43)],
        [T("d2.a", (77, 33), "normal", 44), T("d2.b", (4097,), "normal", 45)],
        [T("d3.w", (2000, 1000), "normal", 46)],
        [T("d4.w", (33, 4096), "t4", 47), T("d4.n", (128,), "normal", 48, 1.0, 0.05)],
        [T("d5.w", (4096, 700), "normal", 49)],
    ]
    path = str(tmp_path / "model.afxs")
    say("[gpu] case disk store: write")
    st = store.write_store(path, units_specs, threads=8)
    try:
        fd = os.open(path, os.O_RDONLY | os.O_DIRECT)
        os.close(fd)
        direct = True
    except OSError:
        direct = False
    ds = store.DiskStreamer(st, threads=4, direct=direct)
    ok = []
    say(f"[gpu] case disk store: checked pass (direct={direct})")
    ds.run(on_unit=lambda i, u, out: ok.append(store.check_unit(out, units_specs[i])))
    assert ok == [True] * len(units_specs)
    say("[gpu] case disk store: free-running pass")
    res = ds.run()
    torch.cuda.synchronize()
    n = len(units_specs)
    assert store.check_unit(ds.out[(n - 1) % 2], units_specs[-1])
    assert store.check_unit(ds.out[(n - 2) % 2], units_specs[-2])
    assert res["e2e_s"] > 0 and len(res["decode_ms"]) == n
    del ds
    # the pages' placement: unpack on the host, copy the restored bytes
    hs = store.HostUnpackStreamer(st, read_threads=4, unpack_threads=4, direct=direct)
    ok = []
    say("[gpu] case disk store: host-unpack pass")
    hs.run(on_unit=lambda i, u, out: ok.append(store.check_unit(out, units_specs[i])))
    assert ok == [True] * len(units_specs)


def test_tiers_every_mix_bit_exact(tmp_path):
    """Units held in all four tiers at once (restored in HBM, compressed in
    HBM, compressed in pinned RAM, on disk); a pass restores each in order,
    bit-exact, and a plan under budgets uses only what the budgets allow."""
    from lossless_bf16_weight_afx_amd import store, tiers

    T = synth.TensorSpec
    units_specs = [[T(f"r{i}.w", (int(200 + 97 * i), 1024), "normal" if i % 3 else "t4", 60 + i),
                    T(f"r{i}.n", (1024,), "normal", 80 + i, 1.0, 0.05)] for i in range(9)]
    path = str(tmp_path / "tiers.afxs")
    say("[gpu] case tiers: write store")
    st = store.write_store(path, units_specs, threads=8)
    try:
        fd = os.open(path, os.O_RDONLY | os.O_DIRECT)
        os.close(fd)
        direct = True
    except OSError:
        direct = False
    mix = ["D", "G", "Gc", "H", "D", "D", "H", "Gc", "G"]
    tp = tiers.TieredPass(st, mix, threads=4, direct=direct)
    for rep in range(2):
        ok = []
        say(f"[gpu] case tiers: mixed pass {rep}")
        tp.run(on_unit=lambda i, out: ok.append(store.check_unit(out, units_specs[i])))
        assert ok == [True] * len(units_specs)
    assert tp.run() > 0
    r = tiers.Rates(read_Bps=2e9, copy_Bps=50e9, restore_s=[1e-4] * len(st.units))
    total = sum(u.bytes for u in st.units)
    assert tiers.plan(st, 0, 0, r) == ["D"] * len(st.units)
    assert set(tiers.plan(st, 0, 10 * total, r)) == {"H"}
    assert set(tiers.plan(st, 10 * total, 10 * total, r)) == {"G"}
    p = tiers.plan(st, total // 2, 0, r)
    used = sum(u.bytes if t == "Gc" else (2 * u.n_values if t == "G" else 0) for u, t in zip(st.units, p))
    assert used <= total // 2 and "D" in p


def test_graph_replays_bit_exact():
    """Restores captured into one HIP graph (through torch.cuda.graph) and
    replayed: the library neither allocates nor clears memory on the stream,
    so its launches can be captured. Every replay restores into outputs that
    eager work has overwritten since the last one, and is checked bit for
    bit."""
    T = synth.TensorSpec
    specs = [T("g0", (700, 512), "normal", 901), T("g1", (4096,), "t4", 902), T("g2", (128, 4096), "normal", 903)]
    xs = [synth.generate(sp) for sp in specs]
    blobs = [oracle.encode(x, sp.shape) for x, sp in zip(xs, specs)]
    infos = [afx.afx_query(b) for b in blobs]
    dblobs = [afx.to_device(b) for b in blobs]
    outs = [torch.zeros(x.size, dtype=torch.int16, device="cuda") for x in xs]
    jobs = afx.make_jobs([(i, db.data_ptr(), o.data_ptr(), 2 * x.size) for i, db, o, x in zip(infos, dblobs, outs, xs)])
    refs = [torch.from_numpy(x.view(np.int16)).to("cuda") for x in xs]
    say("[gpu] case graph capture of a 3-tensor restore")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        afx.afx_decode_layer_async(jobs, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        afx.afx_decode_layer_async(jobs, torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        for o in outs:
            o.fill_(0x1234 + rep)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {rep}"


def test_two_streams_at_once():
    """Two batches restored at the same time on two streams (default
    priority): the library keeps no state between or during calls, so the
    launches may overlap; both come out bit-exact, three times over."""
    T = synth.TensorSpec
    sets = [[T(f"c{k}a", (1024, 2048), "normal", 950 + k), T(f"c{k}b", (300, 5120), "t4", 960 + k),
             T(f"c{k}c", (5000,), "normal", 970 + k)] for k in range(2)]
    jobsets, outsets, refsets, keep = [], [], [], []
    for specs in sets:
        xs = [synth.generate(sp) for sp in specs]
        blobs = [oracle.encode(x, sp.shape) for x, sp in zip(xs, specs)]
        infos = [afx.afx_query(b) for b in blobs]
        dblobs = [afx.to_device(b) for b in blobs]
        outs = [torch.zeros(x.size, dtype=torch.int16, device="cuda") for x in xs]
        jobsets.append(afx.make_jobs([(i, db.data_ptr(), o.data_ptr(), 2 * x.size)
                                      for i, db, o, x in zip(infos, dblobs, outs, xs)]))
        outsets.append(outs)
        refsets.append([torch.from_numpy(x.view(np.int16)).to("cuda") for x in xs])
        keep.append((infos, dblobs))
    say("[gpu] case two batches restored concurrently on two streams")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for outs in outsets:
            for o in outs:
                o.fill_(0x2345 + rep)
        torch.cuda.synchronize()
        for jobs, st in zip(jobsets, streams):
            with torch.cuda.stream(st):
                afx.afx_decode_layer_async(jobs, st.cuda_stream)
        torch.cuda.synchronize()
        for outs, refs in zip(outsets, refsets):
            for o, r in zip(outs, refs):
                assert torch.equal(o, r), f"pass {rep}"
