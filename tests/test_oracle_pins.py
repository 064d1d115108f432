"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what it pins: closed forms, brute force, textbook special
cases, and the figures printed on the pages.
"""
import heapq
import itertools
import math

import numpy as np
import pytest

import oracle
from conftest import read_golden
from lossless_bf16_weight_afx_amd import ready, synth


def bits_of(x):
    return np.asarray(x, dtype=np.uint16)


def roundtrip(x, threads=(1, 4)):
    x = bits_of(x)
    blob = oracle.encode(x)
    for t in threads:
        y = oracle.decode(blob, threads=t)
        assert y.dtype == np.uint16 and y.size == x.size
        assert np.array_equal(y, x.ravel()), f"round trip differs (threads={t})"
    return blob


def cost(freq, lens):
    return int(sum(int(f) * int(l) for f, l in zip(freq, lens)))


# ---------------------------------------------------------------------------
# P-RT: decode(encode(x)) == x bit for bit (the coding is lossless: page 2,
# section "Lossless compression").
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [0, 1, 31, 32, 33, 128, 4095, 4096, 4097, 5120, 3 * 4096 + 17])
def test_roundtrip_sizes(n):
    rng = np.random.default_rng(n + 11)
    x = synth.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32) * np.float32(0.02))
    roundtrip(x)


def test_roundtrip_special_patterns():
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x0001, 0x807F,
                         0x0080, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80], np.uint16)
    x = np.tile(specials, 300)
    np.random.default_rng(3).shuffle(x)
    roundtrip(x)


def test_roundtrip_all_zero_and_constant():
    blob = roundtrip(np.zeros(10000, np.uint16))
    s = oracle.sections(blob)
    assert s["header"]["n_symbols"] == 1 and s["code_len"][0] == 1
    assert s["header"]["total_bits"] == 10000  # one bit per element
    roundtrip(np.full(4097, 0x3F80, np.uint16))


def test_roundtrip_c1_tensor():
    x = synth.generate(synth.single_tensor()[0])
    roundtrip(x, threads=(1, 8))


def test_roundtrip_heavy_tail_sample():
    spec = synth.TensorSpec("t", (1 << 20,), "t4", 4)
    roundtrip(synth.generate(spec))


def test_decode_chunk_range_matches_whole():
    x = synth.generate(synth.TensorSpec("t", (10 * 4096 + 100,), "normal", 9))
    blob = oracle.encode(x)
    part = oracle.decode_chunks(blob, 3, 11, threads=3)
    assert np.array_equal(part, x[3 * 4096:])


def test_corrupt_gap_is_detected():
    x = synth.generate(synth.TensorSpec("t", (8192,), "normal", 5))
    blob = oracle.encode(x).copy()
    s = oracle.sections(blob)
    s["gap"][5] += 1
    with pytest.raises(oracle.OracleError):
        oracle.decode(blob)


# ---------------------------------------------------------------------------
# P-K: Kraft equality, and every 12-bit window maps to exactly one codeword.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_kraft_equality_and_prefix_partition(seed):
    spec = synth.TensorSpec("t", (1 << 18,), "t4" if seed == 3 else "normal", seed)
    blob = oracle.encode(synth.generate(spec))
    lens = oracle.sections(blob)["code_len"].astype(int)
    used = lens[lens > 0]
    assert used.size >= 2 and used.max() <= 12
    assert sum(1 << (12 - l) for l in used) == 4096
    codes = oracle.canonical_codes(lens)
    owner = np.full(4096, -1)
    for s in np.nonzero(lens)[0]:
        lo = int(codes[s]) << (12 - lens[s])
        hi = (int(codes[s]) + 1) << (12 - lens[s])
        assert np.all(owner[lo:hi] == -1)
        owner[lo:hi] = s
    assert np.all(owner >= 0)


# ---------------------------------------------------------------------------
# P-BF: package-merge is optimal under the limit. Brute force over every
# length vector (small cases), and over length multisets assigned by the
# rearrangement inequality (larger cases).
# ---------------------------------------------------------------------------
def brute_force_product(freq, lmax):
    best = None
    for lens in itertools.product(range(1, lmax + 1), repeat=len(freq)):
        if sum(2.0 ** -l for l in lens) <= 1.0:
            c = cost(freq, lens)
            best = c if best is None or c < best else best
    return best


def brute_force_multiset(freq, lmax):
    f = sorted(freq, reverse=True)
    best = None
    for lens in itertools.combinations_with_replacement(range(1, lmax + 1), len(f)):
        if sum(2.0 ** -l for l in lens) <= 1.0:
            c = sum(a * b for a, b in zip(f, lens))  # lens ascending, freq descending
            best = c if best is None or c < best else best
    return best


@pytest.mark.parametrize("m,lmax", [(2, 2), (3, 2), (4, 2), (4, 3), (5, 3), (5, 4), (6, 3), (4, 4)])
def test_package_merge_optimal_bruteforce_product(m, lmax):
    rng = np.random.default_rng(100 * m + lmax)
    for _ in range(15):
        freq = rng.integers(1, 2 ** 32, size=m, dtype=np.uint64)
        lens = oracle.code_lengths(freq, lmax)
        assert lens.max() <= lmax and lens.min() >= 1
        assert sum(2.0 ** -int(l) for l in lens) == 1.0
        assert cost(freq, lens) == brute_force_product([int(v) for v in freq], lmax)


@pytest.mark.parametrize("m,lmax", [(6, 12), (7, 12), (7, 4), (7, 3)])
def test_package_merge_optimal_bruteforce_multiset(m, lmax):
    rng = np.random.default_rng(7 * m + lmax)
    for _ in range(10):
        # skewed frequencies so that the limit binds in some draws
        freq = (rng.pareto(0.7, size=m) * 1000 + 1).astype(np.uint64)
        lens = oracle.code_lengths(freq, lmax)
        assert cost(freq, lens) == brute_force_multiset([int(v) for v in freq], lmax)


def test_limit_below_log2_alphabet_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.code_lengths(np.ones(5, np.uint64), 2)  # 2^2 < 5 symbols
    oracle.code_lengths(np.ones(4, np.uint64), 2)


def dp_optimal_limited(freq, lmax):
    """Exact length-limited optimum by dynamic programming over tree levels.

    With weights sorted in decreasing order, optimal lengths are
    non-decreasing. At each depth some of the open nodes become leaves for the
    next symbols; the others split into two nodes one level deeper.
    """
    w = sorted((int(v) for v in freq if v > 0), reverse=True)
    m = len(w)
    prefix = [0]
    for v in w:
        prefix.append(prefix[-1] + v)
    inf = float("inf")
    memo = {}

    def best(depth, i, slots):
        if i == m:
            return 0
        if depth > lmax or slots == 0:
            return inf
        key = (depth, i, slots)
        if key in memo:
            return memo[key]
        r = inf
        for t in range(0, min(slots, m - i) + 1):
            here = (prefix[i + t] - prefix[i]) * depth
            nxt = min(2 * (slots - t), m - i - t)
            r = min(r, here + best(depth + 1, i + t, nxt))
        memo[key] = r
        return r

    return best(1, 0, 2)


@pytest.mark.parametrize("seed", range(6))
def test_package_merge_matches_level_dp(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(8, 40))
    freq = (rng.pareto(0.5, size=m) * 100 + 1).astype(np.uint64)
    for lmax in (6, 8, 12):
        if (1 << lmax) < m:
            continue
        lens = oracle.code_lengths(freq, lmax)
        assert cost(freq, lens) == dp_optimal_limited(freq, lmax)


# ---------------------------------------------------------------------------
# P-X65536: the tensor of all 65,536 BF16 patterns. Every exponent occurs 256
# times, so the unique optimum is length 8 for all symbols and the canonical
# code of a symbol is the symbol itself: the stream is the exponent bytes,
# MSB first, and every section is predictable in closed form.
# ---------------------------------------------------------------------------
def test_all_patterns_closed_form():
    x = np.arange(65536, dtype=np.uint16)
    blob = roundtrip(x)
    s = oracle.sections(blob)
    h = s["header"]
    assert h["magic"] == b"AFX1" and h["version"] == 1 and h["n"] == 65536
    assert (h["chunk"], h["group"], h["lmax"], h["n_symbols"]) == (4096, 32, 12, 256)
    assert h["total_bits"] == 65536 * 8 and h["exp_words"] == 65536 // 4 + 4
    assert np.all(s["code_len"] == 8)
    assert np.array_equal(s["chunk_base"], np.arange(17, dtype=np.uint64) * 32768)
    assert np.array_equal(s["gap"], (np.arange(2048) % 128 * 256).astype(np.uint16))
    i = np.arange(65536)
    assert np.array_equal(s["signmant"], (((i >> 8) & 0x80) | (i & 0x7F)).astype(np.uint8))
    e = ((i >> 7) & 0xFF).astype(np.uint32).reshape(-1, 4)
    words = (e[:, 0] << 24) | (e[:, 1] << 16) | (e[:, 2] << 8) | e[:, 3]
    assert np.array_equal(s["exp"][:16384], words)
    assert np.all(s["exp"][16384:] == 0)
    off = s["offsets"]
    # worked by hand: 17 u64 bases end at 648 -> 768; 2048 u16 gaps end at
    # 4864; 65536 sign/mantissa bytes end at 70400; 16388 words end at 135952
    assert off == {"code_len": 256, "chunk_base": 512, "gap": 768, "signmant": 4864,
                   "exp": 70400, "blob_bytes": 136192}
    assert blob.size == off["blob_bytes"]
    assert np.all(blob[96:256] == 0) and np.all(blob[512 + 17 * 8:768] == 0)


def test_small_blob_offsets_by_hand():
    # 33 equal exponents: one symbol of length 1, 33 stream bits, 2 chunk
    # bases + 1 end (24 B), 2 gaps, 33 bytes, ceil(33/32) + 4 = 6 words.
    blob = roundtrip(np.full(33, 0x3F80, np.uint16))
    s = oracle.sections(blob)
    assert s["offsets"] == {"code_len": 256, "chunk_base": 512, "gap": 768, "signmant": 1024,
                            "exp": 1280, "blob_bytes": 1536}
    assert list(s["chunk_base"]) == [0, 33] and list(s["gap"]) == [0, 32]
    assert list(s["exp"]) == [0, 0, 0, 0, 0, 0]  # the only code is a single 0 bit


# ---------------------------------------------------------------------------
# P-DY: dyadic frequencies give lengths -log2 p exactly; mean length = entropy.
# ---------------------------------------------------------------------------
def test_dyadic_lengths_equal_entropy():
    exps = np.array([127] * 2048 + [126] * 1024 + [120] * 512 + [130] * 512, np.uint16)
    np.random.default_rng(0).shuffle(exps)
    x = (exps << 7) | np.uint16(0x25)
    blob = roundtrip(x)
    s = oracle.sections(blob)
    lens = s["code_len"]
    assert (lens[127], lens[126], lens[120], lens[130]) == (1, 2, 3, 3)
    entropy_bits = 4096 * (0.5 * 1 + 0.25 * 2 + 0.125 * 3 + 0.125 * 3)
    assert s["header"]["total_bits"] == entropy_bits


# ---------------------------------------------------------------------------
# P-FIB: Fibonacci frequencies drive unconstrained Huffman to depth m-1; the
# 12-bit limit binds and package-merge still reaches the optimum.
# ---------------------------------------------------------------------------
def huffman_depths(freq):
    heap = [(int(f), i, [i]) for i, f in enumerate(freq)]
    heapq.heapify(heap)
    depth = [0] * len(freq)
    uid = len(freq)
    while len(heap) > 1:
        a, _, sa = heapq.heappop(heap)
        b, _, sb = heapq.heappop(heap)
        for s in sa + sb:
            depth[s] += 1
        heapq.heappush(heap, (a + b, uid, sa + sb))
        uid += 1
    return depth


def test_fibonacci_limit_binds():
    fib = [1, 1]
    while len(fib) < 20:
        fib.append(fib[-1] + fib[-2])
    assert max(huffman_depths(fib)) == 19
    lens = oracle.code_lengths(np.array(fib, np.uint64), 12)
    assert lens.max() == 12
    assert sum(1 << (12 - int(l)) for l in lens) == 4096
    assert cost(fib, lens) == dp_optimal_limited(fib, 12)
    # unconstrained (limit 32) equals Huffman's cost
    free = oracle.code_lengths(np.array(fib, np.uint64), 32)
    assert cost(fib, free) == cost(fib, huffman_depths(fib))


# ---------------------------------------------------------------------------
# P-H: the generator's exponent histogram against its closed form. A value
# x ~ N(0, s) rounds (to nearest even) to exponent field k exactly when
# 2^(k-127)(1-2^-9) <= |x| < 2^(k-126)(1-2^-9).
# ---------------------------------------------------------------------------
def normal_exponent_pmf(k, sigma):
    def cdf(v):
        return 0.5 * (1.0 + math.erf(v / (sigma * math.sqrt(2.0))))
    lo = 2.0 ** (k - 127) * (1 - 2.0 ** -9)
    hi = 2.0 ** (k - 126) * (1 - 2.0 ** -9)
    return 2.0 * (cdf(hi) - cdf(lo))


def test_generator_histogram_closed_form():
    x = synth.generate(synth.TensorSpec("t", (1 << 20,), "normal", 77))
    e = (x >> 7) & 0xFF
    n = x.size
    hist = np.bincount(e, minlength=256)
    for k in range(100, 128):
        p = normal_exponent_pmf(k, 0.02)
        sd = math.sqrt(n * p * (1 - p)) + 1
        assert abs(hist[k] - n * p) < 6 * sd, (k, hist[k], n * p)
    assert abs(normal_exponent_pmf(121, 0.02) - 0.3167) < 1e-3
    assert abs(normal_exponent_pmf(120, 0.02) - 0.2611) < 1e-3
    assert abs(normal_exponent_pmf(122, 0.02) - 0.1171) < 1e-3


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 0.0], np.float32)
    assert list(synth.f32_to_bf16_bits(f)) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000]


# ---------------------------------------------------------------------------
# P-R: whole-blob ratio near the pages' 20.3 / 29.5 (page 2, "Lossless
# compression"), and Shannon's bound H <= mean code length.
# ---------------------------------------------------------------------------
def test_ratio_near_pages_and_entropy_bounds():
    g = read_golden("time_to_ready.txt")
    pages_ratio = g["stored_GB"] / g["model_GB"]
    assert abs(pages_ratio - 0.688) < 1e-3
    x = synth.generate(synth.TensorSpec("t", (1 << 22,), "normal", 12))
    blob = oracle.encode(x)
    ratio = blob.size / (2 * x.size)
    assert 0.66 < ratio < 0.72 and abs(ratio - pages_ratio) < 0.02
    p = np.bincount((x >> 7) & 0xFF, minlength=256) / x.size
    H = -sum(v * math.log2(v) for v in p if v > 0)
    mean_len = oracle.sections(blob)["header"]["total_bits"] / x.size
    assert H <= mean_len < H + 1
    assert mean_len - H < 0.1  # the 12-bit limit costs little here


# ---------------------------------------------------------------------------
# P-SZ: the synthetic shapes reproduce the page's per-part weight counts
# (page 1, Tables 2 and 4) through the parameter-count formula of page 4.
# ---------------------------------------------------------------------------
def test_sizes_match_pages():
    g = read_golden("qwen3_14b_sizes.txt")
    assert (synth.VOCAB, synth.HIDDEN, synth.N_LAYERS) == (g["vocab_size"], g["hidden_size"], g["num_hidden_layers"])
    assert (synth.N_HEADS, synth.N_KV_HEADS, synth.HEAD_DIM) == (
        g["num_attention_heads"], g["num_key_value_heads"], g["head_dim"])
    layer = sum(t.numel for t in synth.decoder_layer(0))
    h, dh, a, akv, dff = synth.HIDDEN, synth.HEAD_DIM, synth.N_HEADS, synth.N_KV_HEADS, synth.FFN
    formula = h * (a * dh + 2 * akv * dh) + a * dh * h + 3 * h * dff + 2 * h + 2 * dh
    assert layer == formula == 330_311_936
    assert round(layer / 1e6) == g["layer_weights_M"]
    assert round(layer * g["bytes_per_weight"] / 1e9, 2) == g["layer_GB"]
    emb = synth.embedding()[0].numel
    assert round(emb / 1e6) == g["embedding_weights_M"] == g["head_weights_M"]
    assert round(emb * 2 / 1e9, 1) == g["embedding_GB"]
    units = synth.model_units()
    total = sum(t.numel for u in units for t in u)
    assert round(total / 1e9, 1) == g["total_weights_B"]
    assert round(total * 2 / 1e9, 1) == g["total_GB"]
    assert round(40 * layer / 1e9, 1) == g["all_layers_B"]
    assert round(40 * layer * 2 / 1e9, 1) == g["all_layers_GB"]


# ---------------------------------------------------------------------------
# P-E: the reading of page 2's Eq. (1) and Eq. (2) reproduces the figures the
# page derives from them.
# ---------------------------------------------------------------------------
def test_time_to_ready_reading():
    g = read_golden("time_to_ready.txt")
    read_layer = ready.t_prep(g["layer_GB"], g["b_disk_GBps"], 0.0, 0.0, g["b_pcie_GBps"])
    copy_layer = ready.t_prep(0.0, g["b_disk_GBps"], 0.0, g["layer_GB"], g["b_pcie_GBps"])
    assert round(read_layer, 2) == g["layer_read_s"]
    assert round(copy_layer, 2) == g["layer_copy_s"]
    assert round(ready.t_prep(g["model_GB"], g["b_disk_GBps"], 0.0, 0.0, 1.0)) == g["model_read_s"]
    assert ready.t_prep(0.0, 1.0, 0.0, g["model_GB"], g["b_pcie_GBps"]) < g["model_copy_s_below"]
    saving = (g["model_GB"] - g["stored_GB"]) / g["b_disk_GBps"]
    assert round(saving) == g["read_saving_s"]
    assert ready.compression_pays(g["model_GB"], g["stored_GB"], g["b_disk_GBps"], saving - 0.1)
    assert not ready.compression_pays(g["model_GB"], g["stored_GB"], g["b_disk_GBps"], saving + 0.1)
