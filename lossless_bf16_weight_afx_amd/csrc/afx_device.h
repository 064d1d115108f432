// afx_device.h -- device pieces shared by the restore kernel and the fused
// restore-and-multiply kernel (gfx950): the decode table, the staging of a
// chunk's code words in LDS, the decoding chains, and the loads that feed
// them. Not installed; included by the .hip sources of libafx.
//
// A tensor's exponent codes come in chunks of 4096 elements, each starting at
// a recorded bit base, with the start of every 32-element group recorded as a
// gap from its chunk's base (the exponent field is the coded part: "Why
// Weight Offloading Slows Inference", section "Lossless compression").
#pragma once

#include <hip/hip_runtime.h>

#include "afx_index.h"
#include "afx_internal.h"

namespace afx {
namespace {


constexpr int kWave = 64;
constexpr int kWavesPerBlock = 16;  // one workgroup fills a CU (4 waves per SIMD)
constexpr int kWavesPerEU = 4;
constexpr int kSymbolWaves = 256 / kWave;  // waves that hold one exponent value per lane
constexpr int kThreads = kWave * kWavesPerBlock;
constexpr int kLutEntries = 1 << kMaxLen;  // 4096

struct TensorDesc {
    const uint8_t *code_len;
    const uint64_t *chunk_base;
    const uint16_t *gap;
    const uint8_t *signmant;
    const uint32_t *exp;
    uint16_t *out;
    uint64_t n;
    uint64_t exp_words;
    uint64_t last_word4;   // highest 4-aligned word index w with w + 4 <= exp_words
    uint32_t n_chunks;     // ceil(n / 4096)
    uint32_t blk_lo;       // workgroups [blk_lo, blk_hi) of the grid serve this tensor
    uint32_t blk_hi;
    uint32_t reserved;
};

struct LutScratch {
    uint32_t wave_count[kSymbolWaves][kMaxLen + 1];  // symbols of each length per wave
    uint32_t base[kMaxLen + 1];  // position in `sorted` of code 0 of each length, mod 2^32
    uint8_t sorted[256];         // used symbols in (length, value) order
};

// Per-wave LDS: the chunk's code words while decoding (kStageRow words,
// staged in reverse; afx_index.h), then its decoded exponent bytes (4 KB)
// while storing.
static_assert(kStageRow * 4 >= kChunk, "a stage slice also holds a chunk's exponent bytes");

// Rank of the k-th of nb workgroups that serve one tensor, counted XCD by
// XCD. The grid's workgroups go to the 8 XCDs in turn (workgroup b to XCD
// b mod 8) and each XCD has its own L2. Chunk c goes to rank c mod nb, so
// that neighbouring chunks, which share the cache lines at the ends of their
// code words, are mostly restored on one XCD and those lines are fetched
// once. A permutation of 0..nb-1.
__device__ inline uint32_t xcd_rank(uint32_t k, uint32_t nb) {
    constexpr uint32_t kXcds = 8;
    const uint32_t x = k % kXcds, i = k / kXcds;
    return x * (nb / kXcds) + min(x, nb % kXcds) + i;
}

// Order LDS traffic between lanes of one wave (no workgroup barrier needed).
__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bit 31 of a pair-table entry: both codes of the window fit in it (the
// pair table is described with its reads below).
constexpr uint32_t kPairBit = 0x80000000u;

// Build a decode table of one canonical code over the 12-bit windows of the
// stream (MSB first). !kPair: the one-code table, u16 entry i = (symbol <<
// 8) | length of the code word that starts window i; the length sits in the
// low bits so that a 32-bit shift by the whole entry consumes exactly the
// code (the hardware reads only the low 5 bits of a shift amount). kPair:
// the pair table (u32 entries, see pair_read), each entry computed from the
// codes of window i and of the window shifted past its first code. All
// kNThreads threads of the workgroup (256 or more) take part: thread s < 256
// owns symbol s and passes its code length (the others pass 0), then every
// thread s fills table entries [kPer s, kPer s + kPer), kPer = 4096 /
// kNThreads. Callers bracket it with barriers.
template <int kNThreads = kThreads, bool kPair = false>
__device__ void build_lut(uint32_t len, void *table, LutScratch &S) {
    static_assert(kNThreads >= 256 && kLutEntries % (4 * kNThreads) == 0, "4-entry blocks per thread");
    const int s = threadIdx.x;
    const int lane = s & (kWave - 1), wave = s / kWave;
    uint32_t rank = 0;  // among same-length symbols of this wave with smaller value
    len = used_length(len);  // only a corrupt blob has longer ones
    if (wave < kSymbolWaves) {
#pragma unroll
        for (uint32_t l = 1; l <= kMaxLen; ++l) {
            const uint64_t m = __ballot(len == l);
            if (len == l) rank = (uint32_t)__popcll(m & ((1ull << lane) - 1));
            if (lane == 0) S.wave_count[wave][l] = (uint32_t)__popcll(m);
        }
    }
    __syncthreads();

    // Every wave derives the canonical code in registers: lane l (1..12)
    // holds the number of symbols of length l (cnt) and of them in waves
    // before this one (below), the position of the first of them in
    // (length, value) order (start), their first code (first) and the end of
    // their slice of the 12-bit index space (limit).
    const uint32_t ll = (uint32_t)lane;
    uint32_t cnt = 0, below = 0;
    if (ll >= 1 && ll <= kMaxLen) {
#pragma unroll
        for (int w = 0; w < kSymbolWaves; ++w) {
            const uint32_t c = S.wave_count[w][ll];
            cnt += c;
            below += w < wave ? c : 0u;
        }
    }
    uint32_t start = 0, first = 0;
#pragma unroll
    for (uint32_t m = 1; m < kMaxLen; ++m) {
        const uint32_t cm = (uint32_t)__builtin_amdgcn_readlane((int)cnt, (int)m);
        if (m < ll) {
            start += cm;
            first += cm << (ll - m);  // first[l] = (first[l-1] + cnt[l-1]) << 1, unrolled
        }
    }
    const uint32_t limit = (first + cnt) << (kMaxLen - (ll <= kMaxLen ? ll : kMaxLen));
    // (all lanes active: a lane reads another lane's register)
    const uint32_t pos = (uint32_t)__shfl((int)start, (int)len) + (uint32_t)__shfl((int)below, (int)len) + rank;
    if (len) S.sorted[pos & 255] = (uint8_t)s;
    if (wave == 0 && ll >= 1 && ll <= kMaxLen) S.base[ll] = start - first;
    __syncthreads();

    // An entry's length is one more than the number of length slices that
    // end at or before it; its symbol follows from the code's distance to
    // that length's first code.
    uint32_t lim[kMaxLen];
#pragma unroll
    for (uint32_t q = 1; q < kMaxLen; ++q) lim[q] = (uint32_t)__builtin_amdgcn_readlane((int)limit, (int)q);
    auto entry = [&](uint32_t idx) -> uint32_t {
        const uint32_t l = entry_length(idx, lim);
        const uint32_t j = S.base[l] + (idx >> (kMaxLen - l));
        return ((uint32_t)S.sorted[j & 255] << 8) | l;
    };
    constexpr uint32_t kPer = kLutEntries / kNThreads;  // entries per thread
    if constexpr (kPair) {
        uint32_t *plut = static_cast<uint32_t *>(table);
#pragma unroll
        for (uint32_t k = 0; k < kPer; ++k) {
            const uint32_t i = (uint32_t)s * kPer + k;
            const uint32_t e1 = entry(i), l1 = e1 & 0xFF;
            const uint32_t e2 = entry((i << l1) & (kLutEntries - 1)), l2 = e2 & 0xFF;
            const bool both = l1 + l2 <= kMaxLen;
            plut[i] = (both ? l1 + l2 : l1) | (e1 & 0xFF00u) | (both ? (e2 & 0xFF00u) << 8 : 0u) | (l1 << 24) |
                      (both ? kPairBit : 0u);
        }
        return;
    }
    uint16_t *lut = static_cast<uint16_t *>(table);
    // a code of <= 10 bits owns whole 4-aligned blocks of the index space
    auto fill4 = [&](uint32_t i0) {
        const uint32_t e0 = entry(i0);
        if ((e0 & 0xFF) <= kMaxLen - 2) {
            const uint32_t d = e0 | (e0 << 16);
            *reinterpret_cast<uint2 *>(lut + i0) = make_uint2(d, d);
        } else {
            for (uint32_t j = 0; j < 4; ++j) lut[i0 + j] = (uint16_t)entry(i0 + j);
        }
    };
    if constexpr (kPer == 4) {
        fill4((uint32_t)s * 4);
    } else {
#pragma unroll
        for (uint32_t b = 0; b < kPer; b += 4) fill4((uint32_t)s * kPer + b);
    }
}

// Four BF16 values from the sign/mantissa bytes b and exponent bytes e of
// four consecutive elements (byte k of each word: element k). BF16 is
// s | e | m (1, 8 and 7 bits): its high byte is (s << 7) | (e >> 1) and its
// low byte ((e & 1) << 7) | m. One bitfield select forms the four high
// bytes, one the four low bytes (bits shifted across a byte boundary land
// only where the mask takes the other operand), and two byte permutes
// interleave them: w01 holds elements 0 (low half) and 1, w23 elements 2, 3.
__device__ inline void join4(uint32_t b, uint32_t e, uint32_t &w01, uint32_t &w23) {
    const uint32_t hi = (b & 0x80808080u) | ((e >> 1) & 0x7F7F7F7Fu);
    const uint32_t lo = ((e << 7) & 0x80808080u) | (b & 0x7F7F7F7Fu);
    w01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    w23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// Symbols (byte 1 of two table entries) packed as bytes 0,1 of a word.
__device__ inline uint32_t sym_pair(uint32_t e1, uint32_t e2) { return __builtin_amdgcn_perm(e2, e1, 0x0c0c0501u); }
// Bytes 0,1 of lo and of hi as the four bytes of a word.
__device__ inline uint32_t join_halves(uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x05040100u); }

__device__ inline uint32_t lookup(const uint16_t *lut, uint32_t win) { return lut[one_code_index(win)]; }

// One decoding chain. With P the bit position in the staged words (MSB
// first), the chain keeps r = 32 * kRev - P. Then the next 32 stream bits are
// the funnel shift of staged words [r/32 + 1] (high) and [r/32] (low) by
// r mod 32, and consuming a code of length l is r -= l. The two staged words
// of the window and the word after them are kept in registers, the next word
// read one step ahead, so forming a window never waits for LDS. Two chains
// advance together so that their table reads overlap.
struct BufChain {
    uint32_t r, q, hi, lo, nx;  // q = r / 32: hi, lo, nx are staged words q + 1, q, q - 1
};

__device__ inline BufChain buf_chain(const uint32_t *stage, uint32_t r) {
    const uint32_t *p = stage + chain_word(r);
    return BufChain{r, chain_word(r), p[1], p[0], p[-1]};
}

// Consume d bits (at most 24, so the window moves by at most one word).
// The word index itself tells whether the window moved, and addresses the
// word read ahead.
__device__ inline void buf_advance(BufChain &c, const uint32_t *stage, uint32_t d) {
    c.r -= d;
    const uint32_t q = chain_word(c.r);
    const bool moved = q != c.q;
    c.q = q;
    c.hi = moved ? c.lo : c.hi;
    c.lo = moved ? c.nx : c.lo;
    c.nx = stage[q - 1];
}

// Two symbols per chain through the one-code table, two dependent table
// reads per step; sa, sb: the symbols as bytes 0, 1. (The MFMA product, with
// two waves per SIMD, measured about 5% slower with the pair table below,
// also when that table was built as cheaply as the one-code table.)
__device__ inline void buf_chain_pairs(BufChain &a, BufChain &b, const uint32_t *stage, const uint16_t *lut,
                                       uint32_t &sa, uint32_t &sb) {
    const uint32_t wa = __builtin_amdgcn_alignbit(a.hi, a.lo, a.r);
    const uint32_t wb = __builtin_amdgcn_alignbit(b.hi, b.lo, b.r);
    const uint32_t a1 = lookup(lut, wa), b1 = lookup(lut, wb);
    const uint32_t a2 = lookup(lut, wa << (a1 & 31)), b2 = lookup(lut, wb << (b1 & 31));
    buf_advance(a, stage, (a1 + a2) & 0xFF);
    buf_advance(b, stage, (b1 + b2) & 0xFF);
    sa = sym_pair(a1, a2);
    sb = sym_pair(b1, b2);
}

// A second table over the same 12-bit windows (build_lut<.., true>). Entry
// i (32 bits) describes the codes that start window i:
//   byte 0   bits to consume: both codes' lengths when the second code also
//            ends inside the window, else the first code's length;
//   byte 1   the first code's symbol;
//   byte 2   the second code's symbol (when both fit, else 0);
//   byte 3   bits 0-3: the first code's length; bit 7: both codes fit.
// With mean code lengths near 2.6 bits, two codes fit in 12 bits for about
// 99.6% of windows, so most two-symbol steps take one table read instead of
// two dependent ones. The restore and the matrix-vector kernel decode
// through it: the restore's first and last chunks, and all of the fused
// kernel's, are bound by the decode.
// A pair entry whose window holds only one whole code, completed by the
// entry e2 of the window shifted past that code.
__device__ inline uint32_t complete_entry(uint32_t e, uint32_t e2) {
    return (e & 0xFF00u) | ((e2 & 0xFF00u) << 8) | ((e & 0xFFu) + ((e2 >> 24) & 0xFu));
}

// The paired chains run kLead bits behind the code they decode: their
// 32-bit window starts with kLead bits already consumed (or, at a chunk's
// first bit, the pad word above the staged words), so that the next 12
// code bits sit at bits 29..18 of the window, and the pair table's byte
// address (index times 4) is the window's high half-word masked: one
// instruction.
static_assert(kMaxLen + kLead + 2 == 16, "the table address is a masked high half-word");
__device__ inline uint32_t pair_read(const uint32_t *plut, uint32_t win) {
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(plut) + pair_offset(win));
}

// The buffered chains (BufChain, kLead bits behind) advanced through the
// pair table. Both chains' table reads are issued before the (rare) branch
// that completes entries holding one code, so that their latencies overlap.
// ea, eb: the entries (byte 0: bits consumed; bytes 1, 2: the two symbols).
__device__ inline void pair_chain_steps(BufChain &a, BufChain &b, const uint32_t *stage, const uint32_t *plut,
                                        uint32_t &ea, uint32_t &eb) {
    const uint32_t wa = __builtin_amdgcn_alignbit(a.hi, a.lo, a.r);
    const uint32_t wb = __builtin_amdgcn_alignbit(b.hi, b.lo, b.r);
    ea = pair_read(plut, wa);
    eb = pair_read(plut, wb);
    if ((int32_t)(ea & eb) >= 0) {  // some entry holds one code: read the second
        const uint32_t fa = pair_read(plut, wa << (ea & 31));
        const uint32_t fb = pair_read(plut, wb << (eb & 31));
        ea = (int32_t)ea >= 0 ? complete_entry(ea, fa) : ea;
        eb = (int32_t)eb >= 0 ? complete_entry(eb, fb) : eb;
    }
    buf_advance(a, stage, ea & 0xFF);
    buf_advance(b, stage, eb & 0xFF);
}

// The symbols (bytes 1, 2) of two pair entries, first then second, as the
// four bytes of a word.
__device__ inline uint32_t join_entries(uint32_t first, uint32_t second) {
    return __builtin_amdgcn_perm(second, first, 0x06050201u);
}

// The first 512 staged words of a chunk travel through registers so that
// their loads can be issued one chunk ahead; longer chunks (more than about
// 4 bits per element) fetch the rest when they are staged.
constexpr uint32_t kPrefetchWords = 2 * 4 * kWave;

struct StreamRegs {
    uint4 v[2];
};

// Four stream words from 4-aligned index g (clamped to the section).
__device__ inline uint4 load_words4(const TensorDesc &T, uint64_t g) {
    return *reinterpret_cast<const uint4 *>(T.exp + word4_index(g, T.last_word4));
}

// Only the words the chunk needs are requested (typical chunks need ~350).
__device__ inline void load_stream(const TensorDesc &T, const ChunkGeom &g, int lane, StreamRegs &s) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t i = 4 * (uint32_t)lane + (uint32_t)k * 4 * kWave;
        if (i < g.nwords) s.v[k] = load_words4(T, g.w0 + i);
    }
}

// Stream word i goes to index kRev - i (reversed; see Chain).
__device__ inline void put_words4(uint32_t *stage, uint32_t i, uint4 v) {
    *reinterpret_cast<uint4 *>(stage + stage_put_index(i)) = make_uint4(v.w, v.z, v.y, v.x);
}

__device__ inline void put_stream(const TensorDesc &T, const ChunkGeom &g, const StreamRegs &s, uint32_t *stage,
                                  int lane) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t i = 4 * (uint32_t)lane + (uint32_t)k * 4 * kWave;
        if (i < g.nwords) put_words4(stage, i, s.v[k]);
    }
    for (uint32_t i = kPrefetchWords + 4 * (uint32_t)lane; i < g.nwords; i += 4 * kWave)
        put_words4(stage, i, load_words4(T, g.w0 + i));
}

__device__ inline uint32_t readlane(uint32_t v, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)v, l); }

// Chunk bases are fetched with a vector load (lane 0: start, lane 1: end of
// chunk lc) so that waiting for them never involves the LDS counter.
__device__ inline uint64_t load_bases(const TensorDesc &T, uint64_t lc, int lane) {
    return T.chunk_base[lc + (uint64_t)(lane & 1)];
}
__device__ inline ChunkGeom geom_from_lanes(uint64_t v) {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const uint64_t base = ((uint64_t)readlane(hi, 0) << 32) | readlane(lo, 0);
    const uint64_t end = ((uint64_t)readlane(hi, 1) << 32) | readlane(lo, 1);
    return chunk_geom(base, end);
}

struct Gaps {
    uint32_t a, b;  // start of groups lane and lane + 64, relative to the chunk
};

// Groups past the end of a short last chunk take the last group's gap: they
// decode something, but nothing they decode is stored.
__device__ inline Gaps load_gaps(const TensorDesc &T, uint64_t lc, int lane) {
    const uint32_t ng = chunk_groups(T.n, lc);
    const uint16_t *gap = T.gap + lc * kGroupsPerChunk;
    // read once: not kept in the caches
    return Gaps{__builtin_nontemporal_load(gap + gap_slot((uint32_t)lane, ng)),
                __builtin_nontemporal_load(gap + gap_slot((uint32_t)lane + kWave, ng))};
}

// 16 output bytes; the output is written once and not read back here, so the
// stores bypass cache allocation (each store instruction covers whole lines).
__device__ inline void store_out(uint16_t *p, uint4 v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(p));
}

// Decode a staged chunk's 4096 exponent codes through the pair table and
// leave the exponent bytes in element order at the start of `stage` (which
// held the code words). Chain starts are clamped (chain_r0) so that the
// chains stay inside the staged words and the pad word above even on a
// corrupt gap.
__device__ inline void decode_exponents(const ChunkGeom &g, const Gaps &gaps, const uint32_t *plut,
                                               uint32_t *stage, int lane) {
    const uint32_t ra = chain_r0(g.rel, gaps.a);
    const uint32_t rb = chain_r0(g.rel, gaps.b);
    uint32_t wa[8], wb[8];
    BufChain A = buf_chain(stage, ra), B = buf_chain(stage, rb);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        uint32_t a01, b01, a23, b23;
        pair_chain_steps(A, B, stage, plut, a01, b01);
        pair_chain_steps(A, B, stage, plut, a23, b23);
        wa[q] = join_entries(a01, a23);
        wb[q] = join_entries(b01, b23);
    }
    wave_sync();  // every lane is done reading the staged words
    uint4 *pa = reinterpret_cast<uint4 *>(stage + lane * 8);
    uint4 *pb = reinterpret_cast<uint4 *>(stage + (lane + kWave) * 8);
    pa[0] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
    pa[1] = make_uint4(wa[4], wa[5], wa[6], wa[7]);
    pb[0] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
    pb[1] = make_uint4(wb[4], wb[5], wb[6], wb[7]);
    wave_sync();
}

}  // namespace
}  // namespace afx
