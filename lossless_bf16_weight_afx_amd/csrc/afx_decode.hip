// afx_decode.hip -- the GPU restore of losslessly coded BF16 weights (gfx950).
//
// "Why Weight Offloading Slows Inference" (section "Three steps for each
// weight", Eq. (1)) names the unpack time t_unpack that every compressed
// weight pays before use; section "Lossless compression" codes the BF16
// exponent with shorter codes for common values and restores the released
// bits before compute. Here that unpack runs on the GPU after the compressed
// bytes reach device memory.
//
// Work decomposition (one launch per batch of up to 32 tensors):
//   * one workgroup of 16 wave64s fills a CU (4 waves per SIMD). The grid
//     is split among the batch's tensors in proportion to their chunk
//     (4096-element) counts, so a workgroup serves about one tensor; within
//     a tensor the chunks go round its workgroups, so that all of them move
//     through each array together, in one narrow band;
//   * the waves of a workgroup claim its chunks one at a time from a counter
//     in LDS. A SIMD issues for its oldest waves first, so waves run at
//     different speeds; claiming keeps them finishing together;
//   * for every tensor it serves, the workgroup builds the 4096-entry decode
//     table (u16: symbol << 8 | length) of that tensor's canonical code in
//     LDS, from the 256 code lengths alone;
//   * each wave restores one chunk at a time, software-pipelined: while chunk
//     i decodes, the code words and gap offsets of chunk i + 1 and the bit
//     bases of chunk i + 2 are in flight. The code words are staged in the
//     wave's own LDS slice; lane j then decodes groups j and j + 64 (32
//     symbols each, two independent dependency chains), two symbols per
//     32-bit window of the staged stream;
//   * decoded exponent bytes go back to the wave's LDS slice in element order;
//     the wave re-reads them in store order, merges them with the
//     sign/mantissa bytes and writes 16-byte stores, 1 KB per instruction.
// There is no floating point and no matrix work: the kernel is bound by HBM
// bytes and by the serial table-lookup chain of each lane.
#include <hip/hip_runtime.h>

#include <atomic>

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

struct Batch {
    TensorDesc t[AFX_MAX_JOBS_PER_LAUNCH];
    uint32_t n_tensors;
};

struct LutScratch {
    uint32_t wave_count[kSymbolWaves][kMaxLen + 1];  // symbols of each length per wave
    uint32_t base[kMaxLen + 1];  // position in `sorted` of code 0 of each length, mod 2^32
    uint8_t sorted[256];         // used symbols in (length, value) order
};

// Per-wave LDS: the chunk's code words while decoding, then its decoded
// exponent bytes (4 KB) while storing. A chunk spans at most 4096 * 12 bits;
// add the alignment slack of the start and the over-read of the last group.
// Words are staged in reverse order (stream word j at index kRev - j), plus
// one pad word above, so that one counter gives both the LDS address and the
// funnel-shift amount of a 32-bit window (see Chain).
constexpr uint32_t kStageWords = 1568;
constexpr uint32_t kRev = kStageWords - 1;  // == 3 (mod 4): 16-byte aligned reversed stores
static_assert(kRev % 4 == 3, "reversed staging needs kRev = 3 mod 4");
// Each wave's slice, with the pad word, rounded up to 16 bytes so that every
// slice starts 16-byte aligned.
constexpr uint32_t kStageRow = (kStageWords + 1 + 3) & ~3u;

// Order LDS traffic between lanes of one wave (no workgroup barrier needed).
__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Build the decode table of one canonical code: entry i (a 12-bit window of
// the stream, MSB first) holds (symbol << 8) | length of the code word that
// starts the window. The length sits in the low bits so that a 32-bit shift
// by the whole entry consumes exactly the code (the hardware reads only the
// low 5 bits of a shift amount). All 1024 threads take part: thread s < 256
// owns symbol s and passes its code length (the others pass 0), then every
// thread s fills table entries [4 s, 4 s + 4). Callers bracket it with
// barriers.
__device__ void build_lut(uint32_t len, uint16_t *lut, LutScratch &S) {
    const int s = threadIdx.x;
    const int lane = s & (kWave - 1), wave = s / kWave;
    uint32_t rank = 0;  // among same-length symbols of this wave with smaller value
    if (len > kMaxLen) len = 0;  // only a corrupt blob gets here; treat as unused
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
        uint32_t l = 1;
#pragma unroll
        for (uint32_t q = 1; q < kMaxLen; ++q) l += idx >= lim[q] ? 1u : 0u;
        const uint32_t j = S.base[l] + (idx >> (kMaxLen - l));
        return ((uint32_t)S.sorted[j & 255] << 8) | l;
    };
    constexpr uint32_t kPer = kLutEntries / kThreads;  // 4 entries per thread
    const uint32_t i0 = (uint32_t)s * kPer;
    const uint32_t e0 = entry(i0);
    if ((e0 & 0xFF) <= kMaxLen - 2) {
        // a code of <= 10 bits owns whole 4-aligned blocks of the index space
        const uint32_t d = e0 | (e0 << 16);
        *reinterpret_cast<uint2 *>(lut + i0) = make_uint2(d, d);
    } else {
        for (uint32_t j = 0; j < kPer; ++j) lut[i0 + j] = (uint16_t)entry(i0 + j);
    }
}

// Two BF16 values from the sign/mantissa bytes b and exponent bytes e of
// elements 0,1 (kHigh: of elements 2,3). With v = [e1 b1 e0 b0], each 16-bit
// half of v is (e << 8) | (s << 7) | m; the result half is
// (s << 15) | (e << 7) | m.
template <bool kHigh>
__device__ inline uint32_t join_pair(uint32_t b, uint32_t e) {
    // b2, e2: the two elements' bytes in 16-bit lanes. The result half is
    // (e << 7) + m + (s << 15) = (e << 7) + b + 255 * (b & 0x80), and no
    // half overflows into the next.
    constexpr uint32_t sel = kHigh ? 0x0c030c02u : 0x0c010c00u;
    const uint32_t b2 = __builtin_amdgcn_perm(0u, b, sel);
    const uint32_t e2 = __builtin_amdgcn_perm(0u, e, sel);
    return (e2 << 7) + (__umul24(b2 & 0x00800080u, 255u) + b2);
}

// Symbols (byte 1 of two table entries) packed as bytes 0,1 of a word.
__device__ inline uint32_t sym_pair(uint32_t e1, uint32_t e2) { return __builtin_amdgcn_perm(e2, e1, 0x0c0c0501u); }
// Bytes 0,1 of lo and of hi as the four bytes of a word.
__device__ inline uint32_t join_halves(uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x05040100u); }

// One decoding chain. With P the bit position in the staged words (MSB
// first), the chain keeps r = 32 * kRev - P. Then the next 32 stream bits are
// the funnel shift of staged words [r/32 + 1] (high) and [r/32] (low) by
// r mod 32, and consuming a code of length l is r -= l.
struct Chain {
    uint32_t r;
};

__device__ inline uint32_t window(const uint32_t *stage, uint32_t r) {
    const uint32_t *p = stage + (r >> 5);
    return __builtin_amdgcn_alignbit(p[1], p[0], r);
}

__device__ inline uint32_t lookup(const uint16_t *lut, uint32_t win) { return lut[win >> (32 - kMaxLen)]; }

// Decode two symbols from one 32-bit window (two codes take at most 24 bits)
// and return them as bytes 0,1.
__device__ inline uint32_t chain_pair(Chain &c, const uint32_t *stage, const uint16_t *lut) {
    const uint32_t win = window(stage, c.r);
    const uint32_t e1 = lookup(lut, win);
    const uint32_t e2 = lookup(lut, win << (e1 & 31));
    c.r -= (e1 + e2) & 0xFF;
    return sym_pair(e1, e2);
}

__device__ inline uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Where a chunk's code bits lie among the stream words.
struct ChunkGeom {
    uint64_t w0;      // first staged stream word (16-byte aligned)
    uint32_t nwords;  // words to stage: through the chunk's last bit plus over-read slack
    uint32_t rel;     // the chunk's first bit, counted from word w0
};

__device__ inline ChunkGeom chunk_geom(uint64_t base, uint64_t end) {
    ChunkGeom g;
    g.w0 = (base >> 5) & ~(uint64_t)3;
    // unsigned arithmetic saturates through the min on a corrupt base pair
    const uint64_t want = ((end + 31) >> 5) + 16 - g.w0;
    g.nwords = (uint32_t)umin64(want, kStageWords);
    g.rel = (uint32_t)(base - (g.w0 << 5));  // < 128
    return g;
}

// The first 512 staged words of a chunk travel through registers so that
// their loads can be issued one chunk ahead; longer chunks (more than about
// 4 bits per element) fetch the rest when they are staged.
constexpr uint32_t kPrefetchWords = 2 * 4 * kWave;

struct StreamRegs {
    uint4 v[2];
};

// Four stream words from 4-aligned index g. Past the end of the section the
// index is clamped: such words lie beyond the last code bit (the stream ends
// with four zero words), so what they hold never reaches an output.
__device__ inline uint4 load_words4(const TensorDesc &T, uint64_t g) {
    return *reinterpret_cast<const uint4 *>(T.exp + umin64(g, T.last_word4));
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
    *reinterpret_cast<uint4 *>(stage + (kRev - 3 - i)) = make_uint4(v.w, v.z, v.y, v.x);
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
    const uint32_t ng = (uint32_t)((umin64(kChunk, T.n - lc * kChunk) + kGroup - 1) / kGroup);
    const uint16_t *gap = T.gap + lc * kGroupsPerChunk;
    // read once: not kept in the caches
    return Gaps{__builtin_nontemporal_load(gap + min((uint32_t)lane, ng - 1)),
                __builtin_nontemporal_load(gap + min((uint32_t)lane + kWave, ng - 1))};
}

// 16 output bytes; the output is written once and not read back here, so the
// stores bypass cache allocation (each store instruction covers whole lines).
__device__ inline void store_out(uint16_t *p, uint4 v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(p));
}

// Restore one chunk: decode the staged code words, merge with the
// sign/mantissa bytes, store. `stage` holds the chunk's code words on entry
// and is free (but for the exponent bytes just written) on exit.
__device__ inline void restore_chunk(const TensorDesc &T, uint64_t lc, const ChunkGeom &g, const Gaps &gaps,
                                     const uint16_t *lut, uint32_t *stage, int lane, uint64_t later_bases,
                                     ChunkGeom &later) {
    const uint64_t e0 = lc * kChunk;
    const uint32_t ne = (uint32_t)umin64(kChunk, T.n - e0);
    const uint8_t *sm = T.signmant + e0;
    // Sign/mantissa bytes are read exactly once: load them without keeping
    // them in the caches (the code words stay cached: neighbouring chunks
    // share the lines at their ends).
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    uint2 smv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t i = (uint32_t)r * (8 * kWave) + 8 * (uint32_t)lane;
        const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(sm + (i + 8 <= ne ? i : 0)));
        smv[r] = make_uint2(t.x, t.y);  // tail elements are reread below
    }

    // Decode: chain starts clamped so that 32 decodes (at most 384 bits)
    // never leave the staged words even on a corrupt gap.
    constexpr uint32_t kMaxStart = 32 * (kRev - 13);
    Chain A{32 * kRev - min(g.rel + gaps.a, kMaxStart)};
    Chain B{32 * kRev - min(g.rel + gaps.b, kMaxStart)};
    uint32_t wa[8], wb[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t a01 = chain_pair(A, stage, lut);
        const uint32_t b01 = chain_pair(B, stage, lut);
        const uint32_t a23 = chain_pair(A, stage, lut);
        const uint32_t b23 = chain_pair(B, stage, lut);
        wa[q] = join_halves(a01, a23);
        wb[q] = join_halves(b01, b23);
    }
    wave_sync();  // every lane is done reading the staged words
    uint4 *pa = reinterpret_cast<uint4 *>(stage + lane * 8);
    uint4 *pb = reinterpret_cast<uint4 *>(stage + (lane + kWave) * 8);
    pa[0] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
    pa[1] = make_uint4(wa[4], wa[5], wa[6], wa[7]);
    pb[0] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
    pb[1] = make_uint4(wb[4], wb[5], wb[6], wb[7]);
    wave_sync();
    // Read out the bases fetched for a later chunk now, while the only loads
    // issued after them are this chunk's sign/mantissa bytes (needed next
    // anyway): read after the stores below, they would make the wave wait
    // for those stores to complete.
    asm volatile("" : "+v"(later_bases));  // not before the decode above
    later = geom_from_lanes(later_bases);

    // Store order: lane handles elements [r*512 + 8*lane, +8) for r = 0..7,
    // so each store instruction writes 1 KB of output.
    uint16_t *out = T.out + e0;
    const uint8_t *exb = reinterpret_cast<const uint8_t *>(stage);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t i = (uint32_t)r * (8 * kWave) + 8 * (uint32_t)lane;
        if (i + 8 <= ne) {
            const uint2 b = smv[r];
            const uint2 e = *reinterpret_cast<const uint2 *>(exb + i);
            uint4 o;
            o.x = join_pair<false>(b.x, e.x);
            o.y = join_pair<true>(b.x, e.x);
            o.z = join_pair<false>(b.y, e.y);
            o.w = join_pair<true>(b.y, e.y);
            store_out(out + i, o);
            __builtin_amdgcn_sched_barrier(0);  // keep live ranges per step
        } else {
            for (uint32_t j = i; j < ne && j < i + 8; ++j) {
                const uint32_t b = sm[j], e = exb[j];
                out[j] = (uint16_t)(((b & 0x80u) << 8) | (e << 7) | (b & 0x7Fu));
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void afx_decode_kernel(const Batch batch) {
    __shared__ __attribute__((aligned(16))) uint16_t lut[kLutEntries];  // 8 KB
    __shared__ __attribute__((aligned(16))) uint32_t stage[kWavesPerBlock][kStageRow];  // 98 KB
    __shared__ LutScratch scratch;
    __shared__ uint32_t next_j;  // the workgroup's next unclaimed chunk of the tensor

    int lane = threadIdx.x & (kWave - 1);
    // the wave index is uniform across the wave: keep it (and everything
    // derived from it) in scalar registers
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint64_t b = blockIdx.x;
    uint32_t *my_stage = stage[wave];

    for (uint32_t t = 0; t < batch.n_tensors; ++t) {
        const TensorDesc &T = batch.t[t];
        // Workgroups [blk_lo, blk_hi) serve T (the host splits the grid among
        // the tensors in proportion to their chunk counts). Within a tensor the
        // chunks go round its workgroups, so that all of them move through each
        // array together, in one narrow band: the k-th of nb takes chunks
        // k + j nb, j = 0, 1, ... Wave w starts with j = w and j = w + 16;
        // after that each wave claims the next unclaimed j when it starts a
        // chunk, so waves that the SIMDs serve faster restore more chunks and
        // all finish together.
        if (b < T.blk_lo || b >= T.blk_hi) continue;
        const uint32_t k = (uint32_t)b - T.blk_lo, nb = T.blk_hi - T.blk_lo;
        if (k >= T.n_chunks) continue;
        const uint32_t mine = (T.n_chunks - k + nb - 1) / nb;
        uint32_t jc = wave, jn = wave + kWavesPerBlock;
        const bool has_c = jc < mine;
        bool has_n = jn < mine;
        // Fetch the code lengths, the first two chunks' bases and the first
        // one's gaps, then the first chunk's code words; building the decode
        // table hides the second round trip.
        const uint32_t len = wave < kSymbolWaves ? T.code_len[threadIdx.x] : 0;
        uint64_t bases_c = 0, bases_n = 0;
        Gaps gaps{0, 0};
        if (has_c) bases_c = load_bases(T, k + (uint64_t)jc * nb, lane);
        if (has_n) bases_n = load_bases(T, k + (uint64_t)jn * nb, lane);
        if (has_c) gaps = load_gaps(T, k + (uint64_t)jc * nb, lane);
        ChunkGeom g{};
        StreamRegs s;
        if (has_c) {
            g = geom_from_lanes(bases_c);
            load_stream(T, g, lane, s);
        }
        __syncthreads();  // every wave is done with the previous table and counter
        if (threadIdx.x == 0) next_j = 2 * kWavesPerBlock;
        build_lut(len, lut, scratch);  // ends with a barrier
        __syncthreads();
        if (!has_c) continue;
        put_stream(T, g, s, my_stage, lane);
        wave_sync();
        ChunkGeom gn = geom_from_lanes(bases_n);
        while (true) {
            // recompute per-lane offsets every chunk instead of keeping them
            // live across the loop
            asm volatile("" : "+v"(lane));
            // While chunk jc decodes, fetch the code words and gaps of jn,
            // claim the chunk after it and fetch that one's bases.
            uint32_t jnn = ~0u;
            bool has_nn = false;
            StreamRegs sn;
            Gaps gaps_n{0, 0};
            uint64_t bases_nn = 0;
            if (has_n) {
                uint32_t v = 0;
                if (lane == 0) v = atomicAdd(&next_j, 1u);
                jnn = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
                has_nn = jnn < mine;
                load_stream(T, gn, lane, sn);
                gaps_n = load_gaps(T, k + (uint64_t)jn * nb, lane);
                if (has_nn) bases_nn = load_bases(T, k + (uint64_t)jnn * nb, lane);
            }
            ChunkGeom gnn;
            restore_chunk(T, k + (uint64_t)jc * nb, g, gaps, lut, my_stage, lane, bases_nn, gnn);
            if (!has_n) break;
            wave_sync();  // the exponent bytes have been read
            put_stream(T, gn, sn, my_stage, lane);
            wave_sync();
            g = gn;
            gaps = gaps_n;
            gn = gnn;
            jc = jn;
            jn = jnn;
            has_n = has_nn;
        }
    }
}

// Largest useful grid per device: every CU filled to the kernel's occupancy.
std::atomic<int> g_max_blocks[64];

int max_blocks_for_current_device(int *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return AFX_E_HIP;
    if (dev < 0 || dev >= 64) return AFX_E_UNSUPPORTED;
    int v = g_max_blocks[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return AFX_E_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, afx_decode_kernel, kThreads, 0) != hipSuccess)
            return AFX_E_HIP;
        v = std::max(1, cus) * std::max(1, per_cu);
        g_max_blocks[dev].store(v, std::memory_order_relaxed);
    }
    *out = v;
    return AFX_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_job(const afx_job &j) {
    int rc = check_info(j.info);
    if (rc != AFX_OK) return rc;
    if (!j.blob_dev || (!j.out_dev && j.info->n_elems)) return AFX_E_INVALID_ARG;
    if (j.out_bytes < j.info->decoded_bytes) return AFX_E_BUFFER_TOO_SMALL;
    if (!aligned16(j.blob_dev) || !aligned16(j.out_dev)) return AFX_E_MISALIGNED;
    if (j.info->n_elems) {
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(j.blob_dev), b1 = b0 + j.info->blob_bytes;
        const uintptr_t o0 = reinterpret_cast<uintptr_t>(j.out_dev), o1 = o0 + j.info->decoded_bytes;
        if (o0 < b1 && b0 < o1) return AFX_E_INVALID_ARG;  // output overlaps the blob
    }
    return AFX_OK;
}

TensorDesc describe(const afx_job &j) {
    const afx_info &I = *j.info;
    const uint8_t *b = static_cast<const uint8_t *>(j.blob_dev);
    TensorDesc d;
    d.code_len = b + I.off_code_len;
    d.chunk_base = reinterpret_cast<const uint64_t *>(b + I.off_chunk_base);
    d.gap = reinterpret_cast<const uint16_t *>(b + I.off_gap);
    d.signmant = b + I.off_signmant;
    d.exp = reinterpret_cast<const uint32_t *>(b + I.off_exp);
    d.out = static_cast<uint16_t *>(j.out_dev);
    d.n = I.n_elems;
    d.exp_words = I.exp_words;
    d.last_word4 = (I.exp_words - 4) & ~(uint64_t)3;  // exp_words >= 4: the stream ends with 4 zero words
    d.n_chunks = (uint32_t)I.n_chunks;  // n <= 2^40 elements: fewer than 2^28 chunks
    d.blk_lo = d.blk_hi = 0;
    d.reserved = 0;
    return d;
}

// Enqueue one launch for up to AFX_MAX_JOBS_PER_LAUNCH already-checked jobs.
int launch(const afx_job *jobs, size_t n_jobs, hipStream_t stream) {
    Batch batch;
    batch.n_tensors = 0;
    uint64_t total = 0;
    uint64_t first[AFX_MAX_JOBS_PER_LAUNCH];
    for (size_t i = 0; i < n_jobs; ++i) {
        if (jobs[i].info->n_elems == 0) continue;
        first[batch.n_tensors] = total;
        batch.t[batch.n_tensors++] = describe(jobs[i]);
        total += jobs[i].info->n_chunks;
    }
    if (total == 0) return AFX_OK;
    int max_blocks = 0;
    int rc = max_blocks_for_current_device(&max_blocks);
    if (rc != AFX_OK) return rc;
    // Every workgroup should get the same number of chunks, or the launch
    // ends with part of the grid idle: with at most max_blocks workgroups each
    // takes ceil(total / max_blocks) chunks; use just enough workgroups.
    const uint64_t per_block = (total + max_blocks - 1) / max_blocks;
    const uint64_t want = (total + per_block - 1) / per_block;
    const uint64_t grid = std::max<uint64_t>(1, std::min<uint64_t>(want, (uint64_t)max_blocks));
    // Split the grid among the tensors in proportion to their chunk counts;
    // a tensor too small for a workgroup of its own is served by the
    // workgroup at its position (which may serve a neighbour too).
    for (uint32_t t = 0; t < batch.n_tensors; ++t) {
        const uint64_t lo = grid * first[t] / total;
        uint64_t hi = grid * (first[t] + batch.t[t].n_chunks) / total;
        if (hi <= lo) hi = lo + 1;
        batch.t[t].blk_lo = (uint32_t)lo;
        batch.t[t].blk_hi = (uint32_t)hi;
    }
    hipLaunchKernelGGL(afx_decode_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, batch);
    return hipGetLastError() == hipSuccess ? AFX_OK : AFX_E_HIP;
}

}  // namespace
}  // namespace afx

using namespace afx;

extern "C" {

int afx_decode_tensor(const afx_info *info, const void *blob_dev, void *out_dev, size_t out_bytes, void *stream) {
    const afx_job job{info, blob_dev, out_dev, out_bytes};
    int rc = check_job(job);
    if (rc != AFX_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = launch(&job, 1, s);
    if (rc != AFX_OK) return rc;
    return hipStreamSynchronize(s) == hipSuccess ? AFX_OK : AFX_E_HIP;
}

int afx_decode_layer_async(const afx_job *jobs, size_t n_jobs, void *stream) {
    if (!jobs && n_jobs) return AFX_E_INVALID_ARG;
    for (size_t i = 0; i < n_jobs; ++i) {
        const int rc = check_job(jobs[i]);
        if (rc != AFX_OK) return rc;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (size_t i = 0; i < n_jobs; i += AFX_MAX_JOBS_PER_LAUNCH) {
        const size_t k = std::min<size_t>(AFX_MAX_JOBS_PER_LAUNCH, n_jobs - i);
        const int rc = launch(jobs + i, k, s);
        if (rc != AFX_OK) return rc;
    }
    return AFX_OK;
}

}  // extern "C"
