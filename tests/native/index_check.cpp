// index_check.cpp -- on the CPU, every index the restore kernels form from
// blob contents stays inside its buffer, whatever a corrupt device blob holds.
//
// The kernels take each such index from the constexpr functions of
// afx_index.h (chunk geometry, stream-word clamps, gap slots, chain starts
// and steps, table offsets, the MFMA product's row segments). This program
// includes the same header and drives those functions the way the kernels
// compose them, with random bit positions, gaps, code lengths, step sizes
// and section sizes, many of them wild (end before start, values near
// 2^64), and checks every LDS slot and global word index against the buffer
// it addresses; and that the MFMA product's launch order gives every tile
// and token block to exactly one workgroup. Built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_index_bounds.py; exits 1 on the first few violations it prints.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "afx_index.h"

using namespace afx;

namespace {

uint64_t g_fail = 0, g_checks = 0;

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        ++g_checks;                                                       \
        if (!(cond)) {                                                    \
            if (g_fail++ < 20) {                                          \
                std::fprintf(stderr, "index out of range: " __VA_ARGS__); \
                std::fputc('\n', stderr);                                 \
            }                                                             \
        }                                                                 \
    } while (0)

struct Rng {
    std::mt19937_64 g;
    explicit Rng(uint64_t seed) : g(seed) {}
    uint64_t u64() { return g(); }
    uint32_t below(uint32_t m) { return (uint32_t)(g() % m); }
    // A bit position or count as a corrupt blob might hold it: arbitrary
    // bits, small values, values near 2^64, or plausible ones.
    uint64_t wild(uint64_t plausible) {
        switch (below(6)) {
            case 0: return u64();
            case 1: return u64() >> below(64);
            case 2: return ~(uint64_t)0 - below(1 << 16);
            case 3: return below(1 << 16);
            case 4: return plausible ^ ((uint64_t)1 << below(64));  // one flipped bit
            default: return plausible;
        }
    }
};

// One chunk of the restore (and of the fused matrix-vector product, which
// stages and decodes chunks with the same functions).
void restore_chunk(Rng &R, uint64_t n, uint64_t exp_words) {
    const uint64_t n_chunks = (n + kChunk - 1) / kChunk, n_groups = (n + kGroup - 1) / kGroup;
    const uint64_t lc = R.u64() % n_chunks;  // the chunk walk is structural, from n alone
    const uint64_t plausible = lc * kChunk * 3;
    const uint64_t base = R.wild(plausible);
    const uint64_t end = R.below(2) ? R.wild(plausible + kChunk * 3) : base + R.below(kChunk * kMaxLen + 1);
    const ChunkGeom g = chunk_geom(base, end);
    CHECK(g.nwords <= kStageWords, "nwords %u", g.nwords);
    CHECK(g.rel < 128, "rel %u", g.rel);

    // staging: each lane stages the four words at 4-aligned offsets i below
    // nwords (i = 4 lane + 256 k), reversed into the wave's slice
    const uint64_t last4 = last_word4(exp_words);
    // (the loop stops a few words past the slice: beyond, a wild count only
    // repeats the same failure)
    for (uint32_t i = 0; i < g.nwords && i <= kStageWords + 4; i += 4) {
        const uint32_t s = stage_put_index(i);
        CHECK(s <= kRev - 3, "stage slot %u for word %u of %u", s, i, g.nwords);
        const uint64_t w = word4_index(g.w0 + i, last4);
        CHECK(w + 4 <= exp_words, "stream word %llu of %llu", (unsigned long long)w, (unsigned long long)exp_words);
    }

    // gaps: lane l reads groups l and l + 64 of the chunk
    const uint32_t ng = chunk_groups(n, lc);
    CHECK(ng >= 1 && ng <= kGroupsPerChunk, "groups %u", ng);
    for (uint32_t l = 0; l < 2 * 64; ++l) {
        const uint32_t slot = gap_slot(l, ng);
        CHECK(slot < ng, "gap slot %u of %u", slot, ng);
        CHECK(lc * kGroupsPerChunk + slot < n_groups, "gap %llu", (unsigned long long)(lc * kGroupsPerChunk + slot));
    }

    // two chains per lane from corrupt gaps, 16 two-symbol steps each, each
    // step consuming 1..kMaxStep bits (kMaxStep on some lanes throughout)
    for (uint32_t l = 0; l < 2 * 64; ++l) {
        const uint32_t gap = (uint32_t)R.below(1 << 16);
        uint32_t r = chain_r0(g.rel, gap);
        uint32_t q = chain_word(r);
        CHECK(q >= 1 && q + 1 <= kStageWords && q + 1 < kStageRow, "chain start word %u (gap %u)", q, gap);
        const bool worst = R.below(4) == 0;
        for (int step = 0; step < 16; ++step) {
            const uint32_t d = worst ? kMaxStep : 1 + R.below(kMaxStep);
            CHECK(r >= d, "chain counter %u below step %u", r, d);
            r -= d;
            const uint32_t qn = chain_word(r);
            CHECK(qn + 1 >= q, "chain skipped a word");
            q = qn;
            CHECK(q >= 1, "read-ahead below the slice (word %u)", q);  // reads q - 1
            CHECK(q + 1 < kStageRow, "window above the slice (word %u)", q);
        }
    }
    // decoded exponent bytes: lane l writes words [8 l, 8 l + 8) and
    // [8 (l + 64), +8) of its slice
    CHECK(8 * 128 <= kStageRow, "exponent bytes exceed the slice");
}

// A table read: any 32-bit window addresses one of 4096 entries.
void table_reads(Rng &R) {
    const uint32_t w = (uint32_t)R.u64();
    CHECK(pair_offset(w) / 4 < (1u << kMaxLen) && pair_offset(w) % 4 == 0, "pair offset %u", pair_offset(w));
    CHECK(one_code_index(w) < (1u << kMaxLen), "one-code index %u", one_code_index(w));
    const uint32_t s = R.below(32);
    CHECK(pair_offset(w << s) / 4 < (1u << kMaxLen), "shifted pair offset");
    // the table build: code lengths as read, slice ends as computed from them
    const uint32_t len = used_length(R.below(256));
    CHECK(len <= kMaxLen, "length %u", len);
    uint32_t lim[kMaxLen] = {};
    for (uint32_t q = 1; q < kMaxLen; ++q) lim[q] = (uint32_t)R.u64() >> R.below(32);
    const uint32_t l = entry_length(R.below(1 << kMaxLen), lim);
    CHECK(l >= 1 && l <= kMaxLen, "entry length %u", l);
}

// One row segment of the MFMA product: the quad's first group starts at
// p_lo, the segment ends at p_hi, the lane's groups at p1, p2 (all as a
// corrupt blob may hold them).
void gemm_segment(Rng &R, uint64_t exp_words) {
    const uint64_t plausible = R.u64() % (exp_words * 32);
    const uint64_t p_lo = R.wild(plausible);
    const uint64_t p_hi = R.below(2) ? R.wild(plausible + 256 * 3) : p_lo + R.below(256 * kMaxLen + 1);
    const uint64_t wa = seg_first_word(p_lo);
    const uint32_t nw = seg_words(p_lo, p_hi);
    CHECK(nw <= kSegWords, "segment words %u", nw);
    const uint64_t last4 = last_word4(exp_words);
    // words 0..31 are always staged (each lane of the quad 8 of them), the
    // rest by the loop i = 32 + 4 q4 (step 16) below nw
    for (uint32_t i = 0; i < (nw > 32 ? nw : 32) && i <= kSegWords + 4; i += 4) {
        const uint32_t s = seg_put_index(i);
        CHECK(s <= kSegRev - 3, "segment slot %u for word %u", s, i);
        const uint64_t w = word4_index(wa + i, last4);
        CHECK(w + 4 <= exp_words, "segment stream word %llu", (unsigned long long)w);
    }
    for (int c = 0; c < 2; ++c) {
        const uint64_t p = R.below(2) ? R.wild(p_lo + R.below(256 * 3)) : p_lo + R.below(256 * kMaxLen);
        uint32_t r = seg_chain_r0(p, wa);
        uint32_t q = chain_word(r);
        CHECK(q >= 1 && q + 1 < kSegRow, "segment chain start word %u", q);
        const bool worst = R.below(4) == 0;
        for (int step = 0; step < 16; ++step) {  // two one-code reads per step: <= kMaxStep bits
            const uint32_t d = worst ? kMaxStep : 1 + R.below(kMaxStep);
            CHECK(r >= d, "segment chain counter %u below step %u", r, d);
            r -= d;
            q = chain_word(r);
            CHECK(q >= 1 && q + 1 < kSegRow, "segment chain word %u", q);
        }
    }
}

// The MFMA product's launch order: every (tile, token block) pair taken by
// exactly one block, padding blocks only past the last tile.
void gemm_order(Rng &R) {
    const uint64_t tiles = 1 + R.below(R.below(2) ? 40 : 3000);
    const uint32_t nt = 1 + R.below(R.below(2) ? 3 : 9);
    const uint64_t blocks = gemm_blocks(tiles, nt);
    CHECK(blocks >= tiles * nt && blocks < tiles * nt + 8 * nt, "launch of %llu blocks", (unsigned long long)blocks);
    std::vector<uint8_t> seen(tiles * nt, 0);
    for (uint64_t b = 0; b < blocks; ++b) {
        const uint32_t t = gemm_block_tile((uint32_t)b, nt), k = gemm_block_token((uint32_t)b, nt);
        CHECK(k < nt, "token block %u of %u", k, nt);
        if (t >= tiles || k >= nt) continue;
        CHECK(t % 8 == b % 8 || nt == 1, "tile %u off its block's XCD", t);
        CHECK(!seen[t * nt + k], "tile %u token block %u taken twice", t, k);
        seen[t * nt + k] = 1;
    }
    for (uint64_t i = 0; i < tiles * nt; ++i) CHECK(seen[i], "tile %llu token block %llu not taken",
                                                    (unsigned long long)(i / nt), (unsigned long long)(i % nt));
}

}  // namespace

int main(int argc, char **argv) {
    const uint64_t trials = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 200000;
    Rng R(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 12345);
    for (uint64_t t = 0; t < trials; ++t) {
        // tensor sizes from one element to 2^40 (the largest accepted)
        uint64_t n = 1 + (R.u64() >> R.below(64)) % ((uint64_t)1 << 40);
        if (R.below(4) == 0) n = 1 + R.below(3 * kChunk);
        // the stream section's true size, or anything at least 4 words
        const uint64_t true_words = (n * R.below(kMaxLen + 1) + 31) / 32 + kPadWords;
        const uint64_t exp_words = R.below(2) ? true_words : 4 + (R.u64() >> R.below(64)) % ((uint64_t)1 << 44);
        restore_chunk(R, n, exp_words);
        table_reads(R);
        gemm_segment(R, exp_words);
        if (t % 64 == 0) gemm_order(R);
    }
    std::printf("%llu index checks, %llu out of range\n", (unsigned long long)g_checks, (unsigned long long)g_fail);
    return g_fail ? 1 : 0;
}
