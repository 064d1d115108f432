// afx_index.h -- where the restore kernels read and write: the integer index
// arithmetic of chunk staging, the decoding chains, gaps and stream words.
//
// A device blob is trusted only as far as afx_query validated its host copy;
// a device copy that differs (bit flips, a stale or foreign buffer) must
// decode to wrong bits, never to an access outside its buffers. Every index
// that depends on blob contents (chunk bases, gaps, code lengths, code
// words) is formed by one of the functions below and clamped here. They are
// constexpr, so the same code runs in the kernels (clang compiles constexpr
// functions for host and device alike) and in a plain host build that checks
// them against random corrupt inputs on the CPU. No HIP header is needed.
//
// The format: a tensor's exponent codes form one MSB-first bit stream of u32
// words; each 4096-element chunk starts at a recorded u64 bit base, and each
// 32-element group at a u16 gap after its chunk's base (the exponent field is
// the coded part: "Why Weight Offloading Slows Inference", section "Lossless
// compression").
#pragma once

#include <cstdint>

#include "afx_internal.h"

namespace afx {

constexpr uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }
constexpr uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }

// ---- the restore's per-wave stage (LDS) ----------------------------------
// While a chunk decodes, its code words sit in the wave's stage slice in
// reverse order (stream word j at index kRev - j), with one pad word above
// (index kRev + 1), so that one counter r = 32 kRev - P gives both the word
// index of bit P and the funnel-shift amount of the 32-bit window there.
// A chunk spans at most 4096 * 12 bits; add the alignment slack of its start
// and the over-read of its last group.
constexpr uint32_t kStageWords = 1568;
constexpr uint32_t kRev = kStageWords - 1;  // == 3 (mod 4): 16-byte aligned reversed stores
static_assert(kRev % 4 == 3, "reversed staging needs kRev = 3 mod 4");
// A wave's slice with the pad word, rounded up to 16 bytes.
constexpr uint32_t kStageRow = (kStageWords + 1 + 3) & ~3u;

// The paired chains run kLead bits behind the code they decode (the pair
// table's byte address is then a masked high half-word of the window).
constexpr uint32_t kLead = 2;
// One two-symbol step consumes at most two codes of at most kMaxLen bits.
constexpr uint32_t kMaxStep = 2 * kMaxLen;

// Where a chunk's code bits lie among the stream words.
struct ChunkGeom {
    uint64_t w0;      // first staged stream word (16-byte aligned)
    uint32_t nwords;  // words to stage: through the chunk's last bit plus over-read slack
    uint32_t rel;     // the chunk's first bit, counted from word w0
};

// From the chunk's first bit and the next chunk's first bit. A corrupt pair
// (end below base, or huge values) still gives nwords <= kStageWords: the
// unsigned arithmetic saturates through the min.
constexpr ChunkGeom chunk_geom(uint64_t base, uint64_t end) {
    ChunkGeom g{};
    g.w0 = (base >> 5) & ~(uint64_t)3;
    const uint64_t want = ((end + 31) >> 5) + 16 - g.w0;
    g.nwords = (uint32_t)umin64(want, kStageWords);
    g.rel = (uint32_t)(base - (g.w0 << 5));  // < 128
    return g;
}

// Highest 4-aligned word index w with w + 4 <= exp_words (exp_words >= 4:
// the stream ends with four zero words).
constexpr uint64_t last_word4(uint64_t exp_words) { return (exp_words - 4) & ~(uint64_t)3; }

// The stream word index of a 16-byte load from 4-aligned index g. Past the
// end of the section the index is clamped: such words lie beyond the last
// code bit, so what they hold never reaches an output.
constexpr uint64_t word4_index(uint64_t g, uint64_t last4) { return umin64(g, last4); }

// Stage index of the four words loaded from stream word w0 + i (i a multiple
// of 4 below nwords), reversed: they go to [kRev - 3 - i, kRev - i].
constexpr uint32_t stage_put_index(uint32_t i) { return kRev - 3 - i; }

// Groups in chunk lc of an n-element tensor (1..128).
constexpr uint32_t chunk_groups(uint64_t n, uint64_t lc) {
    return (uint32_t)((umin64(kChunk, n - lc * kChunk) + kGroup - 1) / kGroup);
}

// Gap slot read for group g of a chunk with ng groups: groups past the end
// of a short last chunk take the last group's gap (they decode something,
// but nothing they decode is stored).
constexpr uint32_t gap_slot(uint32_t g, uint32_t ng) { return umin32(g, ng - 1); }

// The chain counter of a group that starts `rel + gap` bits after the
// chunk's first staged word. The start is clamped so that 32 codes (at most
// 384 bits) never leave the staged words on a corrupt gap; the chain's read
// ahead (one word below its window) then stays at index >= 0, and its window
// (kLead bits behind) at most reaches the pad word above.
constexpr uint32_t kMaxStart = 32 * (kRev - 13);
constexpr uint32_t chain_r0(uint32_t rel, uint32_t gap) { return 32 * kRev - umin32(rel + gap, kMaxStart) + kLead; }

// A chain with counter r reads staged words chain_word(r) + 1 and
// chain_word(r) (its window) and chain_word(r) - 1 (read ahead); a step
// consumes d <= kMaxStep < 32 bits: r -= d, so the word index falls by at
// most one per step.
constexpr uint32_t chain_word(uint32_t r) { return r >> 5; }

// Byte offset of the pair-table entry of a window (kLead bits behind): the
// 12 code bits at window bits 29..18, times 4.
constexpr uint32_t pair_offset(uint32_t win) { return (win >> 16) & 0x3FFCu; }
// Index of the one-code table entry of a window whose code starts at bit 31.
constexpr uint32_t one_code_index(uint32_t win) { return win >> (32 - kMaxLen); }

// A code length read from the blob: lengths above kMaxLen only come from a
// corrupt blob, and are treated as unused.
constexpr uint32_t used_length(uint32_t len) { return len > kMaxLen ? 0u : len; }

// Length of the code that starts 12-bit window idx, given the end lim[q] of
// each length q's slice of the index space (q = 1..11): one more than the
// number of slices ending at or before idx. 1..12 whatever lim holds, so a
// two-symbol step consumes at most kMaxStep bits even on corrupt lengths.
constexpr uint32_t entry_length(uint32_t idx, const uint32_t (&lim)[kMaxLen]) {
    uint32_t l = 1;
    for (uint32_t q = 1; q < kMaxLen; ++q) l += idx >= lim[q] ? 1u : 0u;
    return l;
}

// ---- the MFMA product's row segments --------------------------------------
// Code words staged per row segment of 256 elements: 256 codes of <= 12 bits
// (96 words), the 16-byte alignment of the first word (3), the bit offset
// inside it and one word of look-ahead for the last two-code window (2),
// rounded to 16 bytes. Staged in reverse order (stream word wa + i at index
// kSegRev - i); a row's slice has one more word above kSegRev for the
// chains' reads.
constexpr uint32_t kSegWords = 104;
constexpr uint32_t kSegRev = kSegWords - 1;  // == 3 (mod 4): aligned reversed stores
constexpr uint32_t kSegRow = kSegWords + 4;  // words per row slice
static_assert(kSegRev % 4 == 3, "reversed staging needs kSegRev = 3 mod 4");

// First staged stream word of a segment whose first group starts at bit
// p_lo, and the words to stage through bit p_hi plus one word of look-ahead
// (none when a corrupt p_hi lies below p_lo; at most kSegWords).
constexpr uint64_t seg_first_word(uint64_t p_lo) { return (p_lo >> 5) & ~(uint64_t)3; }
constexpr uint32_t seg_words(uint64_t p_lo, uint64_t p_hi) {
    const uint64_t wa = seg_first_word(p_lo);
    const uint64_t need = p_hi >= p_lo ? ((p_hi + 31) >> 5) + 1 - wa : 0;
    return (uint32_t)umin64(need, kSegWords);
}
constexpr uint32_t seg_put_index(uint32_t i) { return kSegRev - 3 - i; }

// The chain counter of a group starting at bit p of the stream, in a segment
// staged from word wa: clamped as chain_r0 (a p below 32 wa wraps to a huge
// offset and is clamped too). These chains start on their code (no lead).
constexpr uint32_t kSegMaxStart = 32 * (kSegRev - 13);
constexpr uint32_t seg_chain_r0(uint64_t p, uint64_t wa) {
    return 32 * kSegRev - (uint32_t)umin64(p - 32 * wa, kSegMaxStart);
}

// ---- the MFMA product's launch order ----------------------------------------
// Not derived from blob contents, but checked with the rest: block b of a
// launch with nt token blocks per tile takes tile gemm_block_tile(b, nt) (at
// least the tile count for the padding of the last run) and token block
// gemm_block_token(b, nt). Block b runs on XCD b mod 8, and each run of 8 nt
// blocks covers 8 tiles (one per XCD) times the nt token blocks, so the
// workgroups that restore one tile for different tokens run on one XCD close
// together. With nt = 1 block b takes tile b.
constexpr uint32_t gemm_block_tile(uint32_t b, uint32_t nt) { return (b / (8 * nt)) * 8 + b % 8; }
constexpr uint32_t gemm_block_token(uint32_t b, uint32_t nt) { return (b / 8) % nt; }
constexpr uint64_t gemm_blocks(uint64_t tiles, uint32_t nt) { return nt == 1 ? tiles : (tiles + 7) / 8 * 8 * nt; }

}  // namespace afx
