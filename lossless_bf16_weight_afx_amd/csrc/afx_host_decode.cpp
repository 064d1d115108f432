// afx_host_decode.cpp -- the unpack on the host, where the pages place it.
//
// "Why Weight Offloading Slows Inference" (section "The path from storage to
// the GPU", Figure 1) unpacks a compressed weight in RAM, between the read
// and the copy over PCIe, and section "Lossless compression" finds that this
// host-side unpack cost more than the read time compression saved (Eq. (2)).
// The GPU entry points never call this file: it exists to measure that
// placement against unpacking on the GPU, on the same store and host.
//
// Per tensor, a 4096-entry table maps the next 12 stream bits to
// (symbol << 8) | length of the canonical code word they start with. Every
// chunk decodes on its own from its bit base; inside a chunk, eight groups
// (from their gap offsets) decode interleaved so that their table lookups
// overlap, two codes per 64-bit window. No HIP calls here.
#include "afx_internal.h"

#include <algorithm>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

namespace {

using afx::kChunk;
using afx::kGroup;
using afx::kGroupsPerChunk;
using afx::kMaxLen;

struct Tensor {
    const uint8_t *signmant;
    const uint64_t *base;
    const uint16_t *gap;
    const uint32_t *exp;
    uint64_t n, exp_words;
    uint16_t table[1 << kMaxLen];
};

void build_table(const uint8_t len[256], uint16_t *table) {
    uint32_t code[256];
    afx::canonical(len, code);
    int only = -1, used = 0;
    for (int s = 0; s < 256; ++s) {
        if (!len[s]) continue;
        ++used;
        only = s;
        const uint32_t lo = code[s] << (kMaxLen - len[s]), hi = (code[s] + 1) << (kMaxLen - len[s]);
        for (uint32_t i = lo; i < hi; ++i) table[i] = (uint16_t)((s << 8) | len[s]);
    }
    // a one-value code fills half the windows; the other half is never reached
    if (used == 1)
        for (uint32_t i = 1u << (kMaxLen - 1); i < (1u << kMaxLen); ++i) table[i] = (uint16_t)((only << 8) | 1);
}

// The 12 stream bits at bit position p (MSB first in each u32 word).
inline uint32_t peek12(const Tensor &T, uint64_t p) {
    const uint64_t w = std::min<uint64_t>(p >> 5, T.exp_words - 2);  // a corrupt stream stays inside
    const uint64_t v = ((uint64_t)T.exp[w] << 32) | T.exp[w + 1];
    return (uint32_t)((v << (p & 31)) >> (64 - kMaxLen));
}

inline uint16_t join(uint8_t b, uint32_t e) { return (uint16_t)(((b & 0x80u) << 8) | (e << 7) | (b & 0x7Fu)); }

void decode_chunk(const Tensor &T, uint64_t c, uint16_t *out) {
    const uint64_t e0 = c * kChunk;
    const uint32_t ne = (uint32_t)std::min<uint64_t>(kChunk, T.n - e0);
    const uint32_t ng = (ne + kGroup - 1) / kGroup;
    const uint64_t base = T.base[c];
    const uint16_t *gap = T.gap + c * kGroupsPerChunk;
    const uint8_t *sm = T.signmant + e0;
    uint32_t g = 0;
    constexpr int kWays = 8;
    for (; g + kWays <= ng && (g + kWays) * kGroup <= ne; g += kWays) {
        uint64_t p[kWays];
        for (int k = 0; k < kWays; ++k) p[k] = base + gap[g + k];
        // two codes (at most 24 bits) per 64-bit window of the stream
        for (uint32_t i = 0; i < kGroup; i += 2) {
            for (int k = 0; k < kWays; ++k) {
                const uint64_t w = std::min<uint64_t>(p[k] >> 5, T.exp_words - 2);
                const uint64_t v = (((uint64_t)T.exp[w] << 32) | T.exp[w + 1]) << (p[k] & 31);
                const uint16_t e1 = T.table[v >> (64 - kMaxLen)];
                const uint16_t e2 = T.table[(v << (e1 & 0xFF)) >> (64 - kMaxLen)];
                p[k] += (e1 & 0xFF) + (e2 & 0xFF);
                const uint32_t j = (g + k) * kGroup + i;
                out[e0 + j] = join(sm[j], e1 >> 8);
                out[e0 + j + 1] = join(sm[j + 1], e2 >> 8);
            }
        }
    }
    for (; g < ng; ++g) {  // the groups left over, the last one possibly short
        uint64_t p = base + gap[g];
        const uint32_t j1 = std::min(ne, (g + 1) * kGroup);
        for (uint32_t j = g * kGroup; j < j1; ++j) {
            const uint16_t e = T.table[peek12(T, p)];
            p += e & 0xFF;
            out[e0 + j] = join(sm[j], e >> 8);
        }
    }
}

}  // namespace

static int decode_host(const void *blob, size_t blob_bytes, uint16_t *out, size_t out_bytes, int threads) {
    if (!blob) return AFX_E_INVALID_ARG;
    afx_info info;
    int rc = afx_query(blob, blob_bytes, &info);
    if (rc != AFX_OK) return rc;
    if (info.n_elems && !out) return AFX_E_INVALID_ARG;
    if (out_bytes < info.decoded_bytes) return AFX_E_BUFFER_TOO_SMALL;
    if (info.n_elems == 0) return AFX_OK;
    const uint8_t *b = static_cast<const uint8_t *>(blob);
    std::vector<Tensor> holder(1);  // the table is 8 KB: keep it off the stack
    Tensor &T = holder[0];
    T.signmant = b + info.off_signmant;
    T.base = reinterpret_cast<const uint64_t *>(b + info.off_chunk_base);
    T.gap = reinterpret_cast<const uint16_t *>(b + info.off_gap);
    T.exp = reinterpret_cast<const uint32_t *>(b + info.off_exp);
    T.n = info.n_elems;
    T.exp_words = info.exp_words;
    build_table(b + info.off_code_len, T.table);
    const uint64_t chunks = info.n_chunks;
    int t = threads > 0 ? threads : (int)std::thread::hardware_concurrency();
    t = std::max(1, std::min<int>(t, 64));
    if ((uint64_t)t > chunks) t = (int)chunks;
    auto work = [&](uint64_t c0, uint64_t c1) {
        for (uint64_t c = c0; c < c1; ++c) decode_chunk(T, c, out);
    };
    afx::run_parts(t, [&](int i) { work(chunks * i / t, chunks * (i + 1) / t); });
    return AFX_OK;
}

extern "C" int afx_decode_host(const void *blob, size_t blob_bytes, uint16_t *out, size_t out_bytes, int threads) {
    try {
        return decode_host(blob, blob_bytes, out, out_bytes, threads);
    } catch (const std::bad_alloc &) {
        return AFX_E_HOST_MEMORY;
    }
}
