// afx_host.cpp -- host half of libafx: blob validation (afx_query), the
// encoder, and status strings. No HIP calls here.
//
// The coding follows "Why Weight Offloading Slows Inference", section
// "Lossless compression": the BF16 exponent field gets a per-tensor
// minimum-redundancy code (Huffman, that page's reference [2]), the other
// eight bits stay raw, and decoding gives back every value's exact bits. The
// code lengths are limited to 12 bits so that one 4096-entry table decodes
// any code word.
#include "afx_internal.h"

#include <algorithm>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

namespace afx {

namespace {

inline uint32_t load_u32(const uint8_t *p) {
    uint32_t v;
    std::memcpy(&v, p, 4);
    return v;
}
inline uint64_t load_u64(const uint8_t *p) {
    uint64_t v;
    std::memcpy(&v, p, 8);
    return v;
}
inline uint16_t load_u16(const uint8_t *p) {
    uint16_t v;
    std::memcpy(&v, p, 2);
    return v;
}

int thread_count(int requested, uint64_t work_items) {
    int t = requested > 0 ? requested : (int)std::thread::hardware_concurrency();
    if (t < 1) t = 1;
    if (t > 64) t = 64;
    if ((uint64_t)t > work_items) t = (int)std::max<uint64_t>(work_items, 1);
    return t;
}

template <class F>
void parallel_ranges(int threads, uint64_t items, F &&fn) {
    if (threads <= 1) {
        fn(0, (uint64_t)0, items);
        return;
    }
    run_parts(threads, [&](int t) {
        fn(t, items * (uint64_t)t / (uint64_t)threads, items * (uint64_t)(t + 1) / (uint64_t)threads);
    });
}

}  // namespace

Layout layout_for(uint64_t n, uint64_t total_bits) {
    auto up = [](uint64_t v) { return (v + kAlign - 1) & ~(uint64_t)(kAlign - 1); };
    Layout L;
    L.n_chunks = (n + kChunk - 1) / kChunk;
    L.n_groups = (n + kGroup - 1) / kGroup;
    L.exp_words = (total_bits + 31) / 32 + kPadWords;
    L.off_code_len = kHeaderBytes;
    L.off_chunk_base = kHeaderBytes + 256;
    L.off_gap = up(L.off_chunk_base + 8 * (L.n_chunks + 1));
    L.off_signmant = up(L.off_gap + 2 * L.n_groups);
    L.off_exp = up(L.off_signmant + n);
    L.blob_bytes = up(L.off_exp + 4 * L.exp_words);
    return L;
}

// Optimal code lengths limited to `limit` bits, by dynamic programming over
// the levels of the code tree. Symbols sorted by decreasing frequency take
// non-decreasing lengths in some optimal code. Walking down the tree, at
// depth d there are `open` free nodes; the next t symbols become leaves and
// the other open - t nodes split into 2 (open - t) nodes at depth d + 1.
// cost(d, i, open) is the least sum of freq * depth for symbols i..m-1.
int limited_lengths(const uint64_t freq[256], int limit, uint8_t len[256]) {
    std::memset(len, 0, 256);
    std::vector<int> sym;
    for (int s = 0; s < 256; ++s)
        if (freq[s]) sym.push_back(s);
    const int m = (int)sym.size();
    if (m == 0) return AFX_OK;
    if (m == 1) {
        len[sym[0]] = 1;
        return AFX_OK;
    }
    if ((1 << limit) < m) return AFX_E_UNSUPPORTED;
    std::stable_sort(sym.begin(), sym.end(), [&](int a, int b) { return freq[a] > freq[b]; });
    std::vector<uint64_t> pre(m + 1, 0);
    for (int i = 0; i < m; ++i) pre[i + 1] = pre[i] + freq[sym[i]];

    const uint64_t INF = ~(uint64_t)0 >> 2;
    const int W = m + 1;
    auto at = [W](int i, int open) { return (size_t)i * W + (size_t)open; };
    std::vector<uint64_t> next((size_t)W * W, INF), cur((size_t)W * W, INF);
    std::vector<uint16_t> pick((size_t)(limit + 1) * W * W, 0);
    // depth limit + 1: nothing may remain
    for (int open = 0; open <= m; ++open) next[at(m, open)] = 0;
    for (int d = limit; d >= 1; --d) {
        for (int i = 0; i <= m; ++i) {
            for (int open = 0; open <= m - i || (i == m && open == 0); ++open) {
                if (i == m) {
                    cur[at(i, open)] = 0;
                    continue;
                }
                uint64_t best = INF;
                int bt = 0;
                const int tmax = std::min(open, m - i);
                for (int t = 0; t <= tmax; ++t) {
                    const int rest = m - i - t;
                    const int nopen = std::min(2 * (open - t), rest);
                    const uint64_t tail = next[at(i + t, nopen)];
                    if (tail >= INF) continue;
                    const uint64_t c = (pre[i + t] - pre[i]) * (uint64_t)d + tail;
                    if (c < best) {
                        best = c;
                        bt = t;
                    }
                }
                cur[at(i, open)] = best;
                pick[(size_t)d * W * W + at(i, open)] = (uint16_t)bt;
            }
        }
        std::swap(cur, next);
        std::fill(cur.begin(), cur.end(), INF);
    }
    // next now holds depth 1
    int i = 0, open = std::min(2, m);
    if (next[at(0, open)] >= INF) return AFX_E_UNSUPPORTED;
    for (int d = 1; d <= limit && i < m; ++d) {
        const int t = pick[(size_t)d * W * W + at(i, open)];
        for (int k = 0; k < t; ++k) len[sym[i + k]] = (uint8_t)d;
        open = std::min(2 * (open - t), m - i - t);
        i += t;
    }
    return i == m ? AFX_OK : AFX_E_UNSUPPORTED;
}

// Canonical code words: ordered by (length, symbol), consecutive values,
// shifted left whenever the length grows.
void canonical(const uint8_t len[256], uint32_t code[256]) {
    uint32_t per_len[kMaxLen + 1] = {0};
    for (int s = 0; s < 256; ++s)
        if (len[s]) per_len[len[s]]++;
    uint32_t start[kMaxLen + 2] = {0};
    uint32_t c = 0;
    for (int l = 1; l <= (int)kMaxLen; ++l) {
        start[l] = c;
        c = (c + per_len[l]) << 1;
    }
    for (int s = 0; s < 256; ++s) code[s] = len[s] ? start[len[s]]++ : 0;
}

int validate(const uint8_t *b, size_t nbytes, afx_info *out) {
    if (nbytes < kHeaderBytes + 256) return AFX_E_BUFFER_TOO_SMALL;
    if (std::memcmp(b, "AFX1", 4) != 0) return AFX_E_BAD_MAGIC;
    if (load_u32(b + 4) != AFX_FORMAT_VERSION) return AFX_E_BAD_VERSION;
    if (load_u32(b + 36) != kChunk || load_u32(b + 40) != kGroup || load_u32(b + 44) != kMaxLen)
        return AFX_E_BAD_VERSION;
    const uint64_t n = load_u64(b + 8);
    const uint64_t total_bits = load_u64(b + 16);
    const uint64_t exp_words = load_u64(b + 24);
    const uint32_t ndim = load_u32(b + 32);
    const uint32_t n_symbols = load_u32(b + 48);
    if (n > kMaxElems) return AFX_E_UNSUPPORTED;
    if (ndim > 4 || total_bits > n * kMaxLen) return AFX_E_CORRUPT;
    uint64_t shape[4] = {0, 0, 0, 0}, prod = 1;
    for (uint32_t d = 0; d < 4; ++d) {
        shape[d] = load_u64(b + 64 + 8 * d);
        if (d < ndim) {
            if (shape[d] && prod > kMaxElems / shape[d]) return AFX_E_CORRUPT;
            prod *= shape[d];
        } else if (shape[d] != 0) {
            return AFX_E_CORRUPT;
        }
    }
    if (ndim ? prod != n : n != 1) return AFX_E_CORRUPT;
    const Layout L = layout_for(n, total_bits);
    if (exp_words != L.exp_words) return AFX_E_CORRUPT;
    if (nbytes < L.blob_bytes) return AFX_E_BUFFER_TOO_SMALL;

    // code lengths
    const uint8_t *len = b + L.off_code_len;
    uint32_t used = 0, longest = 0;
    uint64_t kraft = 0;  // in units of 2^-12
    for (int s = 0; s < 256; ++s) {
        if (len[s] > kMaxLen) return AFX_E_CORRUPT;
        if (len[s]) {
            ++used;
            longest = std::max<uint32_t>(longest, len[s]);
            kraft += (uint64_t)1 << (kMaxLen - len[s]);
        }
    }
    if (used != n_symbols) return AFX_E_CORRUPT;
    if ((n == 0) != (used == 0)) return AFX_E_CORRUPT;
    if (used == 1 && longest != 1) return AFX_E_CORRUPT;
    if (used >= 2 && kraft != ((uint64_t)1 << kMaxLen)) return AFX_E_CORRUPT;

    // chunk bases and group gaps
    const uint8_t *base = b + L.off_chunk_base;
    const uint8_t *gap = b + L.off_gap;
    if (load_u64(base) != 0 || load_u64(base + 8 * L.n_chunks) != total_bits) return AFX_E_CORRUPT;
    for (uint64_t c = 0; c < L.n_chunks; ++c) {
        const uint64_t lo = load_u64(base + 8 * c), hi = load_u64(base + 8 * (c + 1));
        const uint64_t elems = std::min<uint64_t>(kChunk, n - c * kChunk);
        if (hi < lo || hi - lo > elems * kMaxLen || hi - lo < elems) return AFX_E_CORRUPT;
        const uint64_t g0 = c * kGroupsPerChunk;
        const uint64_t g1 = std::min<uint64_t>(g0 + kGroupsPerChunk, L.n_groups);
        uint32_t prev = 0;
        for (uint64_t g = g0; g < g1; ++g) {
            const uint32_t v = load_u16(gap + 2 * g);
            if ((g == g0 && v != 0) || v < prev || v > hi - lo) return AFX_E_CORRUPT;
            prev = v;
        }
    }
    if (out) {
        std::memset(out, 0, sizeof(*out));
        out->abi_version = AFX_ABI_VERSION;
        out->format_version = AFX_FORMAT_VERSION;
        out->n_elems = n;
        out->decoded_bytes = 2 * n;
        out->blob_bytes = L.blob_bytes;
        out->total_bits = total_bits;
        out->exp_words = exp_words;
        out->n_chunks = L.n_chunks;
        out->n_groups = L.n_groups;
        out->ndim = ndim;
        out->n_symbols = used;
        for (int d = 0; d < 4; ++d) out->shape[d] = shape[d];
        out->chunk_elems = kChunk;
        out->group_elems = kGroup;
        out->max_code_len = kMaxLen;
        out->longest_code = longest;
        out->off_code_len = L.off_code_len;
        out->off_chunk_base = L.off_chunk_base;
        out->off_gap = L.off_gap;
        out->off_signmant = L.off_signmant;
        out->off_exp = L.off_exp;
    }
    return AFX_OK;
}

// Check that an afx_info handed back by a caller still describes a blob this
// library can decode (it was produced by afx_query, possibly long ago).
int check_info(const afx_info *info) {
    if (!info) return AFX_E_INVALID_ARG;
    if (info->abi_version != AFX_ABI_VERSION || info->format_version != AFX_FORMAT_VERSION)
        return AFX_E_BAD_VERSION;
    if (info->n_elems > kMaxElems) return AFX_E_UNSUPPORTED;
    const Layout L = layout_for(info->n_elems, info->total_bits);
    if (info->exp_words != L.exp_words || info->n_chunks != L.n_chunks || info->n_groups != L.n_groups ||
        info->off_code_len != L.off_code_len || info->off_chunk_base != L.off_chunk_base ||
        info->off_gap != L.off_gap || info->off_signmant != L.off_signmant || info->off_exp != L.off_exp ||
        info->blob_bytes != L.blob_bytes || info->decoded_bytes != 2 * info->n_elems)
        return AFX_E_CORRUPT;
    return AFX_OK;
}

}  // namespace afx

using namespace afx;

extern "C" {

int afx_query(const void *blob_host, size_t blob_bytes, afx_info *info) {
    if (!blob_host || !info) return AFX_E_INVALID_ARG;
    afx_info tmp;
    const int rc = validate(static_cast<const uint8_t *>(blob_host), blob_bytes, &tmp);
    if (rc == AFX_OK) *info = tmp;
    return rc;
}

const char *afx_status_str(int status) {
    switch (status) {
        case AFX_OK: return "ok";
        case AFX_E_INVALID_ARG: return "invalid argument";
        case AFX_E_BAD_MAGIC: return "not an AFX1 blob";
        case AFX_E_BAD_VERSION: return "unsupported format version or fixed field";
        case AFX_E_CORRUPT: return "corrupt blob (header, code lengths, chunk bases or gaps)";
        case AFX_E_BUFFER_TOO_SMALL: return "buffer too small";
        case AFX_E_MISALIGNED: return "device pointer not 16-byte aligned";
        case AFX_E_HIP: return "HIP runtime error";
        case AFX_E_UNSUPPORTED: return "unsupported request";
        case AFX_E_IO: return "file could not be opened or read in full";
        case AFX_E_HOST_MEMORY: return "host memory could not be allocated";
        default: return "unknown status";
    }
}

static int encode_plan(const uint16_t *x, uint64_t n, int threads, uint8_t code_len[256], uint64_t *total_bits,
                       uint64_t *blob_bytes) {
    if ((!x && n) || !code_len || !total_bits || !blob_bytes) return AFX_E_INVALID_ARG;
    if (n > kMaxElems) return AFX_E_UNSUPPORTED;
    const int T = thread_count(threads, n / (1 << 20) + 1);
    std::vector<uint64_t> hist((size_t)T * 256, 0);
    parallel_ranges(T, n, [&](int t, uint64_t a, uint64_t b) {
        uint64_t *h = hist.data() + (size_t)t * 256;
        for (uint64_t i = a; i < b; ++i) h[(x[i] >> 7) & 0xFF]++;
    });
    uint64_t freq[256] = {0};
    for (int t = 0; t < T; ++t)
        for (int s = 0; s < 256; ++s) freq[s] += hist[(size_t)t * 256 + s];
    uint8_t len[256];
    const int rc = limited_lengths(freq, (int)kMaxLen, len);
    if (rc != AFX_OK) return rc;
    uint64_t bits = 0;
    for (int s = 0; s < 256; ++s) bits += freq[s] * len[s];
    std::memcpy(code_len, len, 256);
    *total_bits = bits;
    *blob_bytes = layout_for(n, bits).blob_bytes;
    return AFX_OK;
}

static int encode(const uint16_t *x, uint64_t n, uint32_t ndim, const uint64_t *shape, const uint8_t code_len[256],
                  uint64_t total_bits, void *blob_out, size_t blob_bytes, int threads) {
    if ((!x && n) || !code_len || !blob_out || ndim < 1 || ndim > 4 || !shape) return AFX_E_INVALID_ARG;
    if (n > kMaxElems) return AFX_E_UNSUPPORTED;
    uint64_t prod = 1;
    for (uint32_t d = 0; d < ndim; ++d) {
        if (shape[d] && prod > kMaxElems / shape[d]) return AFX_E_INVALID_ARG;  // would wrap
        prod *= shape[d];
    }
    if (prod != n) return AFX_E_INVALID_ARG;
    if (total_bits > n * kMaxLen) return AFX_E_INVALID_ARG;
    // The lengths must form a complete prefix code (as afx_query demands):
    // Kraft sum exactly 1, or a single symbol of length 1.
    uint32_t used = 0, longest = 0;
    uint64_t kraft = 0;  // in units of 2^-12
    for (int s = 0; s < 256; ++s) {
        if (code_len[s] > kMaxLen) return AFX_E_INVALID_ARG;
        if (code_len[s]) {
            ++used;
            longest = std::max<uint32_t>(longest, code_len[s]);
            kraft += (uint64_t)1 << (kMaxLen - code_len[s]);
        }
    }
    if ((n == 0) != (used == 0)) return AFX_E_INVALID_ARG;
    if (used == 1 && longest != 1) return AFX_E_INVALID_ARG;
    if (used >= 2 && kraft != ((uint64_t)1 << kMaxLen)) return AFX_E_INVALID_ARG;
    const Layout L = layout_for(n, total_bits);
    if (blob_bytes < L.blob_bytes) return AFX_E_BUFFER_TOO_SMALL;
    uint32_t code[256];
    canonical(code_len, code);
    uint8_t *b = static_cast<uint8_t *>(blob_out);

    // Bits per chunk, then chunk bases by prefix sum.
    const int T = thread_count(threads, L.n_chunks);
    std::vector<uint64_t> chunk_bits(L.n_chunks + 1, 0);
    std::vector<int> bad(T, 0);
    parallel_ranges(T, L.n_chunks, [&](int t, uint64_t c0, uint64_t c1) {
        for (uint64_t c = c0; c < c1; ++c) {
            const uint64_t i0 = c * kChunk, i1 = std::min<uint64_t>(i0 + kChunk, n);
            uint64_t s = 0;
            for (uint64_t i = i0; i < i1; ++i) {
                const uint32_t l = code_len[(x[i] >> 7) & 0xFF];
                if (!l) bad[t] = 1;
                s += l;
            }
            chunk_bits[c] = s;
        }
    });
    for (int t = 0; t < T; ++t)
        if (bad[t]) return AFX_E_INVALID_ARG;
    uint64_t run = 0;
    for (uint64_t c = 0; c < L.n_chunks; ++c) {
        const uint64_t v = chunk_bits[c];
        chunk_bits[c] = run;
        run += v;
    }
    chunk_bits[L.n_chunks] = run;
    if (run != total_bits) return AFX_E_INVALID_ARG;

    // Header and fixed sections.
    std::memset(b, 0, L.off_code_len + 256);
    std::memcpy(b, "AFX1", 4);
    auto put32 = [&](size_t off, uint32_t v) { std::memcpy(b + off, &v, 4); };
    auto put64 = [&](size_t off, uint64_t v) { std::memcpy(b + off, &v, 8); };
    put32(4, AFX_FORMAT_VERSION);
    put64(8, n);
    put64(16, total_bits);
    put64(24, L.exp_words);
    put32(32, ndim);
    put32(36, kChunk);
    put32(40, kGroup);
    put32(44, kMaxLen);
    put32(48, used);
    for (uint32_t d = 0; d < ndim; ++d) put64(64 + 8 * d, shape[d]);
    std::memcpy(b + L.off_code_len, code_len, 256);
    std::memcpy(b + L.off_chunk_base, chunk_bits.data(), 8 * (L.n_chunks + 1));
    // zero the alignment padding between and after sections
    std::memset(b + L.off_chunk_base + 8 * (L.n_chunks + 1), 0,
                L.off_gap - (L.off_chunk_base + 8 * (L.n_chunks + 1)));
    std::memset(b + L.off_gap + 2 * L.n_groups, 0, L.off_signmant - (L.off_gap + 2 * L.n_groups));
    std::memset(b + L.off_signmant + n, 0, L.off_exp - (L.off_signmant + n));
    uint32_t *words = reinterpret_cast<uint32_t *>(b + L.off_exp);
    const uint64_t data_words = (total_bits + 31) / 32;
    std::memset(words + data_words, 0, (size_t)(L.blob_bytes - L.off_exp - 4 * data_words));

    // Streams. Each thread owns a contiguous range of chunks and writes the
    // words that lie entirely inside its bit range; the (at most two) words
    // it shares with its neighbours are OR-ed in after the join.
    uint16_t *gaps = reinterpret_cast<uint16_t *>(b + L.off_gap);
    uint8_t *sm = b + L.off_signmant;
    struct Edge { uint64_t word; uint32_t bits; };
    std::vector<Edge> edges((size_t)T * 2, Edge{~(uint64_t)0, 0});
    parallel_ranges(T, L.n_chunks, [&](int t, uint64_t c0, uint64_t c1) {
        if (c0 >= c1) return;
        const uint64_t bit0 = chunk_bits[c0], bit1 = chunk_bits[c1];
        const uint64_t first_word = bit0 / 32;
        const uint64_t last_word = (bit1 - 1) / 32;  // every chunk holds >= 1 bit
        uint64_t cur_word = first_word;
        uint64_t pos = bit0;
        uint64_t acc = 0;              // pending bits, right-aligned
        int nacc = (int)(bit0 % 32);   // zeros standing in for the shared prefix
        auto flush_word = [&](uint32_t v) {
            if (cur_word == first_word && bit0 % 32 != 0) edges[2 * t] = {cur_word, v};
            else if (cur_word == last_word && bit1 % 32 != 0) edges[2 * t + 1] = {cur_word, v};
            else words[cur_word] = v;
            ++cur_word;
        };
        for (uint64_t c = c0; c < c1; ++c) {
            const uint64_t cb = chunk_bits[c];
            const uint64_t i0 = c * kChunk, i1 = std::min<uint64_t>(i0 + kChunk, n);
            for (uint64_t i = i0; i < i1; ++i) {
                if ((i & (kGroup - 1)) == 0) gaps[i / kGroup] = (uint16_t)(pos - cb);
                const uint16_t h = x[i];
                const uint32_t e = (h >> 7) & 0xFF;
                sm[i] = (uint8_t)(((h >> 8) & 0x80) | (h & 0x7F));
                const uint32_t l = code_len[e];
                acc = (acc << l) | code[e];
                nacc += (int)l;
                pos += l;
                if (nacc >= 32) {
                    nacc -= 32;
                    flush_word((uint32_t)(acc >> nacc));
                }
            }
        }
        if (nacc > 0) flush_word((uint32_t)(acc << (32 - nacc)));
    });
    for (auto &e : edges)
        if (e.word != ~(uint64_t)0) words[e.word] = 0;
    for (auto &e : edges)
        if (e.word != ~(uint64_t)0) words[e.word] |= e.bits;
    return AFX_OK;
}

int afx_encode_plan(const uint16_t *x, uint64_t n, int threads, uint8_t code_len[256], uint64_t *total_bits,
                    uint64_t *blob_bytes) {
    try {
        return encode_plan(x, n, threads, code_len, total_bits, blob_bytes);
    } catch (const std::bad_alloc &) {
        return AFX_E_HOST_MEMORY;
    }
}

int afx_encode(const uint16_t *x, uint64_t n, uint32_t ndim, const uint64_t *shape, const uint8_t code_len[256],
               uint64_t total_bits, void *blob_out, size_t blob_bytes, int threads) {
    try {
        return encode(x, n, ndim, shape, code_len, total_bits, blob_out, blob_bytes, threads);
    } catch (const std::bad_alloc &) {
        return AFX_E_HOST_MEMORY;
    }
}

}  // extern "C"
