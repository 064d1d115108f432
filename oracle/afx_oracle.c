/*
 * afx_oracle.c -- plain, slow CPU oracle for the lossless BF16 exponent codec.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this file. The GPU library shares no
 * code, header, table or constant generator with it.
 *
 * What it computes. "Why Weight Offloading Slows Inference" (section
 * "Lossless compression") codes the BF16 exponent field with Huffman's
 * minimum-redundancy prefix code (1952, that page's reference [2]): frequent
 * exponents cost fewer bits, nothing is lost, and decoding gives back every
 * weight's original 16 bits. The pages fix nothing else, so this oracle
 * takes these readings:
 *
 *   - BF16 layout: bit 15 sign, bits 14..7 biased exponent, bits 6..0
 *     mantissa. The 8-bit exponent field is the coded symbol (all 256 values,
 *     including 0 and 255); sign and mantissa are kept raw as one byte
 *     (sign << 7) | mantissa.
 *   - One code per tensor: an optimal prefix code whose lengths are limited
 *     to 12 bits, found by package-merge (Larmore and Hirschberg, 1990),
 *     made canonical (symbols ordered by (length, value); DEFLATE-style
 *     consecutive codes). A tensor with one distinct exponent uses length 1.
 *   - One bit stream per tensor, MSB first inside little-endian u32 words.
 *     Every 4096 elements (a chunk) the absolute bit position is recorded as
 *     a u64; every 32 elements (a group) the offset from the chunk's position
 *     is recorded as a u16.
 *
 * Blob layout (little-endian; every section starts on a 256-byte boundary):
 *   header (256 B: magic "AFX1", version 1, n, total_bits, exp_words, ndim,
 *   4096, 32, 12, n_symbols, shape[4]), code_len[256] u8,
 *   chunk_base[n_chunks + 1] u64, gap[n_groups] u16, signmant[n] u8,
 *   exp[exp_words] u32 (the code stream, zero padded to whole words plus
 *   four zero words). The blob ends on a 256-byte boundary, zero filled.
 *
 * The decoder deliberately uses a different procedure from any table-driven
 * decoder: it reads the stream one bit at a time and walks the canonical
 * code length by length (count and first code per length).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_E_ARG (-1)
#define OR_E_FORMAT (-2)
#define OR_E_MISMATCH (-3)
#define OR_E_NOMEM (-4)

#define OR_CHUNK 4096u
#define OR_GROUP 32u
#define OR_LMAX 12u
#define OR_PAD_WORDS 4u
#define OR_ALIGN 256u

static uint64_t align_up(uint64_t v) { return (v + OR_ALIGN - 1) / OR_ALIGN * OR_ALIGN; }

static uint32_t rd32(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static uint64_t rd64(const uint8_t *p) { return (uint64_t)rd32(p) | ((uint64_t)rd32(p + 4) << 32); }
static void wr32(uint8_t *p, uint32_t v) {
    p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); p[2] = (uint8_t)(v >> 16); p[3] = (uint8_t)(v >> 24);
}
static void wr64(uint8_t *p, uint64_t v) { wr32(p, (uint32_t)v); wr32(p + 4, (uint32_t)(v >> 32)); }

/* ------------------------------------------------------------------------
 * Section offsets. off[0] code_len, off[1] chunk_base, off[2] gap,
 * off[3] signmant, off[4] exp, off[5] total blob bytes.
 * ------------------------------------------------------------------------ */
int afx_oracle_layout(uint64_t n, uint64_t total_bits, uint64_t off[6]) {
    uint64_t n_chunks = (n + OR_CHUNK - 1) / OR_CHUNK;
    uint64_t n_groups = (n + OR_GROUP - 1) / OR_GROUP;
    uint64_t exp_words = (total_bits + 31) / 32 + OR_PAD_WORDS;
    off[0] = 256;
    off[1] = 512;
    off[2] = align_up(off[1] + 8 * (n_chunks + 1));
    off[3] = align_up(off[2] + 2 * n_groups);
    off[4] = align_up(off[3] + n);
    off[5] = align_up(off[4] + 4 * exp_words);
    return OR_OK;
}

uint64_t afx_oracle_blob_bytes(uint64_t n, uint64_t total_bits) {
    uint64_t off[6];
    afx_oracle_layout(n, total_bits, off);
    return off[5];
}

/* ------------------------------------------------------------------------
 * Package-merge: optimal code lengths under a length limit.
 *
 * Items of the coin collector's problem: each symbol is a coin of every
 * denomination 2^-1 .. 2^-lmax with the symbol's frequency as its cost. The
 * lists are built from the smallest denomination (level lmax) up: the list at
 * level j merges the leaves with the packages made from consecutive pairs of
 * the level j+1 list. The first 2m-2 items of the level-1 list form the
 * cheapest collection of total denomination m-1; a symbol's length is the
 * number of levels at which its leaf is part of the selection.
 * ------------------------------------------------------------------------ */
typedef struct { uint64_t w; int leaf; } pm_item;  /* leaf >= 0: symbol rank; -1: package */

static void sort_by_weight(const uint64_t *freq, int *sym, int m) {
    /* insertion sort by (freq, symbol) ascending: m <= 256 */
    for (int i = 1; i < m; i++) {
        int s = sym[i], j = i - 1;
        while (j >= 0 && (freq[sym[j]] > freq[s] || (freq[sym[j]] == freq[s] && sym[j] > s))) {
            sym[j + 1] = sym[j];
            j--;
        }
        sym[j + 1] = s;
    }
}

int afx_oracle_code_lengths(const uint64_t *freq, int nsym, int lmax, uint8_t *len) {
    if (!freq || !len || nsym < 0 || nsym > 4096 || lmax < 1 || lmax > 32) return OR_E_ARG;
    int *sym = (int *)malloc(sizeof(int) * (size_t)(nsym > 0 ? nsym : 1));
    if (!sym) return OR_E_NOMEM;
    int m = 0;
    for (int s = 0; s < nsym; s++) {
        len[s] = 0;
        if (freq[s] > 0) sym[m++] = s;
    }
    if (m == 0) { free(sym); return OR_OK; }
    if (m == 1) { len[sym[0]] = 1; free(sym); return OR_OK; }
    if (lmax < 31 && (1u << lmax) < (unsigned)m) { free(sym); return OR_E_ARG; }
    sort_by_weight(freq, sym, m);

    /* lists[j] for j = 1..lmax (index 0 unused); each has at most 2m-1 items */
    size_t cap = (size_t)2 * (size_t)m;
    pm_item *lists = (pm_item *)malloc(sizeof(pm_item) * cap * (size_t)(lmax + 1));
    int *count = (int *)calloc((size_t)lmax + 1, sizeof(int));
    if (!lists || !count) { free(sym); free(lists); free(count); return OR_E_NOMEM; }

    /* deepest level: the leaves alone */
    pm_item *deep = lists + cap * (size_t)lmax;
    for (int i = 0; i < m; i++) { deep[i].w = freq[sym[i]]; deep[i].leaf = i; }
    count[lmax] = m;
    for (int j = lmax - 1; j >= 1; j--) {
        pm_item *below = lists + cap * (size_t)(j + 1);
        pm_item *cur = lists + cap * (size_t)j;
        int npk = count[j + 1] / 2, li = 0, pi = 0, k = 0;
        while (li < m || pi < npk) {
            uint64_t pw = pi < npk ? below[2 * pi].w + below[2 * pi + 1].w : 0;
            /* ties: the leaf comes first */
            if (li < m && (pi >= npk || freq[sym[li]] <= pw)) {
                cur[k].w = freq[sym[li]]; cur[k].leaf = li; li++;
            } else {
                cur[k].w = pw; cur[k].leaf = -1; pi++;
            }
            k++;
        }
        count[j] = k;
    }

    /* walk the selection down the levels */
    int take = 2 * m - 2;
    for (int j = 1; j <= lmax && take > 0; j++) {
        pm_item *cur = lists + cap * (size_t)j;
        if (take > count[j]) { free(sym); free(lists); free(count); return OR_E_ARG; }
        int packages = 0;
        for (int i = 0; i < take; i++) {
            if (cur[i].leaf >= 0) len[sym[cur[i].leaf]]++;
            else packages++;
        }
        take = 2 * packages;
    }
    free(sym); free(lists); free(count);
    return OR_OK;
}

/* Canonical codes: symbols in (length, value) order get consecutive codes;
 * moving to a longer length appends zeros. */
static void canonical_codes(const uint8_t len[256], uint32_t code[256]) {
    int order[256], m = 0;
    for (int l = 1; l <= 32; l++)
        for (int s = 0; s < 256; s++)
            if (len[s] == l) order[m++] = s;
    uint32_t c = 0;
    for (int i = 0; i < m; i++) {
        if (i > 0) c = (c + 1) << (len[order[i]] - len[order[i - 1]]);
        code[order[i]] = c;
    }
}

/* ------------------------------------------------------------------------
 * Encoder
 * ------------------------------------------------------------------------ */
int afx_oracle_plan(const uint16_t *x, uint64_t n, int lmax, uint8_t len[256], uint64_t *total_bits) {
    if ((!x && n) || !len || !total_bits || lmax < 1 || lmax > 12) return OR_E_ARG;
    uint64_t freq[256];
    memset(freq, 0, sizeof(freq));
    for (uint64_t i = 0; i < n; i++) freq[(x[i] >> 7) & 0xFF]++;
    int rc = afx_oracle_code_lengths(freq, 256, lmax, len);
    if (rc) return rc;
    uint64_t bits = 0;
    for (int s = 0; s < 256; s++) bits += freq[s] * len[s];
    *total_bits = bits;
    return OR_OK;
}

static void put_bits(uint8_t *exp_bytes, uint64_t *pos, uint32_t code, int len) {
    for (int b = len - 1; b >= 0; b--) {
        if ((code >> b) & 1u) {
            uint64_t w = *pos / 32, k = 31 - (*pos % 32);
            uint8_t *p = exp_bytes + 4 * w;
            wr32(p, rd32(p) | (1u << k));
        }
        (*pos)++;
    }
}

int afx_oracle_encode(const uint16_t *x, uint64_t n, uint32_t ndim, const uint64_t *shape,
                      const uint8_t len[256], uint64_t total_bits, uint8_t *blob, uint64_t blob_bytes) {
    if ((!x && n) || !len || !blob || ndim > 4 || (ndim && !shape)) return OR_E_ARG;
    uint64_t off[6];
    afx_oracle_layout(n, total_bits, off);
    if (blob_bytes < off[5]) return OR_E_ARG;
    uint64_t prod = 1;
    for (uint32_t d = 0; d < ndim; d++) prod *= shape[d];
    if (ndim ? prod != n : n != 1) return OR_E_ARG;
    int used = 0;
    for (int s = 0; s < 256; s++) {
        if (len[s] > OR_LMAX) return OR_E_ARG;
        used += len[s] > 0;
    }
    uint32_t code[256];
    memset(code, 0, sizeof(code));
    canonical_codes(len, code);

    uint64_t n_chunks = (n + OR_CHUNK - 1) / OR_CHUNK;
    uint64_t exp_words = (total_bits + 31) / 32 + OR_PAD_WORDS;
    memset(blob, 0, off[5]);
    memcpy(blob, "AFX1", 4);
    wr32(blob + 4, 1);
    wr64(blob + 8, n);
    wr64(blob + 16, total_bits);
    wr64(blob + 24, exp_words);
    wr32(blob + 32, ndim);
    wr32(blob + 36, OR_CHUNK);
    wr32(blob + 40, OR_GROUP);
    wr32(blob + 44, OR_LMAX);
    wr32(blob + 48, (uint32_t)used);
    for (uint32_t d = 0; d < ndim; d++) wr64(blob + 64 + 8 * d, shape[d]);
    memcpy(blob + off[0], len, 256);

    uint8_t *base_p = blob + off[1], *gap_p = blob + off[2], *sm_p = blob + off[3], *exp_p = blob + off[4];
    uint64_t pos = 0, cbase = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (i % OR_CHUNK == 0) { cbase = pos; wr64(base_p + 8 * (i / OR_CHUNK), pos); }
        if (i % OR_GROUP == 0) {
            uint64_t g = i / OR_GROUP, d = pos - cbase;
            gap_p[2 * g] = (uint8_t)d;
            gap_p[2 * g + 1] = (uint8_t)(d >> 8);
        }
        uint16_t h = x[i];
        uint32_t e = (h >> 7) & 0xFF;
        if (len[e] == 0) return OR_E_ARG;
        sm_p[i] = (uint8_t)(((h >> 8) & 0x80) | (h & 0x7F));
        put_bits(exp_p, &pos, code[e], len[e]);
    }
    wr64(base_p + 8 * n_chunks, pos);
    return pos == total_bits ? OR_OK : OR_E_ARG;
}

/* ------------------------------------------------------------------------
 * Decoder
 * ------------------------------------------------------------------------ */
typedef struct {
    const uint8_t *blob;
    uint64_t n, total_bits, exp_words, n_chunks;
    uint64_t off[6];
    int count[OR_LMAX + 1];      /* symbols of each length */
    uint32_t first[OR_LMAX + 1]; /* first canonical code of each length */
    int offset[OR_LMAX + 1];     /* index of that length's first symbol in sorted[] */
    uint8_t sorted[256];         /* symbols in (length, value) order */
} or_dec;

static int parse(const uint8_t *blob, uint64_t blob_bytes, or_dec *d) {
    if (!blob || blob_bytes < 512) return OR_E_FORMAT;
    if (memcmp(blob, "AFX1", 4) != 0 || rd32(blob + 4) != 1) return OR_E_FORMAT;
    if (rd32(blob + 36) != OR_CHUNK || rd32(blob + 40) != OR_GROUP || rd32(blob + 44) != OR_LMAX)
        return OR_E_FORMAT;
    d->blob = blob;
    d->n = rd64(blob + 8);
    d->total_bits = rd64(blob + 16);
    d->exp_words = rd64(blob + 24);
    if (d->n > ((uint64_t)1 << 40) || d->total_bits > d->n * OR_LMAX) return OR_E_FORMAT;
    if (d->exp_words != (d->total_bits + 31) / 32 + OR_PAD_WORDS) return OR_E_FORMAT;
    afx_oracle_layout(d->n, d->total_bits, d->off);
    if (blob_bytes < d->off[5]) return OR_E_FORMAT;
    d->n_chunks = (d->n + OR_CHUNK - 1) / OR_CHUNK;

    const uint8_t *len = blob + d->off[0];
    int used = 0;
    uint64_t kraft = 0;
    memset(d->count, 0, sizeof(d->count));
    for (int s = 0; s < 256; s++) {
        if (len[s] > OR_LMAX) return OR_E_FORMAT;
        if (len[s]) { used++; d->count[len[s]]++; kraft += (uint64_t)1 << (OR_LMAX - len[s]); }
    }
    if ((uint32_t)used != rd32(blob + 48)) return OR_E_FORMAT;
    if (d->n == 0 ? used != 0 : used == 0) return OR_E_FORMAT;
    if (used == 1 && d->count[1] != 1) return OR_E_FORMAT;
    if (used >= 2 && kraft != ((uint64_t)1 << OR_LMAX)) return OR_E_FORMAT;

    /* canonical tables, textbook style: first code of each length */
    uint32_t code = 0;
    int idx = 0;
    d->count[0] = 0;
    for (int l = 1; l <= (int)OR_LMAX; l++) {
        code = (code + (uint32_t)d->count[l - 1]) << 1;
        d->first[l] = code;
        d->offset[l] = idx;
        for (int s = 0; s < 256; s++)
            if (len[s] == l) d->sorted[idx++] = (uint8_t)s;
    }
    return OR_OK;
}

static int bit_at(const or_dec *d, uint64_t pos) {
    const uint8_t *w = d->blob + d->off[4] + 4 * (pos / 32);
    return (int)((rd32(w) >> (31 - pos % 32)) & 1u);
}

static uint64_t chunk_base(const or_dec *d, uint64_t c) { return rd64(d->blob + d->off[1] + 8 * c); }
static uint64_t gap_of(const or_dec *d, uint64_t g) {
    const uint8_t *p = d->blob + d->off[2] + 2 * g;
    return (uint64_t)p[0] | ((uint64_t)p[1] << 8);
}

/* Decode one canonical symbol starting at *pos; -1 on an invalid code. */
static int read_symbol(const or_dec *d, uint64_t *pos) {
    uint32_t code = 0;
    for (int l = 1; l <= (int)OR_LMAX; l++) {
        if (*pos >= d->total_bits) return -1;
        code = (code << 1) | (uint32_t)bit_at(d, *pos);
        (*pos)++;
        if (code - d->first[l] < (uint32_t)d->count[l]) return d->sorted[d->offset[l] + (int)(code - d->first[l])];
    }
    return -1;
}

/* Decode chunks [c0, c1) into out (elements of those chunks, in order),
 * checking every chunk and group position against the recorded ones. */
static int decode_range(const or_dec *d, uint64_t c0, uint64_t c1, uint16_t *out) {
    const uint8_t *sm = d->blob + d->off[3];
    for (uint64_t c = c0; c < c1; c++) {
        uint64_t pos = chunk_base(d, c), base = pos;
        uint64_t i0 = c * OR_CHUNK, i1 = i0 + OR_CHUNK < d->n ? i0 + OR_CHUNK : d->n;
        for (uint64_t i = i0; i < i1; i++) {
            if (i % OR_GROUP == 0 && pos != base + gap_of(d, i / OR_GROUP)) return OR_E_MISMATCH;
            int e = read_symbol(d, &pos);
            if (e < 0) return OR_E_MISMATCH;
            uint8_t b = sm[i];
            out[i - c0 * OR_CHUNK] = (uint16_t)(((b & 0x80) << 8) | ((uint32_t)e << 7) | (b & 0x7F));
        }
        if (pos != chunk_base(d, c + 1)) return OR_E_MISMATCH;
    }
    return OR_OK;
}

typedef struct { const or_dec *d; uint64_t c0, c1; uint16_t *out; int rc; } or_job;

static void *run_job(void *arg) {
    or_job *j = (or_job *)arg;
    j->rc = decode_range(j->d, j->c0, j->c1, j->out);
    return NULL;
}

int afx_oracle_decode_chunks(const uint8_t *blob, uint64_t blob_bytes, uint64_t c0, uint64_t c1,
                             uint16_t *out, uint64_t out_elems, int threads) {
    or_dec d;
    int rc = parse(blob, blob_bytes, &d);
    if (rc) return rc;
    if (c0 > c1 || c1 > d.n_chunks) return OR_E_ARG;
    uint64_t e0 = c0 * OR_CHUNK, e1 = c1 * OR_CHUNK < d.n ? c1 * OR_CHUNK : d.n;
    if (c1 > c0 && (!out || out_elems < e1 - e0)) return OR_E_ARG;
    if (chunk_base(&d, 0) != 0 || chunk_base(&d, d.n_chunks) != d.total_bits) return OR_E_MISMATCH;
    if (threads < 1) threads = 1;
    if ((uint64_t)threads > c1 - c0) threads = (int)(c1 - c0 > 0 ? c1 - c0 : 1);
    if (threads == 1) return decode_range(&d, c0, c1, out);

    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)threads);
    or_job *jobs = (or_job *)malloc(sizeof(or_job) * (size_t)threads);
    if (!tid || !jobs) { free(tid); free(jobs); return OR_E_NOMEM; }
    uint64_t span = c1 - c0;
    int started = 0;
    for (int t = 0; t < threads; t++) {
        uint64_t a = c0 + span * (uint64_t)t / (uint64_t)threads;
        uint64_t b = c0 + span * (uint64_t)(t + 1) / (uint64_t)threads;
        jobs[t].d = &d; jobs[t].c0 = a; jobs[t].c1 = b; jobs[t].out = out + (a - c0) * OR_CHUNK; jobs[t].rc = 0;
        if (pthread_create(&tid[t], NULL, run_job, &jobs[t]) != 0) { jobs[t].rc = OR_E_NOMEM; break; }
        started++;
    }
    rc = OR_OK;
    for (int t = 0; t < started; t++) pthread_join(tid[t], NULL);
    for (int t = 0; t < threads; t++)
        if (t >= started || jobs[t].rc) { rc = t >= started ? OR_E_NOMEM : jobs[t].rc; break; }
    free(tid); free(jobs);
    return rc;
}

/* Sequential whole-stream decode (threads <= 1) or chunk-parallel decode. */
int afx_oracle_decode(const uint8_t *blob, uint64_t blob_bytes, uint16_t *out, uint64_t out_elems, int threads) {
    or_dec d;
    int rc = parse(blob, blob_bytes, &d);
    if (rc) return rc;
    if (d.n && (!out || out_elems < d.n)) return OR_E_ARG;
    if (threads > 1) return afx_oracle_decode_chunks(blob, blob_bytes, 0, d.n_chunks, out, out_elems, threads);
    if (chunk_base(&d, 0) != 0 || chunk_base(&d, d.n_chunks) != d.total_bits) return OR_E_MISMATCH;
    /* one pass over the whole stream, position carried across chunks */
    const uint8_t *sm = d.blob + d.off[3];
    uint64_t pos = 0, base = 0;
    for (uint64_t i = 0; i < d.n; i++) {
        if (i % OR_CHUNK == 0) {
            base = chunk_base(&d, i / OR_CHUNK);
            if (pos != base) return OR_E_MISMATCH;
        }
        if (i % OR_GROUP == 0 && pos != base + gap_of(&d, i / OR_GROUP)) return OR_E_MISMATCH;
        int e = read_symbol(&d, &pos);
        if (e < 0) return OR_E_MISMATCH;
        uint8_t b = sm[i];
        out[i] = (uint16_t)(((b & 0x80) << 8) | ((uint32_t)e << 7) | (b & 0x7F));
    }
    return pos == d.total_bits ? OR_OK : OR_E_MISMATCH;
}
