// afx_gemm.hip -- the restore fused into a matrix product on the matrix cores
// (gfx950): Y += X W^T for a weight matrix W held only in its coded form.
//
// "Why Weight Offloading Slows Inference" (section "Lossless compression")
// reconstructs a coded weight's bits ahead of the computation that uses it.
// For a product over many tokens at once (a prompt), restoring W into HBM first
// writes and rereads 2 bytes per weight; here tiles of W are restored into
// LDS and consumed there by MFMA, and only the coded matrix is read from HBM.
//
// W is row-major [rows, cols] (the blob's element order), X is BF16 [m, cols]
// and Y is FP32 [m, rows], both row-major: Y[t, r] += sum_k X[t, k] W[r, k].
//
// Work decomposition:
//   * a tile is 64 rows of W by a range of up to 2560 columns (5120 when a
//     workgroup takes 256 tokens); a workgroup of 4 wave64s takes one tile
//     and up to 256 tokens (the block index picks the token block). Every
//     tile adds its partial sums into Y with atomic adds, so ranges of one
//     row may run on different workgroups;
//   * the tile's columns are restored 256 at a time (a slab of 64 x 256
//     values). A 32-element group decodes on its own from its chunk's bit
//     base and its gap, so a slab is 64 x 8 groups: wave w restores rows
//     16w..16w+15, one quad of lanes per row, two groups per lane. The row's
//     code words for the slab (one contiguous bit range) are staged in LDS by
//     its quad; each lane then runs its two groups' table-driven chains;
//   * the restored slab goes to LDS in row-major order (rows padded by 16
//     bytes), where it is the B operand of v_mfma_f32_32x32x16_bf16: wave w
//     multiplies tokens 32w..32w+31 (X read from L2 straight into the A
//     operand) with the slab's two 32-row halves.
// Lane layout of v_mfma_f32_32x32x16_bf16: lane l holds A[l % 32][8 (l / 32)
// + 0..7] and B[8 (l / 32) + 0..7][l % 32]; accumulator v of lane l is
// D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
#include <hip/hip_runtime.h>

#include "afx_device.h"

namespace afx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = kGemmWaves * kWave;             // 256
constexpr uint32_t kTileRows = 64;                           // W rows per tile (two MFMA N blocks)
constexpr uint32_t kSlabCols = 256;                          // columns restored per step
constexpr uint32_t kRangeSlabs = 10;                         // slabs per tile per 32-token block of a wave
// Columns of a tile: 2560 with one 32-token block per wave, 5120 with two
// (their slabs take longer to multiply, so fewer tiles balance the grid).
template <int kB>
constexpr uint32_t range_cols() { return kRangeSlabs * kB * kSlabCols; }
constexpr uint32_t kMaxTokenBlocks = 2;                      // 32-token blocks per wave (1 or 2)
constexpr uint32_t kRowsPerWave = kTileRows / kGemmWaves;    // 16
// A row segment's code words (kSegWords, staged in reverse in a slice of
// kSegRow words: afx_index.h), so that the decoding chains of afx_device.h
// apply.
static_assert(kSegWords * 32 >= kSlabCols * kMaxLen + 5 * 32, "a segment's words fit its slice");
constexpr uint32_t kSlabStride = kSlabCols * 2 + 16;         // bytes per restored row in LDS

struct GemmJob {
    TensorDesc t;        // t.out, t.blk_* unused
    const uint16_t *x;   // BF16 [m, cols]
    float *y;            // FP32 [m, rows], added into
    uint32_t rows, cols;
    uint32_t tile0;      // first tile of this job in the grid
    uint32_t n_rtiles;   // rows / 64
};

struct GemmBatch {
    GemmJob j[AFX_MAX_GEMV_JOBS_PER_LAUNCH];
    uint32_t n;
    uint32_t m;
    uint32_t tiles;  // tiles of all jobs
    uint32_t n_tok;  // token blocks (workgroups per tile)
};

// 16 bytes of x as the A operand (zeros for a token beyond m).
__device__ inline bf16x8 load_a(const uint16_t *p, bool ok) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ok) v = *reinterpret_cast<const uint4 *>(p);
    return __builtin_bit_cast(bf16x8, v);
}

// Stage four stream words (those at wa + i .. wa + i + 3) of a row segment,
// reversed: stream word wa + j goes to index kSegRev - j.
__device__ inline void put_seg4(uint32_t *seg, uint32_t i, uint4 v) {
    *reinterpret_cast<uint4 *>(seg + seg_put_index(i)) = make_uint4(v.w, v.z, v.y, v.x);
}

// Decode the 32 exponent codes of the lane's two groups, whose chains start
// at counters r1 and r2 of the row's staged segment (two interleaved
// buffered chains); ex1[j], ex2[j] receive the exponent bytes of elements
// 4j..4j+3. The starts come clamped (seg_chain_r0), so that 32 codes of <=
// 12 bits, and the chains' read-ahead, remain inside the slice even on a
// corrupt stream.
__device__ inline void decode_groups(const uint32_t *seg, uint32_t r1, uint32_t r2, const uint16_t *lut,
                                     uint32_t (&ex1)[8], uint32_t (&ex2)[8]) {
    BufChain A = buf_chain(seg, r1);
    BufChain B = buf_chain(seg, r2);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        uint32_t a01, b01, a23, b23;
        buf_chain_pairs(A, B, seg, lut, a01, b01);
        buf_chain_pairs(A, B, seg, lut, a23, b23);
        ex1[q] = join_halves(a01, a23);
        ex2[q] = join_halves(b01, b23);
    }
}

__device__ inline uint64_t quad_first(uint64_t v) {  // every lane gets lane 4 (l / 4)'s value
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, 0x00, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), 0x00, 0xF, 0xF, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// What the bit offsets of a row segment (starting at element e_seg) are
// made of: chunk base and gap of the lane's two groups (q4 and q4 + 4 of the
// segment's 8) and of the group after the segment (at the end of the
// tensor: the stream's end, with gap 0). Kept as loaded and added up only
// where used, so that issuing them never waits for them.
struct SlabBits {
    uint64_t b1, b2, be;
    uint32_t g1, g2, ge;
    bool last;  // the segment ends the tensor
};
__device__ inline SlabBits slab_bits(const TensorDesc &T, uint64_t e_seg, uint32_t q4) {
    SlabBits b;
    const uint64_t e1 = e_seg + kGroup * q4, e2 = e1 + kGroup * 4, e_end = e_seg + kSlabCols;
    b.last = e_end >= T.n;
    b.b1 = T.chunk_base[e1 >> 12];
    b.g1 = T.gap[e1 >> 5];
    b.b2 = T.chunk_base[e2 >> 12];
    b.g2 = T.gap[e2 >> 5];
    b.be = T.chunk_base[b.last ? T.n_chunks : e_end >> 12];
    b.ge = T.gap[b.last ? 0 : e_end >> 5];
    return b;
}
__device__ inline uint64_t bit1(const SlabBits &b) { return b.b1 + b.g1; }
__device__ inline uint64_t bit2(const SlabBits &b) { return b.b2 + b.g2; }
__device__ inline uint64_t bit_end(const SlabBits &b) { return b.be + (b.last ? 0u : b.ge); }

// The segment's staged word range [wa, wa + nw) (16-byte aligned), the
// first 32 of those words (lane q4 of the quad holds words 4 q4.. and
// 16 + 4 q4..), and the sign/mantissa bytes of the lane's two groups.
struct SlabData {
    uint64_t wa;
    uint32_t nw;
    uint4 w0, w1;
    u32x4 s1a, s1b, s2a, s2b;
};
__device__ inline SlabData slab_data(const TensorDesc &T, uint64_t e_seg, uint32_t q4, const SlabBits &b) {
    SlabData d;
    const uint64_t p_lo = quad_first(bit1(b)), p_hi = bit_end(b);
    d.wa = seg_first_word(p_lo);
    d.nw = seg_words(p_lo, p_hi);
    // (words past the segment's end are staged too, and never read)
    d.w0 = load_words4(T, d.wa + 4 * q4);
    d.w1 = load_words4(T, d.wa + 16 + 4 * q4);
    // sign/mantissa bytes are read once: keep them out of the caches
    const u32x4 *sm1 = reinterpret_cast<const u32x4 *>(T.signmant + e_seg + kGroup * q4);
    const u32x4 *sm2 = reinterpret_cast<const u32x4 *>(T.signmant + e_seg + kGroup * (q4 + 4));
    d.s1a = __builtin_nontemporal_load(sm1);
    d.s1b = __builtin_nontemporal_load(sm1 + 1);
    d.s2a = __builtin_nontemporal_load(sm2);
    d.s2b = __builtin_nontemporal_load(sm2 + 1);
    return d;
}

// The workgroup's LDS as one object, the decode table first: at LDS address
// 0 a table read needs no base added to its index.
// Row r of the tile has one kSlabStride-byte slice: it holds the row's
// staged code words while the row decodes, then its restored values (the
// same lanes do both, so a wave-level order between them suffices).
static_assert(kSegRow * 4 <= kSlabStride, "a row's staged words fit its slab row");
struct GemmLds {
    uint16_t lut[kLutEntries];                    // 8 KB
    uint8_t slab[kTileRows * kSlabStride];        // 33 KB
    LutScratch scratch;
};

// kB: 32-token blocks per wave; kWays: waves that share a token block, each
// multiplying kSlabCols / 16 / kWays of the slab's 16-column steps (their
// partial sums meet in LDS at the end of the tile), so that no wave
// multiplies alone while the others wait at the barrier. A workgroup thus multiplies each restored slab with
// 32 kB (4 / kWays) tokens: 32 (kWays 4), 64 (2), 128 (1) or 256 (kB 2).
// With kB = 2, only the A operands of the slab's first 6 steps are fetched
// before the restore; each later step's are fetched 6 steps ahead, during
// the matrix instructions (250 registers, two waves per SIMD: 4 steps ahead
// left more of the loads' latency exposed, 8 spill). With 128 tokens per
// workgroup (kB = 1, kWays = 1) the lead is 5 of 16 steps, the most that
// keeps three workgroups per CU without spills.
template <int kB, int kWays>
__global__ __launch_bounds__(kGemmThreads, kB == 1 ? 3 : 2)
void afx_gemm_kernel(const GemmBatch batch) {
    __shared__ __attribute__((aligned(16))) GemmLds lds;
    uint16_t *lut = lds.lut;
    uint8_t *slab = lds.slab;
    LutScratch &scratch = lds.scratch;

    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // The launch order (afx_index.h): the workgroups that restore one tile
    // for different tokens run on the same XCD close in time and find its
    // compressed bytes in that XCD's L2.
    const uint32_t gtile = gemm_block_tile(blockIdx.x, batch.n_tok), tblk = gemm_block_token(blockIdx.x, batch.n_tok);
    if (gtile >= batch.tiles) return;  // the last run's padding
    uint32_t jb = 0;
    for (uint32_t i = 1; i < batch.n; ++i)
        if (gtile >= batch.j[i].tile0) jb = i;
    const GemmJob &J = batch.j[jb];
    const TensorDesc &T = J.t;
    const uint32_t tile = gtile - J.tile0;
    const uint32_t r0 = (tile % J.n_rtiles) * kTileRows;
    constexpr uint32_t kRangeCols = range_cols<kB>();
    const uint32_t kbeg = (tile / J.n_rtiles) * kRangeCols;
    const uint32_t kend = min(J.cols, kbeg + kRangeCols);
    static_assert(kGemmWaves % kWays == 0 && (kSlabCols / 16) % kWays == 0, "waves share a token block's steps");
    const uint32_t t0 = tblk * (32 * kB * (kGemmWaves / kWays));
    const uint32_t m = batch.m;

    // The code lengths and the first slabs' bit offsets are requested
    // together, then the first slab's words (which need the offsets); the
    // table is built while those are in flight.
    const uint32_t len = T.code_len[threadIdx.x];

    // Restore: this lane's row (one quad per row) and its two groups.
    const uint32_t q4 = (uint32_t)lane & 3;
    const uint32_t row = wave * kRowsPerWave + ((uint32_t)lane >> 2);  // tile-local
    const uint64_t row_e = (uint64_t)(r0 + row) * J.cols;              // element of W[r0 + row, 0]
    uint32_t *seg = reinterpret_cast<uint32_t *>(slab + row * kSlabStride);
    uint8_t *out_row = slab + row * kSlabStride;
    // Multiply: this lane's token (A row) in each of the wave's token blocks.
    const uint32_t t_wave = t0 + (wave / kWays) * 32 * kB;
    bool tok_ok[kB], blk_mul[kB];
    const uint16_t *xa_p[kB];
#pragma unroll
    for (int tb = 0; tb < kB; ++tb) {
        const uint32_t tok = t_wave + 32 * tb + ((uint32_t)lane & 31);
        tok_ok[tb] = tok < m;
        blk_mul[tb] = t_wave + 32 * tb < m;  // the block holds a token
        xa_p[tb] = J.x + (uint64_t)(tok_ok[tb] ? tok : 0) * J.cols + 8 * ((uint32_t)lane >> 5);
    }
    const bool wave_mul = blk_mul[0];
    const uint8_t *b_row0 = slab + ((uint32_t)lane & 31) * kSlabStride + 16 * ((uint32_t)lane >> 5);
    const uint8_t *b_row1 = b_row0 + 32 * kSlabStride;

    // Software pipeline over the slabs: while slab s is restored and
    // multiplied, the code words and sign/mantissa bytes of slab s + 1 and
    // the group bit offsets of slab s + 2 are in flight, so that the two
    // dependent round trips (offsets, then the words they point at) stay off
    // the path of every slab but the first.
    SlabBits bits_c = slab_bits(T, row_e + kbeg, q4);
    const bool two = kbeg + kSlabCols < kend;
    SlabBits bits_n = slab_bits(T, row_e + kbeg + (two ? kSlabCols : 0u), q4);
    SlabData data_c = slab_data(T, row_e + kbeg, q4, bits_c);
    build_lut<kGemmThreads>(len, lut, scratch);
    __syncthreads();
    f32x16 acc[kB][2];
#pragma unroll
    for (int tb = 0; tb < kB; ++tb) acc[tb][0] = acc[tb][1] = f32x16{};
    // 16-column steps of a slab that this wave multiplies: all, or its share
    // of the kWays waves that multiply its token blocks
    constexpr uint32_t kSteps = kSlabCols / 16 / kWays;
    const uint32_t ks0 = kSteps * (wave % kWays);
    // A steps fetched before the restore (the rest a few steps ahead during
    // the matrix instructions, where the registers are short)
    constexpr uint32_t kPre = kB == 2 ? 6 : kWays == 1 ? 5 : kWays == 2 ? kSteps / 2 : kSteps;
    for (uint32_t k0 = kbeg; k0 < kend; k0 += kSlabCols) {
        const bool has_n = k0 + kSlabCols < kend, has_nn = k0 + 2 * kSlabCols < kend;
        // Stage this slab's code words (loaded a slab ago; a segment longer
        // than the prefetched 32 words loads the rest now).
        put_seg4(seg, 4 * q4, data_c.w0);
        put_seg4(seg, 16 + 4 * q4, data_c.w1);
        for (uint32_t i = 32 + 4 * q4; i < data_c.nw; i += 16) put_seg4(seg, i, load_words4(T, data_c.wa + i));
        // Issue the next slabs' loads, then this slab's A operands.
        SlabData data_n = data_c;
        if (has_n) data_n = slab_data(T, row_e + k0 + kSlabCols, q4, bits_n);
        SlabBits bits_nn = bits_n;
        if (has_nn) bits_nn = slab_bits(T, row_e + k0 + 2 * kSlabCols, q4);
        bf16x8 xa[kSteps][kB];
        if (wave_mul) {
#pragma unroll
            for (uint32_t ks = 0; ks < kPre; ++ks)
#pragma unroll
                for (int tb = 0; tb < kB; ++tb) xa[ks][tb] = load_a(xa_p[tb] + k0 + 16 * (ks0 + ks), tok_ok[tb]);
        }
        wave_sync();
        uint32_t ex1[8], ex2[8];
        decode_groups(seg, seg_chain_r0(bit1(bits_c), data_c.wa), seg_chain_r0(bit2(bits_c), data_c.wa), lut, ex1,
                      ex2);
        wave_sync();  // the row's staged words have been read: its slab row may be written
        // Join and put both groups into the slab.
        const uint32_t b1[8] = {data_c.s1a.x, data_c.s1a.y, data_c.s1a.z, data_c.s1a.w,
                                data_c.s1b.x, data_c.s1b.y, data_c.s1b.z, data_c.s1b.w};
        const uint32_t b2[8] = {data_c.s2a.x, data_c.s2a.y, data_c.s2a.z, data_c.s2a.w,
                                data_c.s2b.x, data_c.s2b.y, data_c.s2b.z, data_c.s2b.w};
        uint4 *o1 = reinterpret_cast<uint4 *>(out_row + 64 * q4);
        uint4 *o2 = reinterpret_cast<uint4 *>(out_row + 64 * (q4 + 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 v1, v2;
            join4(b1[2 * j], ex1[2 * j], v1.x, v1.y);
            join4(b1[2 * j + 1], ex1[2 * j + 1], v1.z, v1.w);
            join4(b2[2 * j], ex2[2 * j], v2.x, v2.y);
            join4(b2[2 * j + 1], ex2[2 * j + 1], v2.z, v2.w);
            o1[j] = v1;
            o2[j] = v2;
        }
        __syncthreads();  // the slab is complete
        if (wave_mul) {
#pragma unroll
            for (uint32_t ks = 0; ks < kSteps; ++ks) {
                if (ks + kPre < kSteps) {
#pragma unroll
                    for (int tb = 0; tb < kB; ++tb)
                        xa[ks + kPre][tb] = load_a(xa_p[tb] + k0 + 16 * (ks0 + ks + kPre), tok_ok[tb]);
                }
                const uint32_t kb = 32 * (ks0 + ks);  // the step's byte offset in a slab row
                const bf16x8 w0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(b_row0 + kb));
                const bf16x8 w1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(b_row1 + kb));
#pragma unroll
                for (int tb = 0; tb < kB; ++tb) {
                    if (!blk_mul[tb]) continue;  // uniform: no token of this block is below m
                    acc[tb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[ks][tb], w0, acc[tb][0], 0, 0, 0);
                    acc[tb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[ks][tb], w1, acc[tb][1], 0, 0, 0);
                }
            }
        }
        __syncthreads();  // every wave is done with the slab and its staged words
        bits_c = bits_n;
        bits_n = bits_nn;
        data_c = data_n;
    }
    if constexpr (kWays > 1) {
        // The waves that share a token block add their partial sums in LDS
        // (the slab's space, free after the last barrier), so that one wave
        // per block adds into y: as many atomic adds as without the split.
        static_assert(kB == 1 && kGemmWaves * 2 * 16 * kWave * 4 <= sizeof(GemmLds::slab), "partial sums fit the slab");
        float *part = reinterpret_cast<float *>(slab) + wave * (2 * 16 * kWave);
        if (wave_mul && wave % kWays != 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                part[v * kWave + lane] = acc[0][0][v];
                part[(16 + v) * kWave + lane] = acc[0][1][v];
            }
        }
        __syncthreads();
        if (wave % kWays != 0) return;
#pragma unroll
        for (int w = 1; w < kWays; ++w) {
            const float *pw = part + w * (2 * 16 * kWave);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc[0][0][v] += pw[v * kWave + lane];
                acc[0][1][v] += pw[(16 + v) * kWave + lane];
            }
        }
    }
    if (!wave_mul) return;
    const uint32_t col = r0 + ((uint32_t)lane & 31);
#pragma unroll
    for (int tb = 0; tb < kB; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const uint32_t t = t_wave + 32 * tb + 8 * (v / 4) + 4 * ((uint32_t)lane >> 5) + (v & 3);
            if (t < m) {
                float *yr = J.y + (uint64_t)t * J.rows;
                atomicAdd(yr + col, acc[tb][0][v]);
                atomicAdd(yr + col + 32, acc[tb][1][v]);
            }
        }
}

}  // namespace

int check_gemm_job(const afx_gemv_job &j, uint32_t m) {
    int rc = check_info(j.info);
    if (rc != AFX_OK) return rc;
    if (!j.blob_dev || !j.x_dev || !j.y_dev || j.rows == 0 || j.cols == 0) return AFX_E_INVALID_ARG;
    if (j.rows * j.cols != j.info->n_elems || j.info->n_elems / j.cols != j.rows) return AFX_E_INVALID_ARG;
    if (m == 0 || m > 65535u * kGemmWaves * 32 * kMaxTokenBlocks) return AFX_E_UNSUPPORTED;
    if (j.rows % kTileRows || j.cols % kSlabCols || j.rows >= (1ull << 31) || j.cols >= (1ull << 31))
        return AFX_E_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(j.blob_dev) & 15) || (reinterpret_cast<uintptr_t>(j.x_dev) & 15) ||
        (reinterpret_cast<uintptr_t>(j.y_dev) & 3))
        return AFX_E_MISALIGNED;
    return AFX_OK;
}

namespace {

GemmJob gemm_job(const afx_gemv_job &j) {
    const afx_info *info = j.info;
    const uint8_t *b = static_cast<const uint8_t *>(j.blob_dev);
    GemmJob g{};
    g.t.code_len = b + info->off_code_len;
    g.t.chunk_base = reinterpret_cast<const uint64_t *>(b + info->off_chunk_base);
    g.t.gap = reinterpret_cast<const uint16_t *>(b + info->off_gap);
    g.t.signmant = b + info->off_signmant;
    g.t.exp = reinterpret_cast<const uint32_t *>(b + info->off_exp);
    g.t.out = nullptr;
    g.t.n = info->n_elems;
    g.t.exp_words = info->exp_words;
    g.t.last_word4 = (info->exp_words - 4) & ~(uint64_t)3;
    g.t.n_chunks = (uint32_t)info->n_chunks;
    g.x = j.x_dev;
    g.y = j.y_dev;
    g.rows = (uint32_t)j.rows;
    g.cols = (uint32_t)j.cols;
    g.n_rtiles = (uint32_t)(j.rows / kTileRows);
    return g;
}

int launch_gemm(const afx_gemv_job *jobs, size_t n_jobs, uint32_t m, hipStream_t stream) {
    GemmBatch batch{};
    batch.m = m;
    uint64_t tiles = 0;
    const uint32_t rc = m > kGemmWaves * 32 ? range_cols<2>() : range_cols<1>();  // as the kernel launched below
    for (size_t i = 0; i < n_jobs; ++i) {
        GemmJob g = gemm_job(jobs[i]);
        g.tile0 = (uint32_t)tiles;
        tiles += (uint64_t)g.n_rtiles * ((g.cols + rc - 1) / rc);
        batch.j[batch.n++] = g;
    }
    if (tiles == 0) return AFX_OK;
    if (tiles >= (1ull << 31)) return AFX_E_UNSUPPORTED;
    // one block of 32 tokens shared by the four waves while it covers m, two
    // blocks shared by two waves each while they do, one block per wave while
    // 128 tokens cover m, else two per wave
    const uint32_t per_wg = m <= 32 ? 32 : m <= 64 ? 64 : m <= kGemmWaves * 32 ? kGemmWaves * 32 : kGemmWaves * 64;
    const uint32_t tok_blocks = (m + per_wg - 1) / per_wg;
    // with several token blocks, the tiles padded to a multiple of 8 (see the kernel)
    const uint64_t blocks = gemm_blocks(tiles, tok_blocks);
    if (blocks >= (1ull << 31)) return AFX_E_UNSUPPORTED;
    batch.tiles = (uint32_t)tiles;
    batch.n_tok = tok_blocks;
    void *args[] = {&batch};  // hipLaunchKernel reports this launch's own status
    const void *fn = m <= 32   ? reinterpret_cast<const void *>(&afx_gemm_kernel<1, 4>)
                     : m <= 64 ? reinterpret_cast<const void *>(&afx_gemm_kernel<1, 2>)
                     : m <= kGemmWaves * 32 ? reinterpret_cast<const void *>(&afx_gemm_kernel<1, 1>)
                                            : reinterpret_cast<const void *>(&afx_gemm_kernel<2, 1>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kGemmThreads), args, 0, stream) == hipSuccess
               ? AFX_OK
               : AFX_E_HIP;
}

}  // namespace
}  // namespace afx

using namespace afx;

extern "C" {

int afx_restore_gemm_batch_async(const afx_gemv_job *jobs, size_t n_jobs, uint32_t m, void *stream) {
    if (!jobs && n_jobs) return AFX_E_INVALID_ARG;
    for (size_t i = 0; i < n_jobs; ++i) {
        const int rc = check_gemm_job(jobs[i], m);
        if (rc != AFX_OK) return rc;
    }
    if (fused_outputs_overlap_inputs(jobs, n_jobs, m)) return AFX_E_INVALID_ARG;
    // For 1, 2 or 4 tokens the matrix-vector kernel computes the same y on
    // the vector ALUs faster (it accepts every job this one does).
    if (m == 1 || m == 2 || m == 4) return afx_restore_gemv_batch_async(jobs, n_jobs, m, stream);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (size_t i = 0; i < n_jobs; i += AFX_MAX_GEMV_JOBS_PER_LAUNCH) {
        const size_t k = std::min<size_t>(AFX_MAX_GEMV_JOBS_PER_LAUNCH, n_jobs - i);
        const int rc = launch_gemm(jobs + i, k, m, s);
        if (rc != AFX_OK) return rc;
    }
    return AFX_OK;
}

int afx_restore_gemm_async(const afx_info *info, const void *blob_dev, uint64_t rows, uint64_t cols,
                           const uint16_t *x_dev, uint32_t m, float *y_dev, void *stream) {
    const afx_gemv_job job{info, blob_dev, rows, cols, x_dev, y_dev};
    return afx_restore_gemm_batch_async(&job, 1, m, stream);
}

}  // extern "C"
