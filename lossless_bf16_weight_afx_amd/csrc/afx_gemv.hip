// afx_gemv.hip -- the restore fused into its consumer (gfx950): y += W x for a
// weight matrix W held only in its coded form.
//
// "Why Weight Offloading Slows Inference" (section "Lossless compression")
// reconstructs a coded weight's bits ahead of the computation that uses it.
// Restoring into HBM and then multiplying writes the BF16 matrix (2 bytes per
// value) and reads it back; for the matrix-vector products of token-by-token
// generation, which read every weight once per token, that traffic is the
// cost. Here each wave restores a chunk exactly as afx_decode.hip does, up to
// the exponent bytes in LDS, and multiplies the restored values by the
// activations in registers: HBM sees the coded matrix (~1.39 bytes per value)
// and nothing else.
//
// W is row-major [rows, cols] (the blob's element order), x is BF16 [m, cols]
// and y is FP32 [m, rows], both row-major; m is 1, 2 or 4 (a handful of
// tokens). The products of two BF16 values are exact in FP32; sums are FP32:
// per lane over 8 consecutive values, two products at a time
// (v_dot2_f32_bf16, which on this hardware measures within one rounding per
// addition), then across the wave, then into y with atomic adds (in no fixed
// order).
//
// Work decomposition and decode as in the restore: one 16-wave workgroup per
// CU, chunks round the workgroups, claimed one at a time by the waves from an
// LDS counter, code words staged a chunk ahead, decoded through the pair
// table.
#include <hip/hip_runtime.h>

#include <atomic>
#include <numeric>

#include "afx_device.h"
#include "afx_split.h"

namespace afx {
namespace {

struct GemvArgs {
    TensorDesc t;       // t.blk_lo/blk_hi: the workgroups that serve this matrix
    const uint16_t *x;  // [m, cols] BF16
    float *y;           // [m, rows] FP32, accumulated into
    uint64_t rows;
    uint32_t cols;      // a multiple of 8 (every 8 consecutive values lie in one row), below 2^31
    // 0, or P when x is staged as a window of one chunk's columns per token:
    // the columns of chunk c start at (c kChunk) mod cols, which repeats with
    // period P = cols / gcd(cols, kChunk) in c, and every workgroup of this
    // matrix serves chunks of one residue mod P (its count is a multiple of P)
    uint32_t xwin;
};

constexpr uint32_t kMaxGemvJobs = AFX_MAX_GEMV_JOBS_PER_LAUNCH;

// Whether the kernel for M tokens can stage x as a window of one chunk's
// columns (for one token, x of rows up to 20,480 columns fits whole; the
// window path stays out of that kernel, whose instruction count is its bound).
template <int M>
constexpr bool kWindowed = M >= 2;

struct GemvBatch {
    GemvArgs j[kMaxGemvJobs];
    uint32_t n;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Word 3 of a raw buffer resource on this architecture: 32-bit data format,
// byte offsets, range-checked against the record count.
constexpr int kBufferFlags = 0x00020000;
__device__ inline bf16x2 bf16_pair(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// Sum over the wave with DPP moves (no LDS); the total lands in lane 63.
template <int kCtrl, int kRowMask = 0xF>
__device__ inline float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}
__device__ inline float wave_sum_to_lane63(float v) {
    v = dpp_add<0xB1>(v);         // quad_perm [1,0,3,2]: pairs
    v = dpp_add<0x4E>(v);         // quad_perm [2,3,0,1]: quads
    v = dpp_add<0x141>(v);        // row_half_mirror: 8 lanes
    v = dpp_add<0x140>(v);        // row_mirror: rows of 16
    v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// Activations of one matrix staged in LDS when they fit (m * cols BF16).
constexpr uint32_t kXStageBytes = 40 * 1024;  // 4 tokens of 5120 values, one of 17408

// Request chunk lc's sign/mantissa bytes in store order (lane: bytes
// [r*512 + 8*lane, +8) for r = 0..7); read once, not kept in the caches.
__device__ inline void load_signmant(const TensorDesc &T, uint64_t lc, int lane, uint2 (&smv)[8]) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const uint64_t e0 = lc * kChunk;
    const uint32_t ne = (uint32_t)umin64(kChunk, T.n - e0);
    const uint8_t *sm = T.signmant + e0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t i = (uint32_t)r * (8 * kWave) + 8 * (uint32_t)lane;
        const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(sm + (i + 8 <= ne ? i : 0)));
        smv[r] = make_uint2(t.x, t.y);  // tail elements are reread below
    }
}

// x's 8 values at columns col..col+7 of each token row. The staged copy is
// read with an LDS load and x in L2 with a buffer load: as two plain loads,
// the compiler merges them into one generic (flat) load of a selected
// pointer, which waits on both memory counters.
template <int M>
__device__ inline void load_x(const GemvArgs &a, const uint16_t *xs, bool x_in_lds,
                              const __amdgpu_buffer_rsrc_t (&xrow)[M], uint32_t col, uint4 (&xv)[M],
                              uint32_t xs_stride, uint32_t xs_col) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (x_in_lds) {
            xv[m] = *reinterpret_cast<const uint4 *>(xs + (uint32_t)m * xs_stride + xs_col);
        } else {
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(xrow[m], 2 * col, 0, 0);
            xv[m] = make_uint4(t.x, t.y, t.z, t.w);
        }
    }
}

// Add the products of the lane's 8 values of one round (elements i..i+7 of
// the chunk, columns col..col+7 of one row) with x (xv: those columns of
// each token row) into acc[m], token m.
template <int M>
__device__ inline void round_products(const GemvArgs &a, const uint4 (&xv)[M], uint2 b, const uint8_t *exb,
                                      const uint8_t *sm, uint32_t i, uint32_t ne, uint32_t col, float (&acc)[M]) {
    if (i + 8 <= ne) {
        const uint2 e = *reinterpret_cast<const uint2 *>(exb + i);
        // restored values as BF16 pairs (element 2q in the low half),
        // multiplied two at a time against x's pairs
        uint32_t p01, p23, p45, p67;
        join4(b.x, e.x, p01, p23);
        join4(b.y, e.y, p45, p67);
        const bf16x2 w01 = bf16_pair(p01), w23 = bf16_pair(p23), w45 = bf16_pair(p45), w67 = bf16_pair(p67);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float s = __builtin_amdgcn_fdot2_f32_bf16(w01, bf16_pair(xv[m].x), acc[m], false);
            s = __builtin_amdgcn_fdot2_f32_bf16(w23, bf16_pair(xv[m].y), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(w45, bf16_pair(xv[m].z), s, false);
            acc[m] = __builtin_amdgcn_fdot2_f32_bf16(w67, bf16_pair(xv[m].w), s, false);
        }
    } else {  // the matrix's last, partial round
        for (uint32_t j = i; j < ne && j < i + 8; ++j) {
            const uint32_t bb = sm[j], ee = exb[j];
            const float w = __uint_as_float((((bb & 0x80u) << 8) | (ee << 7) | (bb & 0x7Fu)) << 16);
#pragma unroll
            for (int m = 0; m < M; ++m)
                acc[m] = fmaf(w, __uint_as_float((uint32_t)a.x[(uint64_t)m * a.cols + col + (j - i)] << 16), acc[m]);
        }
    }
}

// The eight rounds of a chunk whose rows are a chunk or longer: each lane's
// rounds lie in one row until its columns wrap, then in the next; the
// products go into a0 (first row) or a1 (second), per token. x is requested
// kBatch rounds at a time.
template <int M, int kBatch, bool kWin>
__device__ inline void long_rounds(const GemvArgs &a, const uint16_t *xs, bool x_in_lds,
                                   const __amdgpu_buffer_rsrc_t (&xrow)[M], const uint2 (&smv)[8],
                                   const uint8_t *exb, const uint8_t *sm, uint32_t ne, uint32_t c0, int lane,
                                   float (&a0)[M], float (&a1)[M]) {
#pragma unroll
    for (int r0 = 0; r0 < 8; r0 += kBatch) {
        uint4 xv[kBatch][M];
        uint32_t col[kBatch];
        bool next_row[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const uint32_t i = (uint32_t)(r0 + q) * (8 * kWave) + 8 * (uint32_t)lane;
            const uint32_t c = c0 + i;
            next_row[q] = c >= a.cols;
            col[q] = next_row[q] ? c - a.cols : c;
            // a window holds the chunk's columns in chunk order
            load_x<M>(a, xs, x_in_lds, xrow, col[q], xv[q], kWin ? kChunk : a.cols, kWin ? i : col[q]);
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const uint32_t i = (uint32_t)(r0 + q) * (8 * kWave) + 8 * (uint32_t)lane;
            float t[M];
#pragma unroll
            for (int m = 0; m < M; ++m) t[m] = next_row[q] ? a1[m] : a0[m];
            round_products<M>(a, xv[q], smv[r0 + q], exb, sm, i, ne, col[q], t);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                a0[m] = next_row[q] ? a0[m] : t[m];
                a1[m] = next_row[q] ? t[m] : a1[m];
            }
        }
    }
}

// Restore chunk lc of W and add its products with x into y. smv holds (or
// is receiving) chunk lc's sign/mantissa bytes on entry; as soon as they
// have been used, the bytes of chunk next_lc (if any) are requested into it,
// so that their latency overlaps the rest of this chunk and the next decode.
template <int M, bool kLong>
__device__ inline void gemv_chunk(const GemvArgs &a, const uint16_t *xs, bool x_in_lds, bool x_win, uint64_t lc, uint2 (&smv)[8],
                                  bool has_next, uint64_t next_lc, const ChunkGeom &g, const Gaps &gaps,
                                  const uint32_t *plut, uint32_t *stage, int lane, uint64_t later_bases,
                                  ChunkGeom &later) {
    const TensorDesc &T = a.t;
    const uint64_t e0 = lc * kChunk;
    const uint32_t ne = (uint32_t)umin64(kChunk, T.n - e0);
    const uint8_t *sm = T.signmant + e0;
    decode_exponents(g, gaps, plut, stage, lane);
    asm volatile("" : "+v"(later_bases));  // not before the decode above
    later = geom_from_lanes(later_bases);

    // The chunk starts in row row0 at column c0; lane handles values
    // [r*512 + 8*lane, +8) for r = 0..7, which lie in one row.
    const uint64_t row0 = e0 / a.cols;
    const uint32_t c0 = (uint32_t)(e0 - row0 * a.cols);
    const uint8_t *exb = reinterpret_cast<const uint8_t *>(stage);
    __amdgpu_buffer_rsrc_t xrow[M];  // row m of x (cols * 2 < 2^32 bytes)
#pragma unroll
    for (int m = 0; m < M; ++m)
        xrow[m] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.x + (uint64_t)m * a.cols), (short)0,
                                                    (int)(2 * a.cols), kBufferFlags);
    if constexpr (kLong) {  // cols >= kChunk
        // The chunk spans at most two rows: each lane's rounds lie in row
        // row0 until its columns wrap, then in row0 + 1. The products go
        // straight into one accumulator per row and token.
        float a0[M], a1[M];
#pragma unroll
        for (int m = 0; m < M; ++m) a0[m] = a1[m] = 0.f;
        // x in L2: request x of several rounds together (16 registers),
        // so that the reads wait once per batch rather than once per round.
        // x staged in LDS: one round at a time (batched, the LDS reads
        // conflicted more).
        if (kWindowed<M> && x_win)
            long_rounds<M, 1, true>(a, xs, true, xrow, smv, exb, sm, ne, c0, lane, a0, a1);
        else if (x_in_lds)
            long_rounds<M, 1, false>(a, xs, true, xrow, smv, exb, sm, ne, c0, lane, a0, a1);
        else
            long_rounds<M, (M >= 4 ? 1 : 4 / M), false>(a, xs, false, xrow, smv, exb, sm, ne, c0, lane, a0, a1);
        if (has_next) load_signmant(T, next_lc, lane, smv);
        // Sum each row's products over the wave and add them into y.
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float s = wave_sum_to_lane63(a0[m]);
            if (lane == kWave - 1) atomicAdd(a.y + (uint64_t)m * a.rows + row0, s);
        }
        if (c0 + ne > a.cols) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float s = wave_sum_to_lane63(a1[m]);
                if (lane == kWave - 1) atomicAdd(a.y + (uint64_t)m * a.rows + row0 + 1, s);
            }
        }
        return;
    }
    // Any row length: keep each round's products apart and sum them per
    // row at the end.
    float acc[8][M];
    uint32_t drow[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t i = (uint32_t)r * (8 * kWave) + 8 * (uint32_t)lane;
        uint32_t col = c0 + i;
        const uint32_t d = a.cols >= kChunk ? (col >= a.cols ? 1u : 0u) : col / a.cols;
        col -= d * a.cols;
        drow[r] = d;
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
        uint4 xv[M];
        load_x<M>(a, xs, x_in_lds, xrow, col, xv, a.cols, col);
        round_products<M>(a, xv, smv[r], exb, sm, i, ne, col, acc[r]);
    }
    if (has_next) load_signmant(T, next_lc, lane, smv);
    // Sum each row's products over the wave and add them into y.
    const uint32_t nrows = (c0 + ne - 1) / a.cols + 1;
    for (uint32_t d = 0; d < nrows; ++d) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float s = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r) s += drow[r] == d ? acc[r][m] : 0.f;
            s = wave_sum_to_lane63(s);
            if (lane == kWave - 1) atomicAdd(a.y + (uint64_t)m * a.rows + row0 + d, s);
        }
    }
}

// The workgroup's LDS as one object, the decode table first: at LDS address
// 0 a table read needs no base added to its index (the base of a table
// placed higher does not fit the read instruction's 16-bit offset).
struct GemvLds {
    uint32_t plut[kLutEntries];                   // 16 KB
    uint32_t stage[kWavesPerBlock][kStageRow];    // 98 KB
    uint16_t xs[kXStageBytes / 2];                // 40 KB
    LutScratch scratch;
    uint32_t next_j;  // the workgroup's next unclaimed chunk of the matrix
};

// kLong: every matrix of the batch has rows of a chunk or longer (cols >=
// 4096), so a chunk spans at most two rows and the products need only two
// accumulators per token (the general kernel keeps one per round and spills
// registers at m = 4).
template <int M, bool kLong>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void afx_gemv_kernel(const GemvBatch batch) {
    __shared__ __attribute__((aligned(16))) GemvLds lds;
    uint32_t *plut = lds.plut;
    auto &stage = lds.stage;
    LutScratch &scratch = lds.scratch;
    uint32_t &next_j = lds.next_j;
    uint16_t *xs = lds.xs;

    int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t b = blockIdx.x;
    uint32_t *my_stage = stage[wave];
    for (uint32_t t = 0; t < batch.n; ++t) {
        const GemvArgs &a = batch.j[t];
        const TensorDesc &T = a.t;
        // Workgroups [blk_lo, blk_hi) serve this matrix; the one of rank k of
        // nb (ranks counted XCD by XCD) takes chunks k + j nb; wave w starts with j = w and j = w + 16, then
        // claims the next unclaimed j.
        if (b < T.blk_lo || b >= T.blk_hi) continue;
        const uint32_t nb = T.blk_hi - T.blk_lo, k = xcd_rank(b - T.blk_lo, nb);
        if (k >= T.n_chunks) continue;
        const uint32_t mine = (T.n_chunks - k + nb - 1) / nb;
        uint32_t jc = wave, jn = wave + kWavesPerBlock;
        const bool has_c = jc < mine;
        bool has_n = jn < mine;
        // Every thread loads a code length (threads past 255 repeat some), so
        // that no branch around the load makes the compiler wait for it
        // before the bases below are requested; only waves 0-3 pass theirs on.
        const uint32_t len_any = T.code_len[threadIdx.x & 255];
        // Unconditional loads (of chunk k, which exists, for a wave without
        // such a chunk): around a branch, the compiler's wait at the join
        // would hold the bases back until the code lengths arrive.
        const uint64_t lc_c = k + (uint64_t)(has_c ? jc : 0u) * nb;
        const uint64_t lc_n = k + (uint64_t)(has_n ? jn : 0u) * nb;
        uint64_t bases_c = load_bases(T, lc_c, lane);
        uint64_t bases_n = load_bases(T, lc_n, lane);
        Gaps gaps = load_gaps(T, lc_c, lane);
        ChunkGeom g{};
        StreamRegs s;
        if (has_c) {
            g = geom_from_lanes(bases_c);
            load_stream(T, g, lane, s);
        }
        __syncthreads();  // every wave is done with the previous table, counter and activations
        if (threadIdx.x == 0) next_j = 2 * kWavesPerBlock;
        // stage the activations (read by every chunk) when they fit
        const uint64_t xbytes = (uint64_t)M * a.cols * 2;
        const bool x_win = kLong && kWindowed<M> && a.xwin != 0;
        const bool x_in_lds = xbytes <= kXStageBytes || x_win;
        if (x_win) {
            // the columns of this workgroup's chunks: (s + j) mod cols, j < kChunk
            // (s and cols are multiples of 8, so no 8 values straddle the wrap)
            const uint32_t s = (uint32_t)((uint64_t)(k % a.xwin) * kChunk % a.cols);
            for (uint32_t i = threadIdx.x; i < M * (kChunk / 8); i += kThreads) {
                const uint32_t m = i / (kChunk / 8), j = 8 * (i % (kChunk / 8));
                const uint32_t c = s + j >= a.cols ? s + j - a.cols : s + j;
                reinterpret_cast<uint4 *>(xs)[i] = *reinterpret_cast<const uint4 *>(a.x + (uint64_t)m * a.cols + c);
            }
        } else if (x_in_lds) {
            for (uint32_t i = threadIdx.x; i < xbytes / 16; i += kThreads)
                reinterpret_cast<uint4 *>(xs)[i] = reinterpret_cast<const uint4 *>(a.x)[i];
        }
        build_lut<kThreads, true>(wave < kSymbolWaves ? len_any : 0u, plut, scratch);
        __syncthreads();  // the pair table is complete
        if (!has_c) continue;
        uint2 smv[8];
        load_signmant(T, k + (uint64_t)jc * nb, lane, smv);
        put_stream(T, g, s, my_stage, lane);
        wave_sync();
        ChunkGeom gn = geom_from_lanes(bases_n);
        while (true) {
            asm volatile("" : "+v"(lane));
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
            gemv_chunk<M, kLong>(a, xs, x_in_lds, x_win, k + (uint64_t)jc * nb, smv, has_n, k + (uint64_t)jn * nb, g, gaps, plut, my_stage,
                          lane, bases_nn, gnn);
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

template <int M, bool kLong>
int gemv_max_blocks(int *out) {
    static std::atomic<int> blocks[64];  // per device, for this kernel
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return AFX_E_HIP;
    if (dev < 0 || dev >= 64) return AFX_E_UNSUPPORTED;
    int v = blocks[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return AFX_E_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, afx_gemv_kernel<M, kLong>, kThreads, 0) !=
            hipSuccess)
            return AFX_E_HIP;
        v = std::max(1, cus) * std::max(1, per_cu);
        blocks[dev].store(v, std::memory_order_relaxed);
    }
    *out = v;
    return AFX_OK;
}

// One launch for up to kMaxGemvJobs checked matrices (each of at least one
// chunk): the grid is split among them by their chunk counts with the
// restore's split (afx_split.h), every matrix counted as large.
template <int M, bool kLong>
int launch_gemv_kernel(GemvBatch &batch, hipStream_t stream) {
    uint64_t chunks[kMaxGemvJobs];
    uint32_t lo[kMaxGemvJobs], hi[kMaxGemvJobs];
    for (uint32_t t = 0; t < batch.n; ++t) chunks[t] = batch.j[t].t.n_chunks;
    if (batch.n == 0) return AFX_OK;
    int max_blocks = 0;
    const int rc = gemv_max_blocks<M, kLong>(&max_blocks);
    if (rc != AFX_OK) return rc;
    const uint32_t grid = split_grid(chunks, batch.n, batch.n, (uint32_t)max_blocks, lo, hi);
    const uint64_t busiest = split_max_load(chunks, batch.n, grid, lo, hi);  // 0: not computed
    for (uint32_t t = 0; t < batch.n; ++t) {
        GemvArgs &a = batch.j[t];
        // When x is too large to stage whole but one chunk's columns of it
        // fit, stage those: every workgroup's chunks then need the same
        // columns if the matrix's workgroup count is a multiple of their
        // period, so trim the range to one when that loads no workgroup more
        // than the busiest of the launch (the trimmed ones skip the matrix).
        a.xwin = 0;
        const uint32_t period = a.cols / std::gcd(a.cols, kChunk);
        const uint32_t nb = hi[t] - lo[t], nbw = nb / period * period;
        if (kLong && kWindowed<M> && busiest && (uint64_t)M * a.cols * 2 > kXStageBytes && M * kChunk * 2 <= kXStageBytes &&
            nbw > 0 && (chunks[t] + nbw - 1) / nbw <= busiest) {
            hi[t] = lo[t] + nbw;
            a.xwin = period;
        }
        a.t.blk_lo = lo[t];
        a.t.blk_hi = hi[t];
    }
    void *args[] = {&batch};  // hipLaunchKernel reports this launch's own status
    return hipLaunchKernel(reinterpret_cast<const void *>(&afx_gemv_kernel<M, kLong>), dim3((unsigned)grid),
                           dim3(kThreads), args, 0, stream) == hipSuccess
               ? AFX_OK
               : AFX_E_HIP;
}

template <int M>
int launch_gemv(GemvBatch &batch, hipStream_t stream) {
    bool all_long = true;
    for (uint32_t t = 0; t < batch.n; ++t) all_long &= batch.j[t].cols >= kChunk;
    return all_long ? launch_gemv_kernel<M, true>(batch, stream) : launch_gemv_kernel<M, false>(batch, stream);
}

int check_gemv_job(const afx_gemv_job &j, uint32_t m) {
    int rc = check_info(j.info);
    if (rc != AFX_OK) return rc;
    const afx_info *info = j.info;
    if (j.cols == 0 || info->n_elems % j.cols || info->n_elems / j.cols != j.rows) return AFX_E_INVALID_ARG;
    if (info->n_elems == 0) return AFX_OK;  // nothing to add
    if (!j.blob_dev) return AFX_E_INVALID_ARG;
    if (j.cols % 8 || j.cols >= (1ull << 31)) return AFX_E_UNSUPPORTED;  // x rows are read by byte offset
    if (m != 1 && m != 2 && m != 4) return AFX_E_UNSUPPORTED;
    if (!j.x_dev || !j.y_dev) return AFX_E_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(j.blob_dev) | reinterpret_cast<uintptr_t>(j.x_dev)) & 15) return AFX_E_MISALIGNED;
    if (reinterpret_cast<uintptr_t>(j.y_dev) & 3) return AFX_E_MISALIGNED;
    return AFX_OK;
}

GemvArgs gemv_args(const afx_gemv_job &j) {
    const afx_info *info = j.info;
    const uint8_t *b = static_cast<const uint8_t *>(j.blob_dev);
    GemvArgs a;
    a.t.code_len = b + info->off_code_len;
    a.t.chunk_base = reinterpret_cast<const uint64_t *>(b + info->off_chunk_base);
    a.t.gap = reinterpret_cast<const uint16_t *>(b + info->off_gap);
    a.t.signmant = b + info->off_signmant;
    a.t.exp = reinterpret_cast<const uint32_t *>(b + info->off_exp);
    a.t.out = nullptr;
    a.t.n = info->n_elems;
    a.t.exp_words = info->exp_words;
    a.t.last_word4 = (info->exp_words - 4) & ~(uint64_t)3;
    a.t.n_chunks = (uint32_t)info->n_chunks;
    a.t.blk_lo = a.t.blk_hi = a.t.reserved = 0;
    a.x = j.x_dev;
    a.y = j.y_dev;
    a.rows = j.rows;
    a.cols = (uint32_t)j.cols;
    a.xwin = 0;
    return a;
}

}  // namespace
}  // namespace afx

using namespace afx;

extern "C" int afx_restore_gemv_batch_async(const afx_gemv_job *jobs, size_t n_jobs, uint32_t m, void *stream) {
    if (!jobs && n_jobs) return AFX_E_INVALID_ARG;
    for (size_t i = 0; i < n_jobs; ++i) {
        const int rc = check_gemv_job(jobs[i], m);
        if (rc != AFX_OK) return rc;
    }
    if (fused_outputs_overlap_inputs(jobs, n_jobs, m)) return AFX_E_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (size_t i = 0; i < n_jobs;) {
        GemvBatch batch;
        batch.n = 0;
        for (; i < n_jobs && batch.n < kMaxGemvJobs; ++i)
            if (jobs[i].info->n_elems) batch.j[batch.n++] = gemv_args(jobs[i]);
        int rc = AFX_OK;
        switch (m) {
            case 1: rc = launch_gemv<1>(batch, s); break;
            case 2: rc = launch_gemv<2>(batch, s); break;
            default: rc = launch_gemv<4>(batch, s); break;
        }
        if (rc != AFX_OK) return rc;
    }
    return AFX_OK;
}

extern "C" int afx_restore_gemv_async(const afx_info *info, const void *blob_dev, uint64_t rows, uint64_t cols,
                                      const uint16_t *x_dev, uint32_t m, float *y_dev, void *stream) {
    const afx_gemv_job job{info, blob_dev, rows, cols, x_dev, y_dev};
    return afx_restore_gemv_batch_async(&job, 1, m, stream);
}
