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
//   * the batch's chunks (4096 elements each) are numbered globally; each
//     workgroup (4 wave64s) takes one contiguous range of chunks;
//   * for every tensor its range touches, the workgroup builds the 4096-entry
//     decode table (u16: length << 8 | symbol) of that tensor's canonical code
//     in LDS, from the 256 code lengths alone;
//   * each wave restores one chunk at a time: it stages the chunk's code words
//     in its own LDS slice with 16-byte loads; lane j then decodes groups j and
//     j + 64 (32 symbols each, two independent dependency chains) from a 64-bit
//     MSB-aligned bit buffer, peeking 12 bits per symbol into the table and
//     topping the buffer up with one prefetched word after every two symbols;
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
constexpr int kWavesPerBlock = 4;
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
    uint64_t first_chunk;  // index of this tensor's chunk 0 in the launch
};

struct Batch {
    TensorDesc t[AFX_MAX_JOBS_PER_LAUNCH];
    uint32_t n_tensors;
    uint32_t reserved;
    uint64_t total_chunks;
};

struct LutScratch {
    uint32_t wave_count[kWavesPerBlock][kMaxLen + 1];
    uint32_t limit[kMaxLen + 1];  // end of each length's slice of the 12-bit index space
    uint32_t first[kMaxLen + 1];  // first canonical code of each length
    uint32_t start[kMaxLen + 1];  // position of that length's first symbol in `sorted`
    uint8_t sorted[256];          // used symbols in (length, value) order
};

// Per-wave LDS: the chunk's code words while decoding, then its decoded
// exponent bytes (4 KB) while storing. A chunk spans at most 4096 * 12 bits;
// add the alignment slack of the start and the over-read of the last group.
constexpr uint32_t kStageWords = 1568;

// Order LDS traffic between lanes of one wave (no workgroup barrier needed).
__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Build the decode table of one canonical code: entry i (a 12-bit window of
// the stream, MSB first) holds (length << 8) | symbol of the code word that
// starts the window. All 256 threads take part; thread s owns symbol s, then
// table entries [16 s, 16 s + 16). Callers bracket it with barriers.
__device__ void build_lut(const uint8_t *__restrict__ code_len, uint16_t *lut, LutScratch &S) {
    const int s = threadIdx.x;
    const int lane = s & (kWave - 1), wave = s / kWave;
    uint32_t len = code_len[s];
    if (len > kMaxLen) len = 0;  // only a corrupt blob gets here; treat as unused

    uint32_t rank = 0;  // among same-length symbols of this wave with smaller value
#pragma unroll
    for (uint32_t l = 1; l <= kMaxLen; ++l) {
        const uint64_t m = __ballot(len == l);
        if (len == l) rank = (uint32_t)__popcll(m & ((1ull << lane) - 1));
        if (lane == 0) S.wave_count[wave][l] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    if (s == 0) {
        uint32_t code = 0, pos = 0;
        for (uint32_t l = 1; l <= kMaxLen; ++l) {
            uint32_t cnt = 0;
            for (int w = 0; w < kWavesPerBlock; ++w) cnt += S.wave_count[w][l];
            S.first[l] = code;
            S.start[l] = pos;
            S.limit[l] = (code + cnt) << (kMaxLen - l);
            pos += cnt;
            code = (code + cnt) << 1;
        }
    }
    __syncthreads();
    if (len) {
        uint32_t before = 0;
        for (int w = 0; w < wave; ++w) before += S.wave_count[w][len];
        S.sorted[(S.start[len] + before + rank) & 255] = (uint8_t)s;
    }
    __syncthreads();

    // An entry's length is one more than the number of length slices that
    // end at or before it; its symbol follows from the code's distance to
    // that length's first code.
    auto entry = [&](uint32_t idx) -> uint32_t {
        uint32_t l = 1;
#pragma unroll
        for (uint32_t k = 1; k < kMaxLen; ++k) l += idx >= S.limit[k] ? 1u : 0u;
        const uint32_t j = S.start[l] + ((idx >> (kMaxLen - l)) - S.first[l]);
        return (l << 8) | S.sorted[j & 255];
    };
    const uint32_t i0 = (uint32_t)s * 16;
    const uint32_t e0 = entry(i0);
    uint32_t v[8];
    if ((e0 >> 8) <= 8) {
        // codes of <= 8 bits own whole 16-aligned blocks of the index space
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = e0 | (e0 << 16);
    } else {
#pragma unroll 1
        for (int j = 0; j < 8; ++j) v[j] = entry(i0 + 2 * j) | (entry(i0 + 2 * j + 1) << 16);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(lut + i0);
    dst[0] = make_uint4(v[0], v[1], v[2], v[3]);
    dst[1] = make_uint4(v[4], v[5], v[6], v[7]);
}

// Two BF16 values from their sign/mantissa bytes and exponent bytes, each
// pair given as 16-bit lanes of a dword (element 0 in the low half).
__device__ inline uint32_t join_pair(uint32_t b2, uint32_t e2) {
    return (b2 & 0x007F007Fu) | (e2 << 7) | ((b2 & 0x00800080u) << 8);
}

// Bytes 0,1 (lo) or 2,3 (hi) of x moved into the two 16-bit halves.
__device__ inline uint32_t spread_lo(uint32_t x) { return __builtin_amdgcn_perm(0u, x, 0x0c010c00u); }
__device__ inline uint32_t spread_hi(uint32_t x) { return __builtin_amdgcn_perm(0u, x, 0x0c030c02u); }

// Put the low byte of e into byte k of w.
template <int k>
__device__ inline uint32_t put_byte(uint32_t w, uint32_t e) {
    // selector bytes 4..7 pick w's bytes, 0 picks e's byte 0
    constexpr uint32_t keep = 0x07060504u;
    constexpr uint32_t sel = (keep & ~(0xFFu << (8 * k)));
    return __builtin_amdgcn_perm(w, e, sel);
}

// One decoding chain: a 64-bit MSB-aligned bit buffer over the staged words.
struct Chain {
    uint64_t buf;    // next stream bits, MSB first
    uint32_t avail;  // valid bits in buf (>= 32 at the start of every pair)
    uint32_t wi;     // staged word that `nxt` came from
    uint32_t nxt;    // that word, loaded ahead of need
};

__device__ inline uint32_t staged(const uint32_t *stage, uint32_t i) {
    return stage[min(i, kStageWords - 1)];
}

__device__ inline void chain_start(Chain &c, const uint32_t *stage, uint32_t bit) {
    const uint32_t w = bit >> 5, sh = bit & 31;
    const uint64_t v = ((uint64_t)staged(stage, w) << 32) | staged(stage, w + 1);
    c.buf = v << sh;
    c.avail = 64 - sh;
    c.wi = w + 2;
    c.nxt = staged(stage, c.wi);
}

__device__ inline uint32_t lookup(const uint16_t *lut, uint64_t buf) {
    return lut[(uint32_t)(buf >> (64 - kMaxLen))];
}

// Decode two symbols, then top the buffer up with one word when it holds
// fewer than 32 bits (two codes take at most 24).
template <int k>
__device__ inline void chain_pair(Chain &c, const uint32_t *stage, const uint16_t *lut, uint32_t &w) {
    const uint32_t e1 = lookup(lut, c.buf);
    const uint32_t l1 = e1 >> 8;
    c.buf <<= l1;
    const uint32_t e2 = lookup(lut, c.buf);
    const uint32_t l2 = e2 >> 8;
    c.buf <<= l2;
    w = put_byte<k + 1>(put_byte<k>(w, e1), e2);
    c.avail -= l1 + l2;
    const bool refill = c.avail < 32;
    const uint32_t word = refill ? c.nxt : 0u;
    c.buf |= (uint64_t)word << ((32 - c.avail) & 63);
    c.avail += refill ? 32u : 0u;
    c.wi += refill ? 1u : 0u;
    c.nxt = staged(stage, c.wi);
}

// One wave restores chunk `lc` of tensor T.
__device__ void decode_chunk(const TensorDesc &T, uint64_t lc, const uint16_t *lut, uint32_t *stage, int lane) {
    const uint64_t e0 = lc * kChunk;
    const uint32_t ne = (uint32_t)min<uint64_t>(kChunk, T.n - e0);
    const uint32_t ng = (ne + kGroup - 1) / kGroup;
    const uint64_t base = T.chunk_base[lc];
    const uint64_t end = T.chunk_base[lc + 1];
    const uint64_t w0 = (base >> 5) & ~(uint64_t)3;  // 16-byte aligned start
    // words to stage: through the chunk's last bit plus over-read slack;
    // the unsigned arithmetic saturates via min() on corrupt bases
    const uint64_t want = ((end + 31) >> 5) + 16 - w0;
    const uint32_t nwords = (uint32_t)min<uint64_t>(want, kStageWords);

    // sign/mantissa bytes of this lane's store slots, fetched early
    const uint8_t *sm = T.signmant + e0;
    const uint16_t *gap = T.gap + lc * kGroupsPerChunk;
    const uint32_t ga = (uint32_t)lane, gb = (uint32_t)lane + kWave;
    const uint32_t gap_a = ga < ng ? gap[ga] : 0u;
    const uint32_t gap_b = gb < ng ? gap[gb] : 0u;

    wave_sync();  // the previous chunk's reads of `stage` are done
    for (uint32_t i = 4 * (uint32_t)lane; i < nwords; i += 4 * kWave) {
        const uint64_t g = w0 + i;
        uint4 v;
        if (g + 4 <= T.exp_words) {
            v = *reinterpret_cast<const uint4 *>(T.exp + g);
        } else {
            v.x = g < T.exp_words ? T.exp[g] : 0u;
            v.y = g + 1 < T.exp_words ? T.exp[g + 1] : 0u;
            v.z = g + 2 < T.exp_words ? T.exp[g + 2] : 0u;
            v.w = g + 3 < T.exp_words ? T.exp[g + 3] : 0u;
        }
        *reinterpret_cast<uint4 *>(stage + i) = v;
    }
    wave_sync();

    const uint32_t rel = (uint32_t)(base - (w0 << 5));  // < 128
    Chain A, B;
    chain_start(A, stage, rel + gap_a);
    chain_start(B, stage, rel + gap_b);
    uint32_t wa[8], wb[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        wa[q] = 0;
        wb[q] = 0;
        chain_pair<0>(A, stage, lut, wa[q]);
        chain_pair<0>(B, stage, lut, wb[q]);
        chain_pair<2>(A, stage, lut, wa[q]);
        chain_pair<2>(B, stage, lut, wb[q]);
    }
    wave_sync();  // every lane is done reading the staged words
    uint4 *pa = reinterpret_cast<uint4 *>(stage + ga * 8);
    uint4 *pb = reinterpret_cast<uint4 *>(stage + gb * 8);
    pa[0] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
    pa[1] = make_uint4(wa[4], wa[5], wa[6], wa[7]);
    pb[0] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
    pb[1] = make_uint4(wb[4], wb[5], wb[6], wb[7]);
    wave_sync();

    // Store order: lane handles elements [r*512 + 8*lane, +8) for r = 0..7,
    // so each store instruction writes 1 KB of consecutive output.
    uint16_t *out = T.out + e0;
    const uint8_t *exb = reinterpret_cast<const uint8_t *>(stage);
#pragma unroll 2
    for (int r = 0; r < 8; ++r) {
        const uint32_t i = (uint32_t)r * (8 * kWave) + 8 * (uint32_t)lane;
        if (i + 8 <= ne) {
            const uint2 b = *reinterpret_cast<const uint2 *>(sm + i);
            const uint2 e = *reinterpret_cast<const uint2 *>(exb + i);
            uint4 o;
            o.x = join_pair(spread_lo(b.x), spread_lo(e.x));
            o.y = join_pair(spread_hi(b.x), spread_hi(e.x));
            o.z = join_pair(spread_lo(b.y), spread_lo(e.y));
            o.w = join_pair(spread_hi(b.y), spread_hi(e.y));
            *reinterpret_cast<uint4 *>(out + i) = o;
        } else {
            for (uint32_t j = i; j < ne && j < i + 8; ++j) {
                const uint32_t b = sm[j], e = exb[j];
                out[j] = (uint16_t)(((b & 0x80u) << 8) | (e << 7) | (b & 0x7Fu));
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void afx_decode_kernel(
    const Batch batch) {
    __shared__ uint16_t lut[kLutEntries];                     // 8 KB
    __shared__ uint32_t stage[kWavesPerBlock][kStageWords];   // 24.5 KB
    __shared__ LutScratch scratch;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint64_t total = batch.total_chunks;
    const uint64_t c_begin = total * blockIdx.x / gridDim.x;
    const uint64_t c_end = total * (blockIdx.x + 1) / gridDim.x;

    uint32_t ti = 0;
    uint64_t c = c_begin;
    while (c < c_end) {
        while (ti + 1 < batch.n_tensors && batch.t[ti + 1].first_chunk <= c) ++ti;
        const TensorDesc &T = batch.t[ti];
        const uint64_t seg_end = min(c_end, T.first_chunk + (T.n + kChunk - 1) / kChunk);
        __syncthreads();  // all waves are done with the previous table
        build_lut(T.code_len, lut, scratch);
        __syncthreads();
        for (uint64_t cc = c + (uint64_t)wave; cc < seg_end; cc += kWavesPerBlock)
            decode_chunk(T, cc - T.first_chunk, lut, stage[wave], lane);
        c = seg_end;
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

TensorDesc describe(const afx_job &j, uint64_t first_chunk) {
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
    d.first_chunk = first_chunk;
    return d;
}

// Enqueue one launch for up to AFX_MAX_JOBS_PER_LAUNCH already-checked jobs.
int launch(const afx_job *jobs, size_t n_jobs, hipStream_t stream) {
    Batch batch;
    batch.n_tensors = 0;
    batch.reserved = 0;
    uint64_t total = 0;
    for (size_t i = 0; i < n_jobs; ++i) {
        if (jobs[i].info->n_elems == 0) continue;
        batch.t[batch.n_tensors++] = describe(jobs[i], total);
        total += jobs[i].info->n_chunks;
    }
    batch.total_chunks = total;
    if (total == 0) return AFX_OK;
    int max_blocks = 0;
    int rc = max_blocks_for_current_device(&max_blocks);
    if (rc != AFX_OK) return rc;
    const uint64_t want = (total + kWavesPerBlock - 1) / kWavesPerBlock;
    const unsigned grid = (unsigned)std::min<uint64_t>(want, (uint64_t)max_blocks);
    hipLaunchKernelGGL(afx_decode_kernel, dim3(grid), dim3(kThreads), 0, stream, batch);
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
