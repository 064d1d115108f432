// afx_decode.hip -- the GPU restore of losslessly coded BF16 weights (gfx950).
//
// "Why Weight Offloading Slows Inference" (section "Three steps for each
// weight", Eq. (1)) names the unpack time t_unpack that every compressed
// weight pays before use; section "Lossless compression" entropy-codes the
// BF16 exponent field, so the unpack reconstructs each weight's exact bits.
// Here that unpack runs on the GPU after the compressed bytes reach device
// memory.
//
// Work decomposition (one launch per batch of up to 32 tensors):
//   * one workgroup of 16 wave64s fills a CU (4 waves per SIMD). The grid
//     is split among the batch's tensors by their chunk (4096-element)
//     counts (afx_split.h), so a workgroup serves about one tensor; within
//     a tensor the chunks go round its workgroups, so that all of them move
//     through each array together, in one narrow band;
//   * the waves of a workgroup claim its chunks one at a time from a counter
//     in LDS. A SIMD issues for its oldest waves first, so waves run at
//     different speeds; claiming keeps them finishing together;
//   * for every tensor it serves, the workgroup builds the 4096-entry decode
//     table (u16: symbol << 8 | length) of that tensor's canonical code in
//     LDS, from the 256 code lengths alone, and from it the pair table (u32:
//     both codes that start a 12-bit window when both fit in it);
//   * each wave restores one chunk at a time, software-pipelined: while chunk
//     i decodes, the code words and gap offsets of chunk i + 1 and the bit
//     bases of chunk i + 2 are in flight. The code words are staged in the
//     wave's own LDS slice; lane j then decodes groups j and j + 64 (32
//     symbols each, two independent dependency chains), two symbols per
//     32-bit window of the staged stream, mostly with one pair-table read;
//   * decoded exponent bytes go back to the wave's LDS slice in element order;
//     the wave re-reads them in store order, merges them with the
//     sign/mantissa bytes and writes 16-byte stores, 1 KB per instruction.
// There is no floating point and no matrix work: the kernel is bound by HBM
// bytes, and its first and last chunks by the serial table-lookup chain of
// each lane.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "afx_device.h"
#include "afx_split.h"

namespace afx {
namespace {

struct Batch {
    TensorDesc t[AFX_MAX_JOBS_PER_LAUNCH];
    uint32_t n_tensors;
};

// Restore one chunk: decode the staged code words, merge with the
// sign/mantissa bytes, store. `stage` holds the chunk's code words on entry
// and is free (but for the exponent bytes just written) on exit.
__device__ inline void restore_chunk(const TensorDesc &T, uint64_t lc, const ChunkGeom &g, const Gaps &gaps,
                                     const uint32_t *plut, uint32_t *stage, int lane, uint64_t later_bases,
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

    decode_exponents(g, gaps, plut, stage, lane);
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
            join4(b.x, e.x, o.x, o.y);
            join4(b.y, e.y, o.z, o.w);
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
    // The workgroup's LDS as one object, the decode table first: at LDS
    // address 0 a table read needs no base added to its index.
    struct Lds {
        uint32_t plut[kLutEntries];                 // 16 KB
        uint32_t stage[kWavesPerBlock][kStageRow];  // 98 KB
        LutScratch scratch;
        uint32_t next_j;  // the workgroup's next unclaimed chunk of the tensor
    };
    __shared__ __attribute__((aligned(16))) Lds lds;
    uint32_t *plut = lds.plut;
    auto &stage = lds.stage;
    LutScratch &scratch = lds.scratch;
    uint32_t &next_j = lds.next_j;

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
        // array together, in one narrow band: the workgroup of rank k of nb
        // (ranks counted XCD by XCD) takes chunks k + j nb, j = 0, 1, ... Wave w starts with j = w and j = w + 16;
        // after that each wave claims the next unclaimed j when it starts a
        // chunk, so waves that the SIMDs serve faster restore more chunks and
        // all finish together.
        if (b < T.blk_lo || b >= T.blk_hi) continue;
        const uint32_t nb = T.blk_hi - T.blk_lo, k = xcd_rank((uint32_t)b - T.blk_lo, nb);
        if (k >= T.n_chunks) continue;
        const uint32_t mine = (T.n_chunks - k + nb - 1) / nb;
        uint32_t jc = wave, jn = wave + kWavesPerBlock;
        const bool has_c = jc < mine;
        bool has_n = jn < mine;
        // Fetch the code lengths, the first two chunks' bases and the first
        // one's gaps, then the first chunk's code words; building the decode
        // table hides the second round trip.
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
        __syncthreads();  // every wave is done with the previous table and counter
        if (threadIdx.x == 0) next_j = 2 * kWavesPerBlock;
        build_lut<kThreads, true>(wave < kSymbolWaves ? len_any : 0u, plut, scratch);
        __syncthreads();  // the pair table is complete
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
            restore_chunk(T, k + (uint64_t)jc * nb, g, gaps, plut, my_stage, lane, bases_nn, gnn);
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

// The jobs of one call may run in one launch: no job's output may share a
// byte with another job's output or with any job's blob (check_job has
// compared each output with its own blob). Sorted by address, the outputs
// must be disjoint, and each blob must miss the output that starts last at
// or below its end (the outputs being disjoint, that is the only one that
// can reach into it). O(n log n): a whole model's tensors in one call.
// Returns -1 when host memory for the sort cannot be had (more than
// kStackRanges jobs only).
int outputs_overlap(const afx_job *jobs, size_t n) {
    struct Range {
        uintptr_t lo, hi;  // [lo, hi)
    };
    // the outputs' ranges: on the stack for up to kStackRanges jobs (a whole
    // model's tensors), on the heap beyond
    constexpr size_t kStackRanges = 1024;
    Range local[kStackRanges];
    std::vector<Range> heap;
    Range *outs = local;
    if (n > kStackRanges) {
        try {
            heap.resize(n);
        } catch (...) {
            return -1;
        }
        outs = heap.data();
    }
    size_t k = 0;
    for (size_t i = 0; i < n; ++i) {
        const uintptr_t o = reinterpret_cast<uintptr_t>(jobs[i].out_dev);
        if (jobs[i].info->decoded_bytes) outs[k++] = Range{o, o + jobs[i].info->decoded_bytes};
    }
    std::sort(outs, outs + k, [](const Range &a, const Range &b) { return a.lo < b.lo; });
    for (size_t i = 1; i < k; ++i)
        if (outs[i].lo < outs[i - 1].hi) return 1;
    for (size_t i = 0; i < n; ++i) {
        if (!jobs[i].info->n_elems) continue;
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(jobs[i].blob_dev), b1 = b0 + jobs[i].info->blob_bytes;
        // the last output starting below the blob's end
        const Range *it = std::lower_bound(outs, outs + k, b1, [](const Range &r, uintptr_t v) { return r.lo < v; });
        if (it != outs && (it - 1)->hi > b0) return 1;
    }
    return 0;
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

// Enqueue one launch for up to AFX_MAX_JOBS_PER_LAUNCH already-checked jobs,
// on at most cap workgroups (cap >= 1).
int launch(const afx_job *jobs, size_t n_jobs, uint32_t cap, hipStream_t stream) {
    Batch batch;
    batch.n_tensors = 0;
    uint64_t chunks[AFX_MAX_JOBS_PER_LAUNCH];
    uint32_t lo[AFX_MAX_JOBS_PER_LAUNCH], hi[AFX_MAX_JOBS_PER_LAUNCH];
    uint32_t n_big = 0;
    // Tensors of fewer chunks than a workgroup has waves (a layer's norm
    // vectors) go last: together they are then a sliver of the grid's last
    // share, served by a workgroup of their own (each tensor a workgroup
    // serves costs it a table build), not added to one that also serves a
    // share of a large tensor.
    for (int pass = 0; pass < 2; ++pass) {
        for (size_t i = 0; i < n_jobs; ++i) {
            const uint64_t nc = jobs[i].info->n_chunks;
            if (nc == 0 || (pass == 0) != (nc >= kWavesPerBlock)) continue;
            chunks[batch.n_tensors] = nc;
            batch.t[batch.n_tensors++] = describe(jobs[i]);
            n_big += pass == 0 ? 1u : 0u;
        }
    }
    if (batch.n_tensors == 0) return AFX_OK;
    int max_blocks = 0;
    int rc = max_blocks_for_current_device(&max_blocks);
    if (rc != AFX_OK) return rc;
    max_blocks = (int)std::min<uint64_t>((uint64_t)max_blocks, cap);
    const uint32_t grid = split_grid(chunks, batch.n_tensors, n_big, (uint32_t)max_blocks, lo, hi);
    for (uint32_t t = 0; t < batch.n_tensors; ++t) {
        batch.t[t].blk_lo = lo[t];
        batch.t[t].blk_hi = hi[t];
    }
    // hipLaunchKernel reports this launch's own status (an error left pending
    // by an earlier, unrelated HIP call is not mistaken for it)
    void *args[] = {&batch};
    return hipLaunchKernel(reinterpret_cast<const void *>(&afx_decode_kernel), dim3((unsigned)grid), dim3(kThreads),
                           args, 0, stream) == hipSuccess
               ? AFX_OK
               : AFX_E_HIP;
}

// Every check of a batch call's jobs.
int check_batch(const afx_job *jobs, size_t n_jobs) {
    if (!jobs && n_jobs) return AFX_E_INVALID_ARG;
    for (size_t i = 0; i < n_jobs; ++i) {
        const int rc = check_job(jobs[i]);
        if (rc != AFX_OK) return rc;
    }
    const int ov = outputs_overlap(jobs, n_jobs);
    if (ov != 0) return ov < 0 ? AFX_E_HOST_MEMORY : AFX_E_INVALID_ARG;
    return AFX_OK;
}

// The launches of a checked batch call.
int decode_batch(const afx_job *jobs, size_t n_jobs, uint32_t cap, hipStream_t s) {
    for (size_t i = 0; i < n_jobs; i += AFX_MAX_JOBS_PER_LAUNCH) {
        const size_t k = std::min<size_t>(AFX_MAX_JOBS_PER_LAUNCH, n_jobs - i);
        const int rc = launch(jobs + i, k, cap, s);
        if (rc != AFX_OK) return rc;
    }
    return AFX_OK;
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
    rc = launch(&job, 1, UINT32_MAX, s);
    if (rc != AFX_OK) return rc;
    return hipStreamSynchronize(s) == hipSuccess ? AFX_OK : AFX_E_HIP;
}

int afx_decode_layer_async(const afx_job *jobs, size_t n_jobs, void *stream) {
    const int rc = check_batch(jobs, n_jobs);
    return rc != AFX_OK ? rc : decode_batch(jobs, n_jobs, UINT32_MAX, static_cast<hipStream_t>(stream));
}

int afx_decode_layer_grid_async(const afx_job *jobs, size_t n_jobs, uint32_t max_workgroups, void *stream) {
    if (max_workgroups == 0) return AFX_E_INVALID_ARG;
    const int rc = check_batch(jobs, n_jobs);
    return rc != AFX_OK ? rc : decode_batch(jobs, n_jobs, max_workgroups, static_cast<hipStream_t>(stream));
}

}  // extern "C"
