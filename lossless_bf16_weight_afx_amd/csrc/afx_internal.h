// afx_internal.h -- private declarations shared by the two halves of libafx
// (host validation/encoder and the HIP decode path). Not installed.
#pragma once

#include <cstddef>
#include <cstdint>
#include <thread>
#include <vector>

#include "../../include/afx.h"

namespace afx {

constexpr uint32_t kChunk = AFX_CHUNK_ELEMS;          // elements per chunk
constexpr uint32_t kGroup = AFX_GROUP_ELEMS;          // elements per group (one lane's work)
constexpr uint32_t kGroupsPerChunk = kChunk / kGroup; // 128
constexpr uint32_t kMaxLen = AFX_MAX_CODE_LEN;        // longest code, bits = LUT index width
constexpr uint32_t kPadWords = 4;                     // zero words after the code stream
constexpr uint32_t kAlign = 256;                      // section alignment in bytes
constexpr uint32_t kHeaderBytes = 256;
constexpr uint64_t kMaxElems = (uint64_t)1 << 40;     // largest tensor accepted

struct Layout {
    uint64_t n_chunks, n_groups, exp_words;
    uint64_t off_code_len, off_chunk_base, off_gap, off_signmant, off_exp, blob_bytes;
};

Layout layout_for(uint64_t n, uint64_t total_bits);
int limited_lengths(const uint64_t freq[256], int limit, uint8_t len[256]);
void canonical(const uint8_t len[256], uint32_t code[256]);
int validate(const uint8_t *blob, size_t nbytes, afx_info *out);
int check_info(const afx_info *info);

// Run fn(i) for every part i in [0, t), one thread per part; the calling
// thread takes part 0, and also every part whose thread could not be started
// (so all parts run, and nothing here throws). fn must not throw.
template <class F>
void run_parts(int t, F &&fn) noexcept {
    std::vector<std::thread> pool;
    int started = 1;
    try {
        pool.reserve(t > 1 ? (size_t)(t - 1) : 0);
        for (; started < t; ++started) {
            const int i = started;
            pool.emplace_back([&fn, i] { fn(i); });
        }
    } catch (...) {
    }
    fn(0);
    for (int i = started; i < t; ++i) fn(i);
    for (auto &th : pool) th.join();
}

// Whether byte ranges [a, a + an) and [b, b + bn) share a byte.
inline bool ranges_overlap(const void *a, uint64_t an, const void *b, uint64_t bn) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return an && bn && a0 < b0 + bn && b0 < a0 + an;
}

// A batch of fused products writes each job's y while it reads every job's
// blob and x: no y may share a byte with any of them (two jobs may add into
// the same y, and share x).
inline bool fused_outputs_overlap_inputs(const afx_gemv_job *jobs, size_t n, uint32_t m) {
    for (size_t i = 0; i < n; ++i) {
        const uint64_t ybytes = (uint64_t)m * jobs[i].rows * 4;
        for (size_t k = 0; k < n; ++k) {
            if (ranges_overlap(jobs[i].y_dev, ybytes, jobs[k].blob_dev, jobs[k].info->blob_bytes) ||
                ranges_overlap(jobs[i].y_dev, ybytes, jobs[k].x_dev, (uint64_t)m * jobs[k].cols * 2))
                return true;
        }
    }
    return false;
}

}  // namespace afx
