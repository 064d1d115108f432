// afx_split.h -- how a restore launch divides its grid among its tensors.
//
// Workgroup b of a launch serves every tensor t with lo[t] <= b < hi[t];
// within a tensor of c chunks served by nb workgroups, the workgroup of rank
// k takes chunks k, k + nb, k + 2 nb, ... (ceil((c - k) / nb) of them). A
// launch lasts about as long as its busiest workgroup, so the split should
// keep the largest per-workgroup chunk count low with few workgroups.
//
// Host code only, no HIP header: the restore's launch code and a plain CPU
// test (tests/native/split_check.cpp) use the same function.
#pragma once

#include <cstdint>

namespace afx {

// Grids above this are split in proportion only (no second candidate).
constexpr uint32_t kSplitMaxGrid = 1024;

// Chunks of the busiest workgroup of a split, or 0 if the grid exceeds
// kSplitMaxGrid. Ranges must lie inside [0, grid).
inline uint64_t split_max_load(const uint64_t *chunks, uint32_t n, uint32_t grid, const uint32_t *lo,
                               const uint32_t *hi) {
    if (grid > kSplitMaxGrid) return 0;
    uint64_t load[kSplitMaxGrid] = {};
    for (uint32_t t = 0; t < n; ++t) {
        const uint64_t nb = hi[t] - lo[t];
        for (uint64_t k = 0; k < nb && k < chunks[t]; ++k) load[lo[t] + k] += (chunks[t] - k + nb - 1) / nb;
    }
    uint64_t m = 0;
    for (uint32_t b = 0; b < grid; ++b) m = load[b] > m ? load[b] : m;
    return m;
}

// Split a grid of at most max_blocks (>= 1) workgroups among n tensors
// (chunks[t] >= 1, the first n_big of them of at least one chunk per wave,
// the rest smaller), filling lo[t], hi[t]; returns the grid size.
//
// First candidate: ranges in proportion to the chunk counts, over just
// enough workgroups for ceil(total / max_blocks) chunks each; a tensor whose
// share rounds to nothing takes the one workgroup at its position (with its
// neighbour). Second candidate, when every large tensor can have workgroups
// of its own and the small ones one more: the smallest maximum L of chunks
// per workgroup that the large tensors can reach with disjoint workgroups,
// each tensor taking the fewest (ceil(c / L)) that reach it, found by
// bisection; the small tensors share a last workgroup. The
// second is used only when its busiest workgroup holds strictly fewer
// chunks: proportional ranges keep each array's workgroups spread over the
// grid in order, and when the rounding of the shares is harmless (a full
// grid over a decoder layer) the launch is exactly the proportional one.
inline uint32_t split_grid(const uint64_t *chunks, uint32_t n, uint32_t n_big, uint32_t max_blocks, uint32_t *lo,
                           uint32_t *hi) {
    uint64_t total = 0;
    for (uint32_t t = 0; t < n; ++t) total += chunks[t];
    const uint64_t per_block = (total + max_blocks - 1) / max_blocks;
    const uint64_t want = (total + per_block - 1) / per_block;
    uint64_t g = want < max_blocks ? want : max_blocks;
    const uint32_t grid = (uint32_t)(g < 1 ? 1 : g);
    uint64_t first = 0;
    for (uint32_t t = 0; t < n; ++t) {
        const uint64_t l = grid * first / total;
        uint64_t h = grid * (first + chunks[t]) / total;
        if (h <= l) h = l + 1;
        lo[t] = (uint32_t)l;
        hi[t] = (uint32_t)h;
        first += chunks[t];
    }
    const uint32_t extra = n_big < n ? 1u : 0u;
    if (n_big == 0 || (uint64_t)n_big + extra > max_blocks || grid > kSplitMaxGrid) return grid;
    const uint64_t prop_max = split_max_load(chunks, n, grid, lo, hi);

    // The fewest chunks L on any large tensor's workgroup such that giving
    // each tensor ceil(c / L) workgroups stays within the budget (the count
    // falls as L grows; at the largest c it is one workgroup per tensor).
    uint64_t budget = (uint64_t)max_blocks - extra;
    if (budget > kSplitMaxGrid) budget = kSplitMaxGrid;
    auto need = [&](uint64_t L) {
        uint64_t k = 0;
        for (uint32_t t = 0; t < n_big; ++t) k += (chunks[t] + L - 1) / L;
        return k;
    };
    uint64_t L_lo = 1, L = 1;
    for (uint32_t t = 0; t < n_big; ++t) L = chunks[t] > L ? chunks[t] : L;
    while (L_lo < L) {
        const uint64_t mid = L_lo + (L - L_lo) / 2;
        if (need(mid) <= budget)
            L = mid;
        else
            L_lo = mid + 1;
    }
    uint64_t small_sum = 0;
    for (uint32_t t = n_big; t < n; ++t) small_sum += chunks[t];
    const uint64_t min_max = L > small_sum ? L : small_sum;
    if (min_max >= prop_max) return grid;
    uint32_t at = 0;
    for (uint32_t t = 0; t < n_big; ++t) {
        const uint32_t nb = (uint32_t)((chunks[t] + L - 1) / L);
        lo[t] = at;
        hi[t] = at + nb;
        at += nb;
    }
    for (uint32_t t = n_big; t < n; ++t) {
        lo[t] = at;
        hi[t] = at + 1;
    }
    return at + extra;
}

}  // namespace afx
