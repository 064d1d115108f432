// split_check.cpp -- on the CPU, the restore's division of a launch's grid
// among its tensors (afx_split.h): every range inside the grid, no idle
// workgroup, never a busier workgroup than the proportional split, the
// fewest possible chunks on the busiest workgroup wherever brute force can
// tell, and the decoder layer's full-grid launch left exactly proportional.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_split.py; prints "split ok" and exits 0, else exits 1.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "afx_split.h"

using namespace afx;

namespace {

int g_fail = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            if (g_fail++ < 20) {                           \
                std::fprintf(stderr, "split: " __VA_ARGS__); \
                std::fputc('\n', stderr);                  \
            }                                              \
        }                                                  \
    } while (0)

// The proportional ranges alone, written out again from their definition.
uint32_t proportional(const std::vector<uint64_t> &c, uint32_t max_blocks, std::vector<uint32_t> &lo,
                      std::vector<uint32_t> &hi) {
    uint64_t total = 0;
    for (uint64_t x : c) total += x;
    const uint64_t per = (total + max_blocks - 1) / max_blocks;
    uint64_t grid = (total + per - 1) / per;
    if (grid > max_blocks) grid = max_blocks;
    uint64_t first = 0;
    for (size_t t = 0; t < c.size(); ++t) {
        lo[t] = (uint32_t)(grid * first / total);
        hi[t] = (uint32_t)(grid * (first + c[t]) / total);
        if (hi[t] <= lo[t]) hi[t] = lo[t] + 1;
        first += c[t];
    }
    return (uint32_t)grid;
}

// Per-workgroup chunk counts under the kernel's rule (rank k of nb takes
// chunks k, k + nb, ...), counted chunk by chunk.
std::vector<uint64_t> loads(const std::vector<uint64_t> &c, uint32_t grid, const std::vector<uint32_t> &lo,
                            const std::vector<uint32_t> &hi) {
    std::vector<uint64_t> l(grid, 0);
    for (size_t t = 0; t < c.size(); ++t) {
        const uint64_t nb = hi[t] - lo[t];
        for (uint64_t j = 0; j < c[t]; ++j) ++l[lo[t] + j % nb];
    }
    return l;
}

uint64_t max_of(const std::vector<uint64_t> &v) {
    uint64_t m = 0;
    for (uint64_t x : v) m = x > m ? x : m;
    return m;
}

// Smallest possible busiest workgroup when the large tensors get disjoint
// workgroups (at least one each, at most budget in all), by brute force.
uint64_t best_disjoint(const std::vector<uint64_t> &c, uint32_t n_big, uint32_t budget) {
    uint64_t best = ~(uint64_t)0;
    std::vector<uint32_t> nb(n_big, 1);
    while (true) {
        uint32_t used = 0;
        uint64_t m = 0;
        for (uint32_t t = 0; t < n_big; ++t) {
            used += nb[t];
            const uint64_t b = (c[t] + nb[t] - 1) / nb[t];
            m = b > m ? b : m;
        }
        if (used <= budget && m < best) best = m;
        uint32_t t = 0;
        while (t < n_big && ++nb[t] > budget) nb[t++] = 1;
        if (t == n_big) break;
    }
    return best;
}

void check_split(const std::vector<uint64_t> &c, uint32_t n_big, uint32_t max_blocks, bool brute) {
    const uint32_t n = (uint32_t)c.size();
    std::vector<uint32_t> lo(n), hi(n), plo(n), phi(n);
    const uint32_t grid = split_grid(c.data(), n, n_big, max_blocks, lo.data(), hi.data());
    const uint32_t pgrid = proportional(c, max_blocks, plo, phi);
    CHECK(grid >= 1 && grid <= max_blocks, "grid %u of at most %u", grid, max_blocks);
    if (grid < 1 || grid > max_blocks) return;
    for (uint32_t t = 0; t < n; ++t)
        CHECK(lo[t] < hi[t] && hi[t] <= grid, "tensor %u range [%u, %u) in a grid of %u", t, lo[t], hi[t], grid);
    if (g_fail) return;
    const std::vector<uint64_t> l = loads(c, grid, lo, hi);
    uint64_t sum = 0;
    for (uint64_t x : l) sum += x;
    uint64_t total = 0;
    for (uint64_t x : c) total += x;
    CHECK(sum == total, "%llu chunks assigned of %llu", (unsigned long long)sum, (unsigned long long)total);
    for (uint32_t b = 0; b < grid; ++b) CHECK(l[b] > 0, "workgroup %u of %u idle", b, grid);
    const uint64_t pmax = max_of(loads(c, pgrid, plo, phi));
    const uint64_t m = max_of(l);
    CHECK(m <= pmax, "busiest workgroup %llu chunks, proportional %llu", (unsigned long long)m,
          (unsigned long long)pmax);
    if (m == pmax) {  // then the launch is the proportional one
        CHECK(grid == pgrid, "grid %u, proportional %u", grid, pgrid);
        for (uint32_t t = 0; t < n; ++t) CHECK(lo[t] == plo[t] && hi[t] == phi[t], "tensor %u not proportional", t);
    }
    if (brute && n_big > 0) {
        const uint32_t extra = n_big < n ? 1 : 0;
        if (n_big + extra <= max_blocks) {
            uint64_t small = 0;
            for (uint32_t t = n_big; t < n; ++t) small += c[t];
            uint64_t opt = best_disjoint(c, n_big, max_blocks - extra);
            opt = opt > small ? opt : small;
            const uint64_t want = opt < pmax ? opt : pmax;
            CHECK(m == want, "busiest workgroup %llu, best possible %llu", (unsigned long long)m,
                  (unsigned long long)want);
        }
    }
}

}  // namespace

int main() {
    // A Qwen3-14B decoder layer: q, k, v, o, gate, up, down, then the four
    // norm vectors (fewer chunks than a workgroup has waves).
    const std::vector<uint64_t> layer = {6400, 1280, 1280, 6400, 21760, 21760, 21760, 1, 1, 2, 2};
    for (uint32_t cap = 1; cap <= 300; ++cap) check_split(layer, 7, cap, false);
    {
        std::vector<uint32_t> lo(11), hi(11), plo(11), phi(11);
        const uint32_t g = split_grid(layer.data(), 11, 7, 256, lo.data(), hi.data());
        const uint32_t pg = proportional(layer, 256, plo, phi);
        CHECK(g == pg && lo == plo && hi == phi, "full-grid layer launch is not the proportional one");
        const uint32_t g96 = split_grid(layer.data(), 11, 7, 96, lo.data(), hi.data());
        CHECK(max_of(loads(layer, g96, lo, hi)) == 871, "layer on 96 workgroups: busiest %llu chunks, want 871",
              (unsigned long long)max_of(loads(layer, g96, lo, hi)));
    }
    std::mt19937_64 rng(11);
    for (int it = 0; it < 5000; ++it) {
        const bool small_case = it % 2 == 0;
        const uint32_t n_big = (uint32_t)(rng() % (small_case ? 4 : 25));
        const uint32_t n_small = (uint32_t)(rng() % (small_case ? 3 : 8));
        if (n_big + n_small == 0) continue;
        std::vector<uint64_t> c;
        for (uint32_t t = 0; t < n_big; ++t)
            c.push_back(16 + (small_case ? rng() % 200 : (rng() % 4 ? rng() % 5000 : rng() % 100000)));
        for (uint32_t t = 0; t < n_small; ++t) c.push_back(1 + rng() % 15);
        const uint32_t max_blocks = small_case ? 1 + (uint32_t)(rng() % 12)
                                               : (rng() % 3 ? 1 + (uint32_t)(rng() % 300) : 256);
        check_split(c, n_big, max_blocks, small_case);
    }
    if (g_fail) {
        std::printf("%d failures\n", g_fail);
        return 1;
    }
    std::printf("split ok\n");
    return 0;
}
