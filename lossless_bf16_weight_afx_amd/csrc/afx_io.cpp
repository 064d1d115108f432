// afx_io.cpp -- the read step of the time-to-ready model: a stored byte range
// of a file read into host memory (typically pinned, so that the next step's
// copy to the GPU can start from it).
//
// "Why Weight Offloading Slows Inference" (section "The path from storage to
// the GPU", Figure 1) reads a stored weight from the SSD into RAM before it is
// unpacked and copied over PCIe; Eq. (1) charges that read S_disk / b_disk.
// The page measures b_disk with the operating system's page cache cleared;
// here direct reads (O_DIRECT) bypass that cache altogether.
//
// The range is cut into pieces of kPiece bytes that `threads` workers read
// with pread, so that several requests are in flight at the device. A direct
// read lands in the worker's own page-aligned bounce buffer (the kernel
// refuses direct transfers into some memory, GPU-pinned host memory among
// it) and is copied from there to its place. No HIP calls here.
#include "afx_internal.h"

#include <fcntl.h>
#include <unistd.h>

#include <atomic>
#include <cerrno>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr uint64_t kPiece = 4ull << 20;  // bytes per request
constexpr uint64_t kDirectAlign = 4096;  // O_DIRECT offset, size and buffer alignment

// Read up to `bytes` at `offset`, stopping early only at the end of the file;
// returns the bytes read, or -1 on an error.
int64_t read_upto(int fd, uint8_t *dst, uint64_t bytes, uint64_t offset) {
    uint64_t got = 0;
    while (got < bytes) {
        const ssize_t r = pread(fd, dst + got, bytes - got, (off_t)(offset + got));
        if (r < 0) {
            if (errno == EINTR) continue;
            return -1;
        }
        if (r == 0) break;  // end of file
        got += (uint64_t)r;
    }
    return (int64_t)got;
}

}  // namespace

extern "C" int afx_file_read(const char *path, uint64_t offset, uint64_t bytes, void *dst, int threads,
                             unsigned flags) {
    if (!path || (!dst && bytes) || (flags & ~AFX_READ_DIRECT)) return AFX_E_INVALID_ARG;
    if (bytes == 0) return AFX_OK;
    if (offset > (uint64_t)INT64_MAX || bytes > (uint64_t)INT64_MAX - offset) return AFX_E_INVALID_ARG;
    const bool direct = flags & AFX_READ_DIRECT;
    const int fd = open(path, O_RDONLY | O_CLOEXEC | (direct ? O_DIRECT : 0));
    if (fd < 0) return direct && errno == EINVAL ? AFX_E_UNSUPPORTED : AFX_E_IO;
    // A direct read covers the enclosing 4096-aligned range.
    const uint64_t lo = direct ? offset / kDirectAlign * kDirectAlign : offset;
    const uint64_t end = offset + bytes;
    const uint64_t pieces = (end - lo + kPiece - 1) / kPiece;
    int t = threads > 0 ? threads : (int)std::thread::hardware_concurrency();
    if (t < 1) t = 1;
    if (t > 64) t = 64;
    if ((uint64_t)t > pieces) t = (int)pieces;
    std::atomic<uint64_t> next{0};
    std::atomic<bool> ok{true};
    std::atomic<int> status{AFX_OK};
    auto fail = [&](int rc) {
        int expected = AFX_OK;
        status.compare_exchange_strong(expected, rc);
        ok = false;
    };
    // Workers take pieces from one counter until none is left, so any
    // number of them reads the whole range.
    auto worker = [&](int) {
        uint8_t *bounce = nullptr;
        if (direct) {
            bounce = static_cast<uint8_t *>(std::aligned_alloc(kDirectAlign, kPiece));
            if (!bounce) {
                fail(AFX_E_HOST_MEMORY);
                return;
            }
        }
        for (uint64_t p; ok.load(std::memory_order_relaxed) && (p = next.fetch_add(1)) < pieces;) {
            const uint64_t at = lo + p * kPiece;              // file offset of this piece
            const uint64_t want = std::min(kPiece, end - at);  // bytes of it inside [lo, end)
            if (!direct) {
                if (read_upto(fd, static_cast<uint8_t *>(dst) + (at - offset), want, at) != (int64_t)want)
                    fail(AFX_E_IO);
                continue;
            }
            const uint64_t len = (want + kDirectAlign - 1) / kDirectAlign * kDirectAlign;
            const int64_t got = read_upto(fd, bounce, len, at);
            if (got < (int64_t)want) {
                fail(AFX_E_IO);
                continue;
            }
            const uint64_t from = std::max(at, offset);  // the part of the piece the caller asked for
            std::memcpy(static_cast<uint8_t *>(dst) + (from - offset), bounce + (from - at), at + want - from);
        }
        std::free(bounce);
    };
    afx::run_parts(t, worker);
    close(fd);
    return status.load();
}
