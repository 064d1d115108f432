// host_check.cpp -- the library's host-side calls and the oracle, run under
// AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.
//
// Exercised: the encoder (afx_encode_plan, afx_encode) on 1 and 8 threads,
// blob validation (afx_query), the host unpack (afx_decode_host) and the
// oracle's encoder and decoders, on tensors of 0 to 200,003 values with
// narrow, wide and degenerate exponent alphabets; then every one of those
// calls that reads a blob on 300 damaged copies per case (one flipped bit
// anywhere, or a cut end), where any status is allowed but no access out of
// bounds; then the file reader (afx_file_read) with and without O_DIRECT on
// ranges that start and end off page boundaries, and past the file's end.
// Built by tests/test_host_sanitizers.py; exits 1 on a wrong result, and the
// sanitizers abort on an invalid access.
#include <fcntl.h>
#include <unistd.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "afx.h"

extern "C" {
int afx_oracle_plan(const uint16_t *x, uint64_t n, int lmax, uint8_t len[256], uint64_t *total_bits);
uint64_t afx_oracle_blob_bytes(uint64_t n, uint64_t total_bits);
int afx_oracle_encode(const uint16_t *x, uint64_t n, uint32_t ndim, const uint64_t *shape, const uint8_t len[256],
                      uint64_t total_bits, uint8_t *blob, uint64_t blob_bytes);
int afx_oracle_decode(const uint8_t *blob, uint64_t blob_bytes, uint16_t *out, uint64_t out_elems, int threads);
}

namespace {

int g_bad = 0;
#define EXPECT(cond, ...)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            ++g_bad;                                        \
            std::fprintf(stderr, "FAILED: " __VA_ARGS__);   \
            std::fputc('\n', stderr);                       \
        }                                                   \
    } while (0)

// BF16 patterns: "narrow" draws exponents near 120 with a geometric spread
// (as weights of small magnitude have), "wide" any exponent, "zero" and
// "const" one exponent value, "all" every pattern in turn.
std::vector<uint16_t> make(const std::string &kind, uint64_t n, std::mt19937_64 &g) {
    std::vector<uint16_t> x(n);
    for (uint64_t i = 0; i < n; ++i) {
        const uint32_t r = (uint32_t)g();
        uint32_t e = 0;
        if (kind == "narrow") {
            int d = 0;
            while (d < 20 && (g() & 1)) ++d;
            e = (r & 1) ? 120 - d : 121 + d;
        } else if (kind == "wide") {
            e = r >> 24;
        } else if (kind == "const") {
            e = 127;
        } else if (kind == "all") {
            x[i] = (uint16_t)i;
            continue;
        }
        x[i] = (uint16_t)(((r & 1) << 15) | (e << 7) | ((r >> 1) & 0x7F));
        if (kind == "zero") x[i] = 0;
    }
    return x;
}

std::vector<uint8_t> lib_encode(const std::vector<uint16_t> &x, int threads) {
    uint8_t len[256];
    uint64_t bits = 0, nbytes = 0;
    int rc = afx_encode_plan(x.data(), x.size(), threads, len, &bits, &nbytes);
    EXPECT(rc == AFX_OK, "afx_encode_plan %d", rc);
    std::vector<uint8_t> blob(nbytes);
    const uint64_t shape[1] = {x.size()};
    rc = afx_encode(x.data(), x.size(), 1, shape, len, bits, blob.data(), blob.size(), threads);
    EXPECT(rc == AFX_OK, "afx_encode %d", rc);
    return blob;
}

std::vector<uint8_t> oracle_encode(const std::vector<uint16_t> &x) {
    uint8_t len[256];
    uint64_t bits = 0;
    EXPECT(afx_oracle_plan(x.data(), x.size(), 12, len, &bits) == 0, "oracle plan");
    std::vector<uint8_t> blob(afx_oracle_blob_bytes(x.size(), bits));
    const uint64_t shape[1] = {x.size()};
    EXPECT(afx_oracle_encode(x.data(), x.size(), 1, shape, len, bits, blob.data(), blob.size()) == 0, "oracle encode");
    return blob;
}

bool same(const uint16_t *a, const uint16_t *b, uint64_t n) { return n == 0 || std::memcmp(a, b, 2 * n) == 0; }

// Every call that reads a blob, on a blob that may be damaged: statuses are
// free, accesses are not. The output buffers are exactly as large as the
// undamaged tensor needs (the sanitizers see writes past them).
void read_blob(const std::vector<uint8_t> &b, uint64_t n) {
    afx_info info;
    (void)afx_query(b.data(), b.size(), &info);
    std::vector<uint16_t> y(n ? n : 1);
    (void)afx_decode_host(b.data(), b.size(), y.data(), 2 * n, 3);
    (void)afx_oracle_decode(b.data(), b.size(), y.data(), n, 1);
    (void)afx_oracle_decode(b.data(), b.size(), y.data(), n, 3);
}

void codec_cases() {
    std::mt19937_64 g(11);
    const uint64_t sizes[] = {0, 1, 31, 32, 33, 4095, 4096, 4097, 3 * 4096 + 77, 65536, 200003};
    const char *kinds[] = {"narrow", "wide", "zero", "const", "all"};
    for (uint64_t n : sizes) {
        for (const char *k : kinds) {
            if (n == 0 && std::string(k) != "narrow") continue;
            const std::vector<uint16_t> x = make(k, n, g);
            const std::vector<uint8_t> b1 = lib_encode(x, 1), b8 = lib_encode(x, 8);
            EXPECT(b1 == b8, "encoder depends on threads (n=%llu %s)", (unsigned long long)n, k);
            afx_info info;
            EXPECT(afx_query(b1.data(), b1.size(), &info) == AFX_OK && info.n_elems == n, "query n=%llu %s",
                   (unsigned long long)n, k);
            for (int th : {1, 4}) {
                std::vector<uint16_t> y(n ? n : 1);
                EXPECT(afx_decode_host(b1.data(), b1.size(), y.data(), 2 * n, th) == AFX_OK &&
                           same(y.data(), x.data(), n),
                       "host unpack n=%llu %s threads %d", (unsigned long long)n, k, th);
                std::vector<uint16_t> z(n ? n : 1);
                EXPECT(afx_oracle_decode(b1.data(), b1.size(), z.data(), n, th) == 0 &&
                           same(z.data(), x.data(), n),
                       "oracle decode of the library's blob n=%llu %s", (unsigned long long)n, k);
            }
            const std::vector<uint8_t> ob = oracle_encode(x);
            std::vector<uint16_t> z(n ? n : 1);
            EXPECT(afx_oracle_decode(ob.data(), ob.size(), z.data(), n, 1) == 0 && same(z.data(), x.data(), n),
                   "oracle round trip n=%llu %s", (unsigned long long)n, k);
            if (n > 200000) continue;  // damaged copies of the smaller tensors only
            for (int t = 0; t < 300; ++t) {
                std::vector<uint8_t> c = (t & 1) ? b1 : ob;
                if (t % 5 == 4) {
                    c.resize(g() % (c.size() + 1));
                } else {
                    c[g() % c.size()] ^= (uint8_t)(1u << (g() % 8));
                }
                read_blob(c, n);
            }
        }
    }
}

void file_cases() {
    char path[] = "/tmp/afx_host_check_XXXXXX";
    const int fd = mkstemp(path);
    EXPECT(fd >= 0, "mkstemp");
    if (fd < 0) return;
    std::mt19937_64 g(5);
    std::vector<uint8_t> data(9000017);
    for (auto &v : data) v = (uint8_t)g();
    EXPECT(write(fd, data.data(), data.size()) == (ssize_t)data.size(), "write");
    close(fd);
    const uint64_t ranges[][2] = {{0, 1}, {5, 4096}, {4095, 8193}, {12345, 4500000}, {0, 9000017}, {9000014, 3}};
    for (const auto &r : ranges) {
        for (unsigned flags : {0u, (unsigned)AFX_READ_DIRECT}) {
            std::vector<uint8_t> dst(r[1]);
            const int rc = afx_file_read(path, r[0], r[1], dst.data(), 4, flags);
            EXPECT(rc == AFX_OK || (flags && rc == AFX_E_UNSUPPORTED), "file read rc %d", rc);
            if (rc == AFX_OK)
                EXPECT(std::memcmp(dst.data(), data.data() + r[0], r[1]) == 0, "file read bytes [%llu, +%llu)",
                       (unsigned long long)r[0], (unsigned long long)r[1]);
        }
    }
    std::vector<uint8_t> dst(10);
    EXPECT(afx_file_read(path, data.size() - 5, 10, dst.data(), 2, 0) == AFX_E_IO, "read past the end");
    unlink(path);
}

}  // namespace

int main() {
    codec_cases();
    std::printf("codec cases done\n");
    file_cases();
    std::printf("file cases done, %d failures\n", g_bad);
    return g_bad ? 1 : 0;
}
