// afx_internal.h -- private declarations shared by the two halves of libafx
// (host validation/encoder and the HIP decode path). Not installed.
#pragma once

#include <cstddef>
#include <cstdint>

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

}  // namespace afx
