/*
 * afx.h -- C ABI of libafx: lossless BF16 weight blobs restored on the GPU.
 *
 * The operation. "Why Weight Offloading Slows Inference" (section "Three
 * steps for each weight", Eq. (1)) puts an unpack step, t_unpack, between
 * reading a stored weight and using it; section "Lossless compression"
 * entropy-codes the BF16 exponent field without loss (a minimum-redundancy
 * prefix code, that page's reference [2]), so that each weight's original
 * 16 bits must be reconstructed before it is used. This library performs that
 * reconstruction on an
 * AMD Instinct MI355X (gfx950), after the compressed bytes have been copied
 * to device memory, and writes the BF16 bit patterns into a caller buffer.
 *
 * Blob format (version 1), little-endian; every section starts on a
 * 256-byte boundary and the blob length is a multiple of 256:
 *   [0,256)        header: "AFX1", u32 version = 1, u64 n, u64 total_bits,
 *                  u64 exp_words, u32 ndim, u32 4096, u32 32, u32 12,
 *                  u32 n_symbols, 12 zero bytes, u64 shape[4] at byte 64, zeros
 *   code_len[256]  u8 code length of each exponent value (0 = unused, <= 12)
 *   chunk_base     u64 x (n_chunks + 1): bit position where each 4096-element
 *                  chunk starts; the last entry equals total_bits
 *   gap            u16 x n_groups: start of each 32-element group, in bits
 *                  after its chunk's base
 *   signmant       u8 x n: (sign << 7) | mantissa7 of each element
 *   exp            u32 x exp_words: the canonical code stream of the 8-bit
 *                  exponent fields, MSB first in each word, then zero words
 * Element i is ((signmant[i] & 0x80) << 8) | (exponent << 7) |
 * (signmant[i] & 0x7F). The code is canonical: symbols ordered by (length,
 * value) take consecutive codes; a tensor with one exponent value uses one
 * 1-bit code.
 *
 * Conventions. Every function returns AFX_OK (0) or a negative afx_status,
 * never aborts and never prints. Argument and format errors are detected
 * before any HIP call and leave every output untouched. The library keeps no
 * pointer after a call returns and allocates no device memory.
 */
#ifndef AFX_H
#define AFX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AFX_ABI_VERSION 1u
#define AFX_FORMAT_VERSION 1u
#define AFX_CHUNK_ELEMS 4096u
#define AFX_GROUP_ELEMS 32u
#define AFX_MAX_CODE_LEN 12u
#define AFX_MAX_JOBS_PER_LAUNCH 32u

typedef enum afx_status {
    AFX_OK = 0,
    AFX_E_INVALID_ARG = -1,     /* NULL pointer, zero-size or inconsistent argument */
    AFX_E_BAD_MAGIC = -2,       /* blob does not start with "AFX1" */
    AFX_E_BAD_VERSION = -3,     /* unknown format version or fixed-field value */
    AFX_E_CORRUPT = -4,         /* inconsistent header, code lengths, bases or gaps */
    AFX_E_BUFFER_TOO_SMALL = -5,/* blob shorter than its header says, or output too small */
    AFX_E_MISALIGNED = -6,      /* device pointer not 16-byte aligned */
    AFX_E_HIP = -7,             /* a HIP runtime call failed (launch or execution) */
    AFX_E_UNSUPPORTED = -8,     /* request beyond what the library supports */
    AFX_E_IO = -9,              /* a file could not be opened or read in full */
    AFX_E_HOST_MEMORY = -10     /* host memory for the call's own work could not be had */
} afx_status;
/* No entry point throws, aborts or prints: the host-side calls that allocate
 * working memory (the encoder, the host unpack, the file reader) return
 * AFX_E_HOST_MEMORY when it cannot be had, and run on fewer threads when
 * threads cannot be started. */

/* What afx_query reports about a blob. Offsets are in bytes from the blob's
 * first byte; sizes count elements unless named *_bytes. */
typedef struct afx_info {
    uint32_t abi_version;     /* AFX_ABI_VERSION of the library that filled it */
    uint32_t format_version;  /* 1 */
    uint64_t n_elems;         /* BF16 elements restored */
    uint64_t decoded_bytes;   /* 2 * n_elems */
    uint64_t blob_bytes;      /* bytes of the blob, a multiple of 256 */
    uint64_t total_bits;      /* length of the exponent code stream */
    uint64_t exp_words;       /* u32 words of the exp section, padding included */
    uint64_t n_chunks;        /* ceil(n / 4096) */
    uint64_t n_groups;        /* ceil(n / 32) */
    uint32_t ndim;            /* 0..4 */
    uint32_t n_symbols;       /* exponent values in use */
    uint64_t shape[4];        /* unused dimensions are 0 */
    uint32_t chunk_elems;     /* 4096 */
    uint32_t group_elems;     /* 32 */
    uint32_t max_code_len;    /* 12 */
    uint32_t longest_code;    /* longest length actually used */
    uint64_t off_code_len, off_chunk_base, off_gap, off_signmant, off_exp;
} afx_info;

/* One tensor of a batch. */
typedef struct afx_job {
    const afx_info *info;  /* filled by afx_query from a host copy of the blob */
    const void *blob_dev;  /* device copy of the same blob, 16-byte aligned */
    void *out_dev;         /* device output of n_elems u16 (BF16), 16-byte aligned */
    size_t out_bytes;      /* capacity of out_dev in bytes, >= 2 * n_elems */
} afx_job;

/* afx_query: inspect a blob held in host memory (pageable or pinned).
 * Checks the header, the code lengths (each <= 12; Kraft sum exactly 1 when
 * two or more values are used, a single 1-bit code otherwise), the chunk
 * bases (start at 0, non-decreasing, at most 12 bits per element, end at
 * total_bits) and the group gaps (0 at each chunk start, non-decreasing,
 * within the chunk), then fills *info. Host only, no HIP call.
 * Errors: AFX_E_INVALID_ARG (NULL), AFX_E_BUFFER_TOO_SMALL (blob_bytes short),
 * AFX_E_BAD_MAGIC, AFX_E_BAD_VERSION, AFX_E_CORRUPT. */
int afx_query(const void *blob_host, size_t blob_bytes, afx_info *info);

/* afx_decode_tensor: restore one tensor and wait for it.
 * info comes from afx_query on a host copy of the blob whose device copy is
 * blob_dev. Writes exactly 2 * n_elems bytes at out_dev and nothing else.
 * stream is a hipStream_t (NULL = the default stream); the call enqueues the
 * decode on it and then synchronizes that stream, so asynchronous kernel
 * errors are reported too. Output must not overlap the blob.
 * Errors: AFX_E_INVALID_ARG, AFX_E_BUFFER_TOO_SMALL (out_bytes < 2n),
 * AFX_E_MISALIGNED, AFX_E_HIP. A device blob that differs from the validated
 * host copy decodes to wrong values but never reads or writes out of bounds. */
int afx_decode_tensor(const afx_info *info, const void *blob_dev, void *out_dev, size_t out_bytes,
                      void *stream);

/* afx_decode_layer_async: restore a batch of tensors (e.g. the 11 tensors of
 * one decoder layer, the unit that page's section "Loading during
 * computation" prefetches) with one launch per AFX_MAX_JOBS_PER_LAUNCH jobs,
 * enqueued on stream; returns without waiting. Completion is observed through
 * the stream or events recorded on it. All jobs are checked before anything
 * is enqueued. Errors: as afx_decode_tensor, but only enqueue-time HIP errors
 * are reported; AFX_E_HOST_MEMORY when the host memory for the overlap check
 * of a batch of more than 1024 jobs cannot be had (up to 1024 it allocates
 * nothing). */
int afx_decode_layer_async(const afx_job *jobs, size_t n_jobs, void *stream);

/* afx_decode_layer_grid_async: afx_decode_layer_async on at most
 * max_workgroups workgroups per launch (one workgroup per CU at most, so
 * this many CUs at most; a larger value is the whole device, as in
 * afx_decode_layer_async). For a caller that restores the next unit while
 * its computation runs on the same GPU ("Why Weight Offloading Slows
 * Inference", section "Loading during computation"): the restore then
 * leaves the other CUs to that computation. Outputs are the same bits for
 * every max_workgroups. Errors: as afx_decode_layer_async;
 * AFX_E_INVALID_ARG when max_workgroups is 0. */
int afx_decode_layer_grid_async(const afx_job *jobs, size_t n_jobs, uint32_t max_workgroups, void *stream);

/* afx_status_str: a static description of a status code. */
const char *afx_status_str(int status);

/* ---- Encoder (host). Produces format-1 blobs; the code lengths are an
 * optimal prefix code limited to 12 bits over the tensor's exponent values. */

/* afx_encode_plan: histogram the exponents of x (n BF16 bit patterns), pick
 * the code lengths, and report the stream length and the blob size.
 * threads <= 0 picks the hardware thread count. Errors: AFX_E_INVALID_ARG
 * (NULL pointer), AFX_E_UNSUPPORTED (n above 2^40), AFX_E_HOST_MEMORY. */
int afx_encode_plan(const uint16_t *x, uint64_t n, int threads, uint8_t code_len[256],
                    uint64_t *total_bits, uint64_t *blob_bytes);

/* afx_encode: write the blob for x with the lengths and stream length from
 * afx_encode_plan into blob (host memory, blob_bytes >= the planned size).
 * shape has ndim entries (ndim 1..4, product == n). Errors: AFX_E_INVALID_ARG
 * (NULL pointer, ndim out of range, shape product != n, code_len not a
 * complete prefix code of lengths <= 12 -- Kraft sum 1, or one symbol of
 * length 1 --, an exponent of x without a code, total_bits not the stream
 * length those lengths give x), AFX_E_UNSUPPORTED (n above 2^40),
 * AFX_E_BUFFER_TOO_SMALL (blob_bytes below the blob size),
 * AFX_E_HOST_MEMORY. On an error the blob's contents are unspecified. */
int afx_encode(const uint16_t *x, uint64_t n, uint32_t ndim, const uint64_t *shape,
               const uint8_t code_len[256], uint64_t total_bits, void *blob, size_t blob_bytes,
               int threads);

/* ---- The restore fused into its consumer. "Why Weight Offloading Slows
 * Inference" (section "Lossless compression") reconstructs a weight's bits
 * ahead of the computation that uses it; when that computation is a product
 * on the GPU, the reconstructed matrix need not reach HBM at all. */

/* afx_restore_gemv_async: y += W x, where W is the tensor of the device blob
 * (info from afx_query on a host copy), taken as row-major [rows, cols]
 * (rows * cols == n_elems), x is BF16 [m, cols] and y FP32 [m, rows], both
 * row-major in device memory; m is 1, 2 or 4. W is restored chunk by chunk
 * in registers and LDS and never written out. Products of two BF16 values
 * are exact in FP32; the sums are FP32 and added into y with atomic adds,
 * so their order (and the last bits) may differ between calls. The caller
 * owns y and its initial contents. Enqueued on stream; returns without
 * waiting. Errors: as afx_decode_layer_async; AFX_E_INVALID_ARG (rows *
 * cols != n_elems, NULL pointer, y sharing a byte with the blob or x),
 * AFX_E_UNSUPPORTED (cols not a multiple of
 * 8 or 2^31 or more; m not 1, 2 or 4), AFX_E_MISALIGNED (blob or x not
 * 16-byte aligned, y not 4-byte aligned). */
int afx_restore_gemv_async(const afx_info *info, const void *blob_dev, uint64_t rows, uint64_t cols,
                           const uint16_t *x_dev, uint32_t m, float *y_dev, void *stream);

#define AFX_MAX_GEMV_JOBS_PER_LAUNCH 16u

/* One matrix of a batch of products (e.g. the seven of a decoder layer). */
typedef struct afx_gemv_job {
    const afx_info *info;  /* filled by afx_query from a host copy of the blob */
    const void *blob_dev;  /* device copy of the same blob, 16-byte aligned */
    uint64_t rows, cols;   /* W is row-major [rows, cols], rows * cols == n_elems */
    const uint16_t *x_dev; /* BF16 [m, cols], 16-byte aligned */
    float *y_dev;          /* FP32 [m, rows], added into, 4-byte aligned */
} afx_gemv_job;

/* afx_restore_gemv_batch_async: afx_restore_gemv_async for every job (all
 * with the same m), one launch per AFX_MAX_GEMV_JOBS_PER_LAUNCH jobs; all
 * jobs are checked before anything is enqueued. Jobs may share x and may
 * add into the same y; no job's y may share a byte with any job's blob or
 * x (AFX_E_INVALID_ARG). Errors otherwise as afx_restore_gemv_async. */
int afx_restore_gemv_batch_async(const afx_gemv_job *jobs, size_t n_jobs, uint32_t m, void *stream);

/* ---- The restore fused into a product over many tokens (prefill). The
 * same restore as above, but tiles of W go from LDS straight into the
 * matrix cores instead of to HBM. */

/* afx_restore_gemm_async: y += x W^T, where W is the tensor of the device
 * blob (info from afx_query on a host copy), taken as row-major
 * [rows, cols] (rows * cols == n_elems), x is BF16 [m, cols] and y FP32
 * [m, rows], both row-major in device memory; any m >= 1. 64-row tiles of W
 * are restored into LDS 256 columns at a time and multiplied there with
 * BF16 matrix instructions (FP32 accumulation); for m = 1, 2 or 4 the call
 * runs afx_restore_gemv_async's kernel instead, which is faster for so few
 * tokens (the same y within the same bound). Tiles over different column
 * ranges of the same rows add their partial sums into y with atomic adds,
 * so their order (and the last bits) may differ between calls. The caller
 * owns y and its initial contents. Enqueued on stream; returns without
 * waiting. Errors: as afx_decode_layer_async; AFX_E_INVALID_ARG (rows *
 * cols != n_elems, a zero size, NULL pointer, y sharing a byte with the
 * blob or x), AFX_E_UNSUPPORTED (rows not
 * a multiple of 64, cols not a multiple of 256, either >= 2^31, m == 0 or
 * m > 8388480), AFX_E_MISALIGNED (blob or x not 16-byte aligned, y not
 * 4-byte aligned). */
int afx_restore_gemm_async(const afx_info *info, const void *blob_dev, uint64_t rows, uint64_t cols,
                           const uint16_t *x_dev, uint32_t m, float *y_dev, void *stream);

/* afx_restore_gemm_batch_async: afx_restore_gemm_async for every job (all
 * with the same m), one launch per AFX_MAX_GEMV_JOBS_PER_LAUNCH jobs; all
 * jobs are checked before anything is enqueued. Jobs may share x and may
 * add into the same y; no job's y may share a byte with any job's blob or
 * x (AFX_E_INVALID_ARG). Errors otherwise as afx_restore_gemm_async. */
int afx_restore_gemm_batch_async(const afx_gemv_job *jobs, size_t n_jobs, uint32_t m, void *stream);

/* ---- Unpack on the host. "Why Weight Offloading Slows Inference" (section
 * "The path from storage to the GPU", Figure 1) unpacks a compressed weight
 * in RAM between the read and the copy to the GPU, and section "Lossless
 * compression" finds that placement too slow for compression to pay
 * (Eq. (2)). The GPU entry points above never call this; it exists to
 * measure that placement beside the GPU restore. */

/* afx_decode_host: validate a host blob as afx_query does, then restore its
 * n_elems BF16 bit patterns into out (host memory, out_bytes >= 2 n), with
 * `threads` workers over chunks (<= 0: hardware thread count).
 * Errors: as afx_query; AFX_E_INVALID_ARG (NULL out with n > 0),
 * AFX_E_BUFFER_TOO_SMALL (out_bytes < 2 n), AFX_E_HOST_MEMORY. */
int afx_decode_host(const void *blob_host, size_t blob_bytes, uint16_t *out, size_t out_bytes, int threads);

/* ---- Storage (host). "Why Weight Offloading Slows Inference" (section
 * "The path from storage to the GPU", Figure 1, and Eq. (1)) reads a stored
 * weight from the SSD into RAM before unpacking it and copying it to the GPU;
 * the page measures that read with the page cache cleared. */

#define AFX_READ_DIRECT 1u /* open with O_DIRECT: bypass the page cache */

/* afx_file_read: read bytes [offset, offset + bytes) of the file at path into
 * dst (host memory owned by the caller, any alignment; pinned memory lets a
 * following copy to the GPU start from it), with `threads` workers (<= 0:
 * the hardware thread count) each issuing 4 MiB preads. With
 * AFX_READ_DIRECT each worker reads the enclosing 4096-aligned range into
 * its own page-aligned 4 MiB buffer and copies the requested part to dst
 * (the kernel refuses direct transfers into GPU-pinned host memory). On
 * error dst may be partly written.
 * Errors: AFX_E_INVALID_ARG (NULL path or dst, unknown flag, offset +
 * bytes above 2^63 - 1), AFX_E_UNSUPPORTED (the file system refuses
 * O_DIRECT), AFX_E_IO (open or read failed, or the file ends inside the
 * range), AFX_E_HOST_MEMORY (no bounce buffer for a direct read). */
int afx_file_read(const char *path, uint64_t offset, uint64_t bytes, void *dst, int threads, unsigned flags);

#ifdef __cplusplus
}
#endif

#endif /* AFX_H */
