/*
 * q4g128_diag.h -- benchmark diagnostics for the int4 group-128 GEMV
 * (libq4g128_diag.so, a library of its own; not part of the product ABI in
 * q4g128.h).  Each kernel bounds what the batch-1 GEMV can reach on the device
 * it runs on; bench.py times them next to the GEMV.
 *
 * The read-only twin follows the rumik int4 write-up ("Step 7: why the GEMV
 * was stuck, and a CUDA kernel"): a copy of the GEMV that issues the same
 * loads and does none of the arithmetic, so that the difference between the
 * two is the cost of the arithmetic.
 *
 * Every pointer is device memory owned by the caller; calls only enqueue on
 * `stream` (a hipStream_t, NULL = the null stream).  Return 0 on success,
 * -1 for a NULL pointer or a bad size, -2 for an unsupported K, -4 when the
 * HIP runtime reported an error.
 */
#ifndef Q4G128_DIAG_H
#define Q4G128_DIAG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4DIAG_API __attribute__((visibility("default")))

/* Size in uint32 words of the `out` buffer of the kernels below (their XOR
   checksums; the twin returns -1 on a device whose GEMV grid has more waves). */
Q4DIAG_API int32_t q4diag_out_words(void);

/* Read-only twin of q4g128_gemv for K = 3,072: same arguments, grid and loads
   as the GEMV (weights [n][1536], scales and mins [n][24], x [3072]); writes
   one XOR checksum per wave to out[q4diag_out_words()] instead of y. */
Q4DIAG_API int32_t q4diag_gemv_read_twin(const uint8_t* packed, const uint16_t* scales,
                                         const uint16_t* mins, const uint16_t* x, uint32_t* out,
                                         int64_t n, int64_t k, void* stream);

/* Streaming read of `bytes` (a positive multiple of 16, 16-byte aligned
   src) with 16-byte non-temporal loads, each word read once by a one-shot
   grid of 1,024-thread blocks (two words per thread); a thread writes its
   XOR checksum to out[q4diag_out_words()] only if it equals 0x9E3779B9. */
Q4DIAG_API int32_t q4diag_stream_read(const void* src, int64_t bytes, uint32_t* out, void* stream);

/* An empty kernel on the GEMV's grid. */
Q4DIAG_API int32_t q4diag_empty(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4G128_DIAG_H */
