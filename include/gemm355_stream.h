/*
 * libgemm355 memory-slope probes.
 *
 * "Advanced CUDA features - starting from GEMM" (section on Little's law and occupancy)
 * states that keeping DRAM busy takes a fixed number of bytes in flight, latency times
 * bandwidth (its worked example: 800 cycles x 165.52 bytes/cycle, about 132 KB), that
 * the resident warps that carry them can be limited through each block's shared-memory
 * allocation, that a memory-bound copy reaches peak bandwidth at 33-50 % occupancy,
 * and that wider per-thread accesses (float4) reach it at lower occupancy.  These entry
 * points let those statements be measured on an MI355X: a streaming kernel whose bytes
 * in flight per wave and resident waves per CU the caller sets, and a dependent-load
 * chase that measures the latency those bytes have to cover.
 *
 * All pointers are device pointers owned by the caller; work is enqueued on `stream`.
 * Arguments are validated on the host before any HIP call (GEMM355_ERR_INVALID_ARG);
 * GEMM355_ERR_DEVICE if the current device is not gfx950; GEMM355_ERR_LAUNCH if the
 * launch fails.  Nothing is allocated.
 */
#ifndef GEMM355_STREAM_H
#define GEMM355_STREAM_H

#include <stdint.h>

#include "gemm355.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GEMM355_STREAM_COPY = 0,     /* dst[0, n_bytes) = src[0, n_bytes) */
    GEMM355_STREAM_READ_XOR = 1, /* dst[g] = XOR of the 32-bit words workgroup g read */
    GEMM355_STREAM_COPY_NT = 2   /* as COPY, with non-temporal stores (no L2 lines allocated
                                    for dst), to measure the store cache policy */
};

/* Streams n_bytes of src through `grid` workgroups of `threads` threads.
 *
 * The source is cut into chunks of threads * vec_bytes * unroll bytes, handed to the
 * workgroups round-robin (chunk c to workgroup c mod grid).  For each chunk every lane
 * first issues its `unroll` loads of vec_bytes (lane t, load u reads the chunk's bytes
 * [(u * threads + t) * vec_bytes, +vec_bytes), so every load instruction is
 * contiguous across the wave), then consumes them: modes COPY and COPY_NT store them to
 * the same offsets of dst, mode READ_XOR folds their 32-bit words into a running XOR.  The
 * 32-bit words after the last whole chunk are handled one word per thread.  Each
 * workgroup also reserves lds_bytes of LDS that it does not otherwise use: at most
 * floor(163840 / lds_bytes) workgroups (and the hardware's own limits) are resident
 * per CU, which is how the caller sets occupancy.  Bytes in flight per wave at the
 * start of a chunk are 64 * vec_bytes * unroll.
 *
 * mode READ_XOR: dst is a uint32 array of `grid` entries; entry g is the XOR of every
 * word workgroup g read, so the XOR of all entries is the XOR of the whole source
 * (which workgroup reads which word depends on grid and threads, the total does not).
 *
 * Arguments: mode COPY, COPY_NT or READ_XOR; n_bytes >= 0 and a multiple of 4; src and
 * (copy modes) dst aligned to vec_bytes, dst aligned to 4 in mode READ_XOR; vec_bytes 4, 8 or
 * 16; unroll 1, 2, 4 or 8; threads a multiple of 64 in [64, 1024]; 0 <= lds_bytes <=
 * 163840; 1 <= grid <= 1048576; src and dst must not overlap; src, dst non-null when
 * they are used (dst always in mode READ_XOR). */
gemm355_status gemm355_stream(int mode, const void *src, void *dst, int64_t n_bytes,
                              int vec_bytes, int unroll, int threads, int lds_bytes, int grid,
                              hipStream_t stream);

/* Dependent-load latency.  One lane starts at word index `start` of `next` (n_words
 * 32-bit words) and performs `hops` dependent loads cur = next[cur]; a loaded index
 * outside [0, n_words) is replaced by n_words - 1 before it is used, so every read is
 * in bounds whatever the buffer holds.  dev_out (two 64-bit words) receives the final
 * index and the shader-clock cycles (s_memtime) the hops took.
 * Arguments: 1 <= n_words <= 2^32; start < n_words; 1 <= hops <= 2^30; next and
 * dev_out non-null. */
gemm355_status gemm355_chase(const uint32_t *next, int64_t n_words, uint32_t start, int hops,
                             uint64_t *dev_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM355_STREAM_H */
