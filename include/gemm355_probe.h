/*
 * libgemm355 diagnostics: lane-layout probes of the gfx950 instructions the kernels
 * are built on.  "Advanced CUDA features - starting from GEMM" (tensor-core section,
 * register layout) stresses that a matrix unit expects its operands spread over the
 * lanes of a wave in a fixed layout, and that getting that layout right is the hard
 * part; these entry points run the instructions on caller-chosen lane data so tests
 * can pin the layouts on the device instead of relying on documentation.
 *
 * All pointers named dev_* are device pointers owned by the caller; work is enqueued
 * on `stream`.  Arguments are validated on the host first (GEMM355_ERR_INVALID_ARG);
 * GEMM355_ERR_DEVICE if the current device is not gfx950.
 */
#ifndef GEMM355_PROBE_H
#define GEMM355_PROBE_H

#include <stdint.h>

#include "gemm355.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Instruction kinds for gemm355_probe_mfma: operand elements per lane E and
 * accumulator registers per lane R.
 *   0  v_mfma_f32_32x32x2_f32    E=1 R=16      1  v_mfma_f32_16x16x4_f32    E=1 R=4
 *   2  v_mfma_f32_32x32x16_f16   E=8 R=16      3  v_mfma_f32_16x16x32_f16   E=8 R=4
 *   4  v_mfma_f32_32x32x16_bf16  E=8 R=16      5  v_mfma_f32_16x16x32_bf16  E=8 R=4 */
int gemm355_probe_mfma_shape(int kind, int *elems_per_lane, int *regs_per_lane);

/* Runs `nruns` independent single-wave MFMAs of `kind` with zero initial accumulators.
 * Run r, lane l, element e takes its A operand from dev_a[(r*64 + l)*E + e] and its B
 * operand from dev_b[(r*64 + l)*E + e] (FP32 values, rounded to FP16/BF16 for kinds
 * 2..5); accumulator register i of lane l is written to dev_d[(r*64 + l)*R + i].
 * 1 <= nruns <= 65535. */
gemm355_status gemm355_probe_mfma(int kind, int nruns, const float *dev_a, const float *dev_b,
                                  float *dev_d, hipStream_t stream);

/* Fills a 4096-byte LDS array with the 16-bit values 0, 1, ..., 2047 (halfword i holds
 * i), then lane l executes ds_read_b64_tr_b16 at byte address host_addr[l] (a host
 * array of 64 entries, each a multiple of 8 and at most 4088).  The four 16-bit results
 * of lane l are written to dev_out[4*l .. 4*l+3]. */
gemm355_status gemm355_probe_ds_read_tr16(const uint32_t *host_addr, uint16_t *dev_out,
                                          hipStream_t stream);

/* One wave: lane l executes global_load_lds_dwordx4 from dev_src + 4*host_src_chunk[l]
 * (16-byte chunks of a caller buffer of at least 4*(max chunk + 1) 32-bit words) into a
 * 2 KiB LDS array zero-filled beforehand, with a wave-uniform LDS base of byte
 * lds_base (a multiple of 16, at most 1024); after a barrier the whole 2 KiB array is
 * copied to dev_out (512 words).  host_src_chunk is a host array of 64 entries, each
 * at most 4095. */
gemm355_status gemm355_probe_global_load_lds(const uint32_t *dev_src, const uint32_t *host_src_chunk,
                                             uint32_t lds_base, uint32_t *dev_out,
                                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM355_PROBE_H */
