/*
 * libgemm355 -- dense general matrix multiply C = A.B on AMD Instinct MI355X (gfx950).
 *
 * The operation (the definition used throughout "Advanced CUDA features - starting
 * from GEMM", roofline section, case (4), and "Kernel optimisation guide", GEMM
 * optimisation path, Level 1):
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j],   0 <= i < M, 0 <= j < N
 *
 * Layout: all matrices are row-major with explicit leading dimensions (row strides,
 * in elements): element (i,k) of A is A[i*lda + k], element (k,j) of B is
 * B[k*ldb + j], element (i,j) of C is C[i*ldc + j].  The pages use packed strides
 * (lda = K, ldb = N, ldc = N); any stride at least the row length is accepted.
 *
 * Result: C is overwritten (no alpha/beta).  Accumulation is in FP32.  FP16 and BF16
 * operands are multiplied exactly and summed in FP32.  Only C[0..M) x [0..N) is
 * written; padding columns N..ldc-1 and memory outside the logical matrices are
 * never read (A, B) or written (C).
 *
 * Ownership: every pointer is a device pointer owned by the caller; the library
 * allocates nothing, keeps no per-call state and needs no workspace.  A and B are
 * read-only.  C must not overlap A or B.
 *
 * Asynchrony: the work is enqueued on `stream` (NULL = the null stream) and the call
 * returns without waiting.  Faults during execution surface at the caller's next
 * synchronisation on that stream.
 *
 * Errors (returned, never aborting the process):
 *   GEMM355_ERR_INVALID_ARG  any dimension < 0; lda < max(1,K), ldb < max(1,N) or
 *                            ldc < max(1,N); a NULL pointer for a matrix with a
 *                            nonzero number of elements; unknown variant or dtype.
 *                            Detected on the host before any HIP call.
 *   GEMM355_ERR_DEVICE       no current HIP device, or it is not gfx950.
 *   GEMM355_ERR_LAUNCH       the kernel launch was rejected by the runtime.
 *   GEMM355_ERR_UNSUPPORTED  the forced variant does not exist for this dtype.
 * Degenerate shapes: M = 0 or N = 0 is a no-op returning GEMM355_OK; K = 0 writes
 * +0.0 to every element of C (the empty sum).
 *
 * Thread safety: calls may be made from several host threads; the only shared state
 * is the cached per-device architecture check.
 */
#ifndef GEMM355_H
#define GEMM355_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same declaration as HIP's own: an opaque stream handle. */
typedef struct ihipStream_t *hipStream_t;

typedef enum gemm355_status {
    GEMM355_OK = 0,
    GEMM355_ERR_INVALID_ARG = 1,
    GEMM355_ERR_DEVICE = 2,
    GEMM355_ERR_LAUNCH = 3,
    GEMM355_ERR_UNSUPPORTED = 4
} gemm355_status;

/* Operand storage types.  FP16 is IEEE binary16, BF16 is bfloat16; both are passed
 * as 16-bit patterns (uint16_t). */
typedef enum gemm355_dtype {
    GEMM355_F32 = 0,
    GEMM355_F16 = 1,
    GEMM355_BF16 = 2
} gemm355_dtype;

/* Kernel families.  NAIVE: one thread per element of C, every operand read from
 * global memory ("Kernel optimisation guide", Level 1).  LDS_TILED: A and B tiles
 * staged in local data share and reused across a workgroup ("Advanced CUDA
 * features", Shared Memory Tiling).  REGBLOCK: FP32 on the vector ALUs with a per-
 * thread register micro-tile and a double-buffered LDS pipeline (same page, Register
 * Tiling; "Kernel optimisation guide", Level 3).  MFMA: the matrix cores (the AMD
 * counterpart of the tensor-core level, "Kernel optimisation guide", Level 4), for
 * FP32 (v_mfma_f32_32x32x2_f32) and FP16/BF16 with FP32 accumulation. */
typedef enum gemm355_variant {
    GEMM355_VARIANT_AUTO = -1,
    GEMM355_VARIANT_NAIVE = 0,
    GEMM355_VARIANT_LDS_TILED = 1,
    GEMM355_VARIANT_REGBLOCK = 2,
    GEMM355_VARIANT_MFMA = 3,
    /* Other schedules of the FP16/BF16 direct-to-LDS kernel, kept to measure them against
     * the dispatched one (plain products of F16 / BF16 operands only; any other dtype,
     * gemm355_gemm_ex flag or a shape the kernel does not take returns
     * GEMM355_ERR_UNSUPPORTED).  Shapes taken: whole tiles (M a multiple of 256, N of
     * the tile width), 16-byte-aligned rows, K a multiple of 128 (MFMA_T256X256 and
     * MFMA_STAGED128 and MFMA_STAGED_SMALL: any shape and gemm355_gemm_ex flags).
     * MFMA_SPLIT: wave specialisation ("Advanced CUDA features - starting from GEMM",
     *   scheduling section, the warp-specialisation path): 256 x 128 tiles, four producer
     *   waves issue every global -> LDS load while four compute waves (128 x 64 of C
     *   each) only read fragments and multiply; one barrier per k-step hands the stages
     *   over.
     * MFMA_W8: 256 x 256 tiles on eight waves, two per SIMD (128 x 64 of C each), every
     *   wave loading its share beside its MFMAs.
     * MFMA_T256X128: 256 x 128 tiles on four waves (128 x 64 of C each), every wave
     *   loading: twice as many tiles, so a CU's second tile starts while the first one's
     *   stores drain.
     * MFMA_T256X256: the dispatched kernels with the 192 x 256 and 256 x 192
     *   direct-to-LDS tiles turned off: the 256 x 256 tile wherever the dispatcher would
     *   take one of them, every other call as dispatched (any F16 / BF16 product the
     *   dispatcher takes, gemm355_gemm_ex flags included; the same results bit for bit,
     *   since every tile sums each element's K products in the same order).
     * MFMA_STAGED128: the dispatched kernels with the two-per-CU 128 x 128 direct-to-LDS
     *   tile turned off: grids of more than 256 128-wide tiles go to the register-staged
     *   kernel, every other call as dispatched (any F16 / BF16 product the dispatcher
     *   takes, gemm355_gemm_ex flags included).
     * MFMA_STAGED_SMALL: the dispatched kernels with the direct-to-LDS tiles of small
     *   grids turned off: no 64 x 64 direct-to-LDS tile, no 4-stage ring for K from 128
     *   to 255 on tiles that otherwise take the 8-stage one, and plain products whose
     *   128 x 128 grid leaves CUs idle on the register-staged 128 x 64 and 64 x 64 tiles;
     *   every other call as dispatched (any F16 / BF16 product the dispatcher takes,
     *   gemm355_gemm_ex flags included). */
    GEMM355_VARIANT_MFMA_SPLIT = 4,
    GEMM355_VARIANT_MFMA_W8 = 5,
    GEMM355_VARIANT_MFMA_T256X128 = 6,
    GEMM355_VARIANT_MFMA_T256X256 = 7,
    GEMM355_VARIANT_MFMA_STAGED128 = 8,
    GEMM355_VARIANT_MFMA_STAGED_SMALL = 9
} gemm355_variant;

/* C = A.B with FP32 operands and FP32 accumulation. */
gemm355_status gemm_f32(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                        float *C, int ldc, hipStream_t stream);

/* C = A.B with IEEE binary16 operands (bit patterns), exact products, FP32 accumulation
 * and FP32 output. */
gemm355_status gemm_f16f32acc(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B,
                              int ldb, float *C, int ldc, hipStream_t stream);

/* C = A.B with bfloat16 operands (bit patterns), exact products, FP32 accumulation and
 * FP32 output. */
gemm355_status gemm_bf16f32acc(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B,
                               int ldb, float *C, int ldc, hipStream_t stream);

/* The same contract with the kernel family chosen by the caller (`variant`, one of
 * gemm355_variant; AUTO picks as the typed entry points do) and the operand type given
 * by `dtype` (one of gemm355_dtype).  Available: NAIVE for all dtypes; LDS_TILED and
 * REGBLOCK for F32; MFMA for all dtypes.  Used to measure and test each family. */
gemm355_status gemm355_run_variant(int variant, int dtype, int M, int N, int K, const void *A,
                                   int lda, const void *B, int ldb, float *C, int ldc,
                                   hipStream_t stream);

/* Operand forms of gemm355_gemm_ex (bit flags).  The tensor-core instruction table of
 * "Advanced CUDA features - starting from GEMM" lists, for its warp-group MMA, D = A*B + D
 * with transposed or negated A and B and D scaled by 0 or 1; these flags provide that
 * operation on top of the same kernels.  The table does not state D's type;
 * GEMM355_C_16 adds the choice of keeping C in the operands' 16-bit type. */
enum {
    GEMM355_TRANS_A = 1,     /* op(A) = A^T: A is stored K x M (element (k,i) at A[k*lda+i]) */
    GEMM355_TRANS_B = 2,     /* op(B) = B^T: B is stored N x K (element (j,k) at B[j*ldb+k]) */
    GEMM355_NEG_A = 4,       /* use -op(A) */
    GEMM355_NEG_B = 8,       /* use -op(B) */
    GEMM355_ACCUMULATE = 16, /* D scaled by 1 (C += ...) instead of 0 (C = ...) */
    GEMM355_C_16 = 32        /* C (and the old C) in the operands' 16-bit type, see below */
};

/* C = (+-op(A)) (+-op(B)) [+ C]:
 *
 *     C[i][j] = s * sum_k op(A)[i][k] op(B)[k][j]  (+ C[i][j] when GEMM355_ACCUMULATE)
 *
 * with s = -1 when exactly one of GEMM355_NEG_A, GEMM355_NEG_B is set, else +1, op(A)
 * M x K and op(B) K x N.  Leading dimensions are those of the stored matrices: lda >=
 * max(1, K) (max(1, M) with GEMM355_TRANS_A), ldb >= max(1, N) (max(1, K) with
 * GEMM355_TRANS_B), ldc >= max(1, N).  `variant` and `dtype` as for gemm355_run_variant;
 * with any flag set only NAIVE, MFMA and AUTO (= MFMA) are available (others return
 * GEMM355_ERR_UNSUPPORTED).  Unknown flag bits are GEMM355_ERR_INVALID_ARG.
 * Accumulation: every kernel adds s * (its FP32 sum) to the old C in its epilogue, one
 * rounding.  K = 0: C = s * (+0.0) without GEMM355_ACCUMULATE, C unchanged with it.
 * C type: C is binary32 (`C` points to float, ldc counts floats), or with GEMM355_C_16
 * and dtype GEMM355_F16 / GEMM355_BF16 it is stored in that same 16-bit format (`C`
 * points to uint16_t patterns, ldc counts them): each result is the binary32 value
 * s * sum (+ old C widened to binary32) rounded to nearest with ties to even (FP32
 * accumulation, 16-bit storage).  GEMM355_C_16 with dtype GEMM355_F32 is
 * GEMM355_ERR_INVALID_ARG.
 * Everything else (ownership, asynchrony, errors) as for gemm_f32. */
gemm355_status gemm355_gemm_ex(int variant, int dtype, unsigned flags, int M, int N, int K,
                               const void *A, int lda, const void *B, int ldb, void *C, int ldc,
                               hipStream_t stream);

/* Host-only: the family the typed entry points would launch for these arguments, or -1
 * if the arguments are invalid.  Makes no HIP call. */
int gemm355_select_variant(int dtype, int M, int N, int K, const void *A, int lda, const void *B,
                           int ldb, const float *C, int ldc);

/* Host-only: a NUL-terminated description of the kernel instance (family, tile shape,
 * load path; for the register-staged 16-bit kernel also its launches: one launch over
 * every tile, or an interior launch and the ragged strips, with their load mode and
 * whether the two-set pipeline runs) that gemm355_run_variant would launch, or
 * "invalid".  Makes no HIP call.  The string is owned by the library and stays valid
 * until the next call of gemm355_kernel_desc or gemm355_kernel_desc_ex on the same
 * thread. */
const char *gemm355_kernel_desc(int variant, int dtype, int M, int N, int K, const void *A, int lda,
                                const void *B, int ldb, const float *C, int ldc);

/* Host-only: the same for gemm355_gemm_ex with operand forms `flags`; "invalid" where
 * gemm355_gemm_ex would return an error status before launching. */
const char *gemm355_kernel_desc_ex(int variant, int dtype, unsigned flags, int M, int N, int K,
                                   const void *A, int lda, const void *B, int ldb, const void *C,
                                   int ldc);

/* Host-only: static strings for status codes and variants ("unknown" otherwise). */
const char *gemm355_status_string(int status);
const char *gemm355_variant_name(int variant);

/* Library version as major*10000 + minor*100 + patch. */
int gemm355_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM355_H */
