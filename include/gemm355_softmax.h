/*
 * libgemm355 row-wise softmax and row sum (binary32).
 *
 * "Kernel optimisation guide" (section on softmax optimisation, the online algorithm)
 * computes the softmax of a vector in one pass for its statistics: a running maximum m
 * and a running sum l of exp(x - m), the sum rescaled by exp(m_old - m_new) whenever the
 * maximum rises, followed by a pass that writes exp(x_i - m) / l.  Its section on
 * warp-shuffle reduction sums a value over the lanes of a warp by exchanging registers
 * between lanes.  These entry points apply both to every row of a matrix on the GPU:
 * each row is held on chip while its statistics are reduced across the 64 lanes of a
 * wave and across the waves of a workgroup, so it is read from memory once (rows of
 * more than 32768 elements are read twice).
 *
 * Layout: X and Y are rows x cols, row-major, row strides ldx and ldy in elements
 * (element (r, c) at X[r * ldx + c]).  All pointers are device pointers owned by the
 * caller; work is enqueued on `stream` and the call returns at once.  Nothing is
 * allocated.
 *
 * Errors: argument errors are detected on the host before any HIP call and return
 * GEMM355_ERR_INVALID_ARG; a current device that is not a gfx950 returns
 * GEMM355_ERR_DEVICE; a failed launch returns GEMM355_ERR_LAUNCH.
 */
#ifndef GEMM355_SOFTMAX_H
#define GEMM355_SOFTMAX_H

#include "gemm355.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Y[r][c] = exp(X[r][c] - m_r) / l_r for every 0 <= r < rows, 0 <= c < cols, with
 * m_r = max_c X[r][c] and l_r = sum_c exp(X[r][c] - m_r) (the online softmax above).
 *
 * Results agree with the exact softmax of the binary32 inputs to a relative error below
 * 2^-24 (2 |X[r][c] - m_r| + 2 n + 64), n the number of elements one lane sums in
 * sequence (at most 64 for rows of up to 32768 elements, cols / 1024 beyond): the
 * rounding of X - m dominates for elements far below the maximum.  Inputs are expected finite; an infinity or NaN in a row makes
 * that row's results unspecified (other rows are unaffected).
 *
 * Arguments: 0 <= rows <= 2^30, 0 <= cols <= 2^30; ldx >= max(1, cols), ldy >= max(1, cols);
 * X and Y non-null unless rows * cols == 0; Y may equal X (in place) when ldy == ldx,
 * any other overlap of the two matrices' spans is an argument error.  rows == 0 or
 * cols == 0 is a no-op.  Elements of Y outside the rows x cols region are not written. */
gemm355_status gemm355_softmax_f32(int rows, int cols, const float *X, int ldx, float *Y,
                                   int ldy, hipStream_t stream);

/* out[r] = sum_c X[r][c] for every 0 <= r < rows (cols == 0 gives +0.0).  The lanes'
 * partial sums are combined by register exchanges within each wave, then across the
 * wave's workgroup, in a fixed order, so repeated calls give identical bits; the result
 * agrees with the exact sum to within about (cols / (64 * waves per row) + 12) * 2^-24
 * times the sum of the magnitudes (sums of small integers are exact).
 *
 * Arguments: 0 <= rows <= 2^30, 0 <= cols <= 2^30, ldx >= max(1, cols); X non-null unless
 * rows * cols == 0; out (rows binary32 values) non-null unless rows == 0, and not
 * overlapping X's span. */
gemm355_status gemm355_row_sum_f32(int rows, int cols, const float *X, int ldx, float *out,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM355_SOFTMAX_H */
