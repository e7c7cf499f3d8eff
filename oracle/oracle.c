/*
 * Reference dense GEMM on the CPU: C = A.B, row-major, plain C, fp64 accumulation.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is checked
 * against.  Only the tests, the smoke check and the bench's CPU-baseline leg may load
 * it; the GPU library never links, includes or calls it, and it shares no code with
 * the GPU library.
 *
 * What it computes (the plain definition): for every 0 <= i < M, 0 <= j < N,
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 *
 * as stated on "Advanced CUDA features - starting from GEMM" (roofline section,
 * case (4): each C_ij is the sum over k of A_ik * B_kj), on "Kernel optimisation
 * guide" (GEMM optimisation path, Level 1: each output is a running sum over k of
 * A[row*K+k]*B[k*N+col]) and on the "GEMM kernels" memo (first, textbook kernel).
 *
 * Storage: A is M x K with row stride lda (element (i,k) at A[i*lda+k]), B is K x N
 * with row stride ldb, C is M x N with row stride ldc; the pages use packed strides
 * (lda = K, ldb = N, ldc = N) and this generalises them to ld >= row length.
 *
 * Arithmetic: every input is converted exactly to double (binary32, binary16 and
 * bfloat16 values are all exactly representable in binary64), each product of two
 * such values is exact in binary64 (at most 24+24 significant bits), and each element
 * is summed in increasing k in binary64, starting from +0.0.  The only roundings are
 * the K-1 binary64 additions and, for the float output, one final round-to-nearest-even
 * conversion to binary32.  The loop nest is i-k-j, which keeps every element's
 * summation in increasing k, so the result equals the textbook i-j-k loop bit for bit
 * and does not depend on the number of threads.  Build with -ffp-contract=off.
 *
 * Degenerate sizes: M = 0 or N = 0 writes nothing; K = 0 writes +0.0 (empty sum).
 *
 * The file also holds the oracles of the memory-slope probes (a word XOR and a
 * dependent-index walk) and of the row-wise softmax and row sum ("Kernel optimisation
 * guide", sections on softmax optimisation and warp-shuffle reduction), each with its
 * own header below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Subnormals (exponent field 0) are fraction * 2^-24; normals are
 * (1024 + fraction) * 2^(e - 25); exponent field 31 encodes infinities and NaNs. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE 754 binary32 pattern. */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int bad_args(int M, int N, int K, int lda, int ldb, int ldc)
{
    if (M < 0 || N < 0 || K < 0) return 1;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1)) return 1;
    return 0;
}

/* The definition on binary64 operands.  C64 (row stride ldc) receives the binary64
 * sums; C32, if not NULL, receives the same sums rounded once to binary32 (same
 * stride).  Returns 0, or -1 on invalid sizes or strides. */
int oracle_gemm_f64(int M, int N, int K, const double *A, int lda, const double *B, int ldb,
                    double *C64, float *C32, int ldc)
{
    if (bad_args(M, N, K, lda, ldb, ldc)) return -1;
    if (M == 0 || N == 0) return 0;
    int fail = 0;
#pragma omp parallel
    {
        double *r = (double *)malloc(sizeof(double) * (size_t)N);
        if (!r) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < M; ++i) {
            if (!r) continue;
            for (int j = 0; j < N; ++j) r[j] = 0.0;
            const double *arow = A + (size_t)i * lda;
            for (int k = 0; k < K; ++k) {
                const double a = arow[k];
                const double *brow = B + (size_t)k * ldb;
                for (int j = 0; j < N; ++j) r[j] += a * brow[j];
            }
            double *c64 = C64 + (size_t)i * ldc;
            for (int j = 0; j < N; ++j) c64[j] = r[j];
            if (C32) {
                float *c32 = C32 + (size_t)i * ldc;
                for (int j = 0; j < N; ++j) c32[j] = (float)r[j];
            }
        }
        free(r);
    }
    return fail ? -1 : 0;
}

/* Widen a rows x cols block with row stride ld into a packed binary64 array. */
typedef double (*decode_fn)(const void *base, size_t idx);

static double dec_f32(const void *p, size_t i) { return (double)((const float *)p)[i]; }
static double dec_f16(const void *p, size_t i) { return oracle_f16_to_f64(((const uint16_t *)p)[i]); }
static double dec_bf16(const void *p, size_t i) { return oracle_bf16_to_f64(((const uint16_t *)p)[i]); }

static double *widen(const void *src, int rows, int cols, int ld, decode_fn dec)
{
    size_t n = (size_t)rows * (size_t)cols;
    double *out = (double *)malloc(sizeof(double) * (n ? n : 1));
    if (!out) return NULL;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            out[(size_t)r * cols + c] = dec(src, (size_t)r * ld + c);
    return out;
}

static int gemm_typed(int M, int N, int K, const void *A, int lda, const void *B, int ldb,
                      double *C64, float *C32, int ldc, decode_fn dec)
{
    if (bad_args(M, N, K, lda, ldb, ldc)) return -1;
    if (M == 0 || N == 0) return 0;
    double *a = widen(A, M, K, lda, dec);
    double *b = widen(B, K, N, ldb, dec);
    int rc = -1;
    if (a && b)
        rc = oracle_gemm_f64(M, N, K, a, K > 0 ? K : 1, b, N, C64, C32, ldc);
    free(a);
    free(b);
    return rc;
}

/* FP32 operands. */
int oracle_gemm_f32(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                    double *C64, float *C32, int ldc)
{
    return gemm_typed(M, N, K, A, lda, B, ldb, C64, C32, ldc, dec_f32);
}

/* IEEE binary16 operands given as bit patterns. */
int oracle_gemm_f16(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B, int ldb,
                    double *C64, float *C32, int ldc)
{
    return gemm_typed(M, N, K, A, lda, B, ldb, C64, C32, ldc, dec_f16);
}

/* bfloat16 operands given as bit patterns. */
int oracle_gemm_bf16(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B, int ldb,
                     double *C64, float *C32, int ldc)
{
    return gemm_typed(M, N, K, A, lda, B, ldb, C64, C32, ldc, dec_bf16);
}

/* ------------------------------------------------------------------------------------
 * The operation of the tensor-core instruction table of "Advanced CUDA features -
 * starting from GEMM" (its warp-group MMA row: D = A*B + D, A and B optionally
 * transposed or negated, D scaled by 0 or 1), written out:
 *
 *     C[i][j] = s * sum_k op(A)[i][k] op(B)[k][j]  (+ Cin[i][j] when accumulate)
 *
 * op(A) is the stored M x K matrix A, or (trans_a) the transpose of the stored K x M
 * matrix: op(A)[i][k] = A[k*lda + i]; op(B) is the stored K x N matrix or (trans_b) the
 * transpose of the stored N x K matrix: op(B)[k][j] = B[j*ldb + k].  s = -1 when
 * exactly one of neg_a, neg_b is nonzero, else +1.  The sum is taken in binary64 by
 * oracle_gemm_f64 on op(A), op(B) widened exactly; then s * sum + Cin in binary64; C32
 * is that value rounded once to binary32.  Cin (binary32, row stride ldc) is read only
 * when accumulate.  dtype: 0 binary32, 1 binary16 bits, 2 bfloat16 bits.
 */

/* op(X) as a packed rows x cols binary64 array: element (r, c) of the stored matrix
 * (row stride ld), or of its transpose when trans. */
static double *widen_op(const void *src, int rows, int cols, int ld, int trans, decode_fn dec)
{
    size_t n = (size_t)rows * (size_t)cols;
    double *out = (double *)malloc(sizeof(double) * (n ? n : 1));
    if (!out) return NULL;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            out[(size_t)r * cols + c] =
                trans ? dec(src, (size_t)c * ld + r) : dec(src, (size_t)r * ld + c);
    return out;
}

int oracle_gemm_ex(int dtype, int trans_a, int trans_b, int neg_a, int neg_b, int accumulate,
                   int M, int N, int K, const void *A, int lda, const void *B, int ldb,
                   const float *Cin, double *C64, float *C32, int ldc)
{
    decode_fn dec = dtype == 0 ? dec_f32 : dtype == 1 ? dec_f16 : dtype == 2 ? dec_bf16 : NULL;
    if (!dec || M < 0 || N < 0 || K < 0) return -1;
    const int min_lda = trans_a ? M : K, min_ldb = trans_b ? K : N;
    if (lda < (min_lda > 1 ? min_lda : 1) || ldb < (min_ldb > 1 ? min_ldb : 1) ||
        ldc < (N > 1 ? N : 1))
        return -1;
    if (M == 0 || N == 0) return 0;
    if (accumulate && !Cin) return -1;
    double *a = widen_op(A, M, K, lda, trans_a, dec);
    double *b = widen_op(B, K, N, ldb, trans_b, dec);
    int rc = -1;
    if (a && b)
        rc = oracle_gemm_f64(M, N, K, a, K > 0 ? K : 1, b, N, C64, NULL, ldc);
    free(a);
    free(b);
    if (rc != 0) return rc;
    const double s = ((neg_a != 0) != (neg_b != 0)) ? -1.0 : 1.0;
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < N; ++j) {
            double v = s * C64[(size_t)i * ldc + j];
            if (accumulate) v += (double)Cin[(size_t)i * ldc + j];
            C64[(size_t)i * ldc + j] = v;
            if (C32) C32[(size_t)i * ldc + j] = (float)v;
        }
    return 0;
}

/*
 * Rounding of a binary64 value to binary16 or bfloat16, to nearest with ties to even,
 * once (never through binary32).  A format with p significant bits and smallest normal
 * exponent emin represents, near v, the multiples of 2^q with q = max(e, emin) - p + 1,
 * e the exponent of v's leading bit; v * 2^-q is exact (a power-of-two scaling), and
 * nearbyint rounds it to an integer with ties to even (the default rounding mode).
 * binary16: p = 11, emin = -14, largest finite 65504; bfloat16: p = 8, emin = -126,
 * largest finite (2 - 2^-7) 2^127.  Results beyond the largest finite value become
 * infinity, as rounding to nearest requires.
 */
static double round_to_format(double v, int p, int emin)
{
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    frexp(v, &e); /* |v| = f 2^e with 0.5 <= f < 1: the leading bit is 2^(e-1) */
    int lead = e - 1;
    if (lead < emin) lead = emin;
    const int q = lead - (p - 1);
    return ldexp(nearbyint(ldexp(v, -q)), q);
}

static uint16_t encode16(double v, int p, int emin, int ebias, double maxfin, uint16_t inf,
                         uint16_t nan)
{
    if (isnan(v)) return nan;
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    const double r = fabs(round_to_format(v, p, emin));
    if (r > maxfin) return sign | inf;
    if (r == 0.0) return sign;
    int e;
    frexp(r, &e);
    const int lead = e - 1;
    if (lead < emin) /* subnormal: the fraction field counts multiples of 2^(emin-p+1) */
        return sign | (uint16_t)ldexp(r, p - 1 - emin);
    const uint16_t frac = (uint16_t)(ldexp(r, p - 1 - lead) - ldexp(1.0, p - 1));
    return sign | (uint16_t)((lead + ebias) << (p - 1)) | frac;
}

uint16_t oracle_f64_to_f16(double v)
{
    return encode16(v, 11, -14, 15, 65504.0, 0x7C00, 0x7E00);
}

uint16_t oracle_f64_to_bf16(double v)
{
    return encode16(v, 8, -126, 127, ldexp(255.0, 120), 0x7F80, 0x7FC0);
}

/*
 * The general form with C stored in the operands' 16-bit type (dtype 1: binary16,
 * 2: bfloat16): as oracle_gemm_ex, with Cin (when accumulate) read in that type and the
 * binary64 value s * sum (+ Cin) rounded once to it into C16 (bit patterns, row stride
 * ldc).  C64 receives the binary64 values.
 */
int oracle_gemm_ex16(int dtype, int trans_a, int trans_b, int neg_a, int neg_b, int accumulate,
                     int M, int N, int K, const void *A, int lda, const void *B, int ldb,
                     const uint16_t *Cin, double *C64, uint16_t *C16, int ldc)
{
    if (dtype != 1 && dtype != 2) return -1;
    if (accumulate && M > 0 && N > 0 && !Cin) return -1;
    int rc = oracle_gemm_ex(dtype, trans_a, trans_b, neg_a, neg_b, 0, M, N, K, A, lda, B, ldb,
                            NULL, C64, NULL, ldc);
    if (rc != 0) return rc;
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < N; ++j) {
            const size_t at = (size_t)i * ldc + j;
            double v = C64[at];
            if (accumulate)
                v += dtype == 1 ? oracle_f16_to_f64(Cin[at]) : oracle_bf16_to_f64(Cin[at]);
            C64[at] = v;
            C16[at] = dtype == 1 ? oracle_f64_to_f16(v) : oracle_f64_to_bf16(v);
        }
    return 0;
}

/* ------------------------------------------------------------------------------------
 * Memory-slope probes ("Advanced CUDA features - starting from GEMM", section on
 * Little's law and occupancy).  The probes only move data; what they must produce is
 * fixed by definition and written out here.
 */

/* XOR of the n 32-bit words w[0..n). */
uint32_t oracle_xor_words(const uint32_t *w, int64_t n)
{
    uint32_t x = 0;
    for (int64_t i = 0; i < n; ++i) x ^= w[i];
    return x;
}

/* The word index reached from `start` after `hops` dependent steps cur = next[cur] over
 * a table of n words, where a loaded index outside [0, n) is replaced by n - 1. */
uint32_t oracle_chase(const uint32_t *next, int64_t n, uint32_t start, int64_t hops)
{
    uint32_t cur = start;
    for (int64_t h = 0; h < hops; ++h) {
        const uint32_t v = next[cur];
        cur = (int64_t)v < n ? v : (uint32_t)(n - 1);
    }
    return cur;
}

/*
 * Softmax of every row of a rows x cols binary32 matrix (row stride ldx), by the online
 * recurrence of "Kernel optimisation guide" (section on softmax optimisation, the online
 * algorithm), in binary64.
 *
 * One pass over the row keeps a running maximum m (starting at -infinity) and a running
 * sum l (starting at 0) of exp(x - m): when an element exceeds m, the sum so far is
 * rescaled to the new maximum by exp(m_old - x) and m becomes x; then exp(x - m) is
 * added.  After the pass m = max_i x_i and l = sum_i exp(x_i - m).  A second pass writes
 * y_i = exp(x_i - m) / l.  Elements are visited in increasing column order.  The row
 * elements are converted exactly to binary64, so each difference x_i - m is exact; the
 * roundings are those of exp, the additions, the rescaling products and the division.
 *
 * Outputs (each may be NULL): Y64 / Y32 (row stride ldy) the binary64 results and their
 * binary32 roundings (RNE); m_out / l_out the per-row m and l.  cols = 0 writes nothing
 * to Y and m = -infinity, l = 0 per row.  Inputs are expected finite (a leading -infinity
 * would make the first exp(x - m) an exp(NaN), as the recurrence is written).
 */
int oracle_softmax(int rows, int cols, const float *X, int ldx, double *Y64, float *Y32,
                   int ldy, double *m_out, double *l_out)
{
    const int need = cols > 1 ? cols : 1;
    if (rows < 0 || cols < 0 || ldx < need || ldy < need) return 1;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const float *x = X + (size_t)r * ldx;
        double m = -INFINITY;
        double l = 0.0;
        for (int i = 0; i < cols; ++i) {
            const double v = (double)x[i];
            if (v > m) {
                l *= exp(m - v);
                m = v;
            }
            l += exp(v - m);
        }
        for (int i = 0; i < cols; ++i) {
            const double y = exp((double)x[i] - m) / l;
            if (Y64) Y64[(size_t)r * ldy + i] = y;
            if (Y32) Y32[(size_t)r * ldy + i] = (float)y;
        }
        if (m_out) m_out[r] = m;
        if (l_out) l_out[r] = l;
    }
    return 0;
}

/*
 * Sum of every row of a rows x cols binary32 matrix (row stride ldx): the reduction the
 * "Kernel optimisation guide" section on warp-shuffle reduction builds from lane sums.
 * Each row is summed in binary64 in increasing column order from +0.0 (cols = 0 gives
 * +0.0); S64 gets the sums, S32 (may be NULL) their binary32 roundings (RNE).
 */
int oracle_row_sum(int rows, int cols, const float *X, int ldx, double *S64, float *S32)
{
    if (rows < 0 || cols < 0 || ldx < (cols > 1 ? cols : 1)) return 1;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const float *x = X + (size_t)r * ldx;
        double s = 0.0;
        for (int i = 0; i < cols; ++i) s += (double)x[i];
        if (S64) S64[r] = s;
        if (S32) S32[r] = (float)s;
    }
    return 0;
}
