// Register-blocked FP32 GEMM on the vector ALUs: each thread accumulates an 8 x 8
// micro-tile of C in registers, fed from LDS tiles that are double-buffered against
// the global loads of the next k-step.
//
// This is the thread-level reuse of "Advanced CUDA features - starting from GEMM"
// (section "Register Tiling": every thread owns a micro-block of accumulators, loads a
// column of A values and a row of B values from shared memory per k and performs all
// their pairwise multiply-adds, so shared-memory reads per FMA drop from 2 to 1/4),
// with the double buffer of "Kernel optimisation guide" (Level 3) and the 2 x 2
// coarsening of the "GEMM kernels" memo generalised to 8 x 8.
//
// gfx950 mapping (256 threads, 128 x 128 tile of C, BK = 16):
//  * thread t = 16 ty + tx owns rows {4ty..4ty+3, 64+4ty..64+4ty+3} and columns
//    {4tx..4tx+3, 64+4tx..64+4tx+3}: split 4 + 4 so every operand read is one
//    ds_read_b128, and a wave's B reads cover 256 contiguous bytes (no bank conflict)
//    while its A reads touch four addresses (broadcast);
//  * A is stored k-major in LDS (transposed on the way in: four ds_write_b32 per
//    loaded dwordx4, lanes arranged so that each write hits distinct banks), B as
//    loaded; A rows are padded to 132 words;
//  * 64 v_fma_f32 per 4 ds_read_b128 per k; accumulation is fmaf in increasing k from
//    +0.0, so every element rounds exactly as in the naive and LDS-tiled kernels.
// The vector ALU peaks at 128 FP32 FLOP/clk/CU with unpacked FMA (packed FP32 math is
// not used by this library), half of the chip's 157.3 TFLOP/s FP32 figure.
#include "common.hpp"
#include "launch.hpp"

namespace g355 {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 16, kThreads = 256;
constexpr int kSA = kBM + 4;  // A (k-major) LDS row stride, words
constexpr int kSB = kBN;      // B LDS row stride, words
constexpr int kLdsA = kBK * kSA, kLdsB = kBK * kSB;
constexpr int kAChunks = kBM * kBK / 4 / kThreads;  // 2
constexpr int kBChunks = kBK * kBN / 4 / kThreads;  // 2

template <bool VEC>
__device__ __forceinline__ floatx4 ld4(const float *__restrict__ row, int c, int ncols, bool row_ok,
                                       bool full) {
    if (full) {
        if (VEC) return *reinterpret_cast<const floatx4 *>(row + c);
        return floatx4{row[c], row[c + 1], row[c + 2], row[c + 3]};
    }
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (!row_ok) return v;
    if (VEC && c + 4 <= ncols) return *reinterpret_cast<const floatx4 *>(row + c);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (c + e < ncols) v[e] = row[c + e];
    return v;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void regblock_f32_kernel(int M, int N, int K, const float *__restrict__ A, int lda,
                         const float *__restrict__ B, int ldb, float *__restrict__ C, int ldc) {
    __shared__ __attribute__((aligned(16))) float lds[2 * (kLdsA + kLdsB)];

    const int tiles_m = cdiv(M, kBM), tiles_n = cdiv(N, kBN);
    int tm, tn;
    grouped_tile(xcd_contiguous_id(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const bool tile_full = (m0 + kBM <= M) && (n0 + kBN <= N);

    const int t = threadIdx.x;
    const int tx = t % 16, ty = t / 16;

    int a_r[kAChunks], a_c[kAChunks], b_r[kBChunks], b_c[kBChunks];
    // A chunks: 64 consecutive q (one wave's instruction) cover 16 rows x 4 chunks, so
    // each row's 64 bytes are read by one instruction.  Within each 32-lane half the rows
    // are arranged so that its four ds_write_b32 of the transposed store hit 32 distinct
    // banks: with the 132-word stride lane (row r, chunk j) writes word (4 j + e) 132 + r,
    // bank (16 j + 4 e + r) mod 32, and the half puts rows 0-7 under chunks {0, 1} and rows
    // 8-15 under chunks {2, 3} (the other half the opposite).  Consecutive rows under every
    // chunk (q / 4) gave two lanes per bank, 16 conflict cycles per wave per k-step.
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
        const int q = t + kThreads * i;
        const int l = q % 64, j = l % 4;
        a_r[i] = 16 * (q / 64) + (l % 32) / 4 + 8 * ((j / 2) ^ (l / 32));
        a_c[i] = 4 * j;
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
        const int q = t + kThreads * i;
        b_r[i] = q / (kBN / 4);
        b_c[i] = (q % (kBN / 4)) * 4;
    }

    floatx4 sa[kAChunks], sb[kBChunks];
    auto load_tile = [&](int k0) {
        const bool full = tile_full && (k0 + kBK <= K);
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int r = m0 + a_r[i];
            const bool ok = r < M;
            sa[i] = ld4<VEC>(A + (size_t)(ok ? r : 0) * lda, k0 + a_c[i], K, ok, full);
        }
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) {
            const int r = k0 + b_r[i];
            const bool ok = r < K;
            sb[i] = ld4<VEC>(B + (size_t)(ok ? r : 0) * ldb, n0 + b_c[i], N, ok, full);
        }
    };
    auto store_tile = [&](int buf) {
        float *As = lds + buf * (kLdsA + kLdsB);
        float *Bs = As + kLdsA;
#pragma unroll
        for (int i = 0; i < kAChunks; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) As[(a_c[i] + e) * kSA + a_r[i]] = sa[i][e];
#pragma unroll
        for (int i = 0; i < kBChunks; ++i)
            *reinterpret_cast<floatx4 *>(Bs + b_r[i] * kSB + b_c[i]) = sb[i];
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    const int nk = cdiv(K, kBK);
    if (nk > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tile((kt + 1) * kBK);
        const float *As = lds + buf * (kLdsA + kLdsB);
        const float *Bs = As + kLdsA;
#pragma unroll 4
        for (int k = 0; k < kBK; ++k) {
            const floatx4 a0 = *reinterpret_cast<const floatx4 *>(As + k * kSA + 4 * ty);
            const floatx4 a1 = *reinterpret_cast<const floatx4 *>(As + k * kSA + 64 + 4 * ty);
            const floatx4 b0 = *reinterpret_cast<const floatx4 *>(Bs + k * kSB + 4 * tx);
            const floatx4 b1 = *reinterpret_cast<const floatx4 *>(Bs + k * kSB + 64 + 4 * tx);
            const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < nk) store_tile(buf ^ 1);
        __syncthreads();
    }

    const bool vec_store = tile_full && ((uintptr_t)C % 16 == 0) && (ldc % 4 == 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + i - 4);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = n0 + 64 * h + 4 * tx;
            float *dst = C + (size_t)row * ldc + col;
            if (vec_store) {
                *reinterpret_cast<floatx4 *>(dst) =
                    floatx4{acc[i][4 * h], acc[i][4 * h + 1], acc[i][4 * h + 2], acc[i][4 * h + 3]};
            } else if (row < M) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < N) dst[e] = acc[i][4 * h + e];
            }
        }
    }
}

bool rb_vec(const GemmArgs &g) {
    return rows_aligned16(g.A, g.lda, 4) && rows_aligned16(g.B, g.ldb, 4);
}

}  // namespace

const char *desc_regblock_f32(const GemmArgs &g) {
    return rb_vec(g) ? "regblock_f32 128x128x16 8x8/thread dwordx4"
                     : "regblock_f32 128x128x16 8x8/thread dword";
}

hipError_t launch_regblock_f32(const GemmArgs &g, hipStream_t s) {
    const dim3 grid(cdiv(g.M, kBM) * cdiv(g.N, kBN));
    const dim3 block(kThreads);
    if (rb_vec(g))
        hipLaunchKernelGGL(regblock_f32_kernel<true>, grid, block, 0, s, g.M, g.N, g.K,
                           (const float *)g.A, g.lda, (const float *)g.B, g.ldb, g.C, g.ldc);
    else
        hipLaunchKernelGGL(regblock_f32_kernel<false>, grid, block, 0, s, g.M, g.N, g.K,
                           (const float *)g.A, g.lda, (const float *)g.B, g.ldb, g.C, g.ldc);
    return hipGetLastError();
}

}  // namespace g355
