// FP16 / BF16 GEMM with FP32 accumulation on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_f16 / _bf16): the AMD counterpart of the tensor-core level of
// "Kernel optimisation guide" (Level 4: 16-bit A and B fragments, FP32 accumulator
// fragments, a matrix multiply-accumulate per fragment step) and of the tensor-core
// section of "Advanced CUDA features - starting from GEMM" (a wave-cooperative
// D = A.B + C unit whose register layout has to be matched by the data movement).
//
// Structure:
//  * a workgroup of 2 x 2 waves owns a 128 x 128 tile of C and walks K in steps of
//    BK = 32 with two LDS stages (dwordx4 loads of step t+1 in flight while step t is
//    multiplied; one barrier per step);
//  * each wave owns 64 x 64 of C as 2 x 2 blocks of 32 x 32 FP32 accumulators;
//  * A fragment: lane l holds 8 consecutive k of row l%32, read with one ds_read_b128
//    from A kept [m][k] in LDS with the 16-byte chunks of each row XOR-swizzled by
//    (m/2) mod 4, so the eight lanes of one LDS cycle hit eight distinct bank groups;
//  * B fragment: lane l needs the same 8 k of column l%32; B is kept [k][n] (as loaded)
//    and the fragment is gathered with 16-bit LDS reads;
//  * edges: per-element predicates with zero fill on tiles crossing M, N or the K tail.
#include "common.hpp"
#include "launch.hpp"

namespace g355 {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 32, kThreads = 256;
constexpr int kSB = kBN + 8;              // B LDS row stride (halves), 16-byte multiple
constexpr int kLdsA = kBM * kBK;          // halves per stage
constexpr int kLdsB = kBK * kSB;
constexpr int kAChunks = kBM * kBK / 8 / kThreads;  // 16-byte chunks per thread
constexpr int kBChunks = kBK * kBN / 8 / kThreads;

template <typename T>
__device__ __forceinline__ floatx16 mfma32x32x16(u16x8 a, u16x8 b, floatx16 c);
template <>
__device__ __forceinline__ floatx16 mfma32x32x16<f16_t>(u16x8 a, u16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                  __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ floatx16 mfma32x32x16<bf16_t>(u16x8 a, u16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Columns [c, c+8) of one row, zero outside [0, ncols) and for invalid rows.
template <bool VEC>
__device__ __forceinline__ u16x8 ld_chunk8(const uint16_t *__restrict__ row, int c, int ncols,
                                           bool row_ok, bool full) {
    if (full && VEC) return *reinterpret_cast<const u16x8 *>(row + c);
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (!row_ok) return v;
    if (VEC && c + 8 <= ncols) return *reinterpret_cast<const u16x8 *>(row + c);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (full || c + e < ncols) v[e] = row[c + e];
    return v;
}

__device__ __forceinline__ int swz_a(int m, int chunk) { return chunk ^ ((m >> 1) & 3); }

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_f16_gemm_kernel(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                          const uint16_t *__restrict__ B, int ldb, float *__restrict__ C,
                          int ldc) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (kLdsA + kLdsB)];

    const int tiles_m = cdiv(M, kBM), tiles_n = cdiv(N, kBN);
    int tm, tn;
    grouped_tile(xcd_contiguous_id(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const bool tile_full = (m0 + kBM <= M) && (n0 + kBN <= N);

    const int t = threadIdx.x;
    const int lane = t % 64, wave = t / 64;
    const int wm = wave / 2, wn = wave % 2;
    const int l32 = lane % 32, lhi = lane / 32;

    int a_r[kAChunks], a_c[kAChunks], b_r[kBChunks], b_c[kBChunks];
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
        const int q = t + kThreads * i;
        a_r[i] = q / (kBK / 8);
        a_c[i] = q % (kBK / 8);
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
        const int q = t + kThreads * i;
        b_r[i] = q / (kBN / 8);
        b_c[i] = q % (kBN / 8);
    }

    u16x8 sa[kAChunks], sb[kBChunks];
    auto load_tile = [&](int k0) {
        const bool full = tile_full && (k0 + kBK <= K);
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int r = m0 + a_r[i];
            const bool ok = r < M;
            sa[i] = ld_chunk8<VEC>(A + (size_t)(ok ? r : 0) * lda, k0 + 8 * a_c[i], K, ok, full);
        }
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) {
            const int r = k0 + b_r[i];
            const bool ok = r < K;
            sb[i] = ld_chunk8<VEC>(B + (size_t)(ok ? r : 0) * ldb, n0 + 8 * b_c[i], N, ok, full);
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t *As = lds + buf * (kLdsA + kLdsB);
        uint16_t *Bs = As + kLdsA;
#pragma unroll
        for (int i = 0; i < kAChunks; ++i)
            *reinterpret_cast<u16x8 *>(As + a_r[i] * kBK + 8 * swz_a(a_r[i], a_c[i])) = sa[i];
#pragma unroll
        for (int i = 0; i < kBChunks; ++i)
            *reinterpret_cast<u16x8 *>(Bs + b_r[i] * kSB + 8 * b_c[i]) = sb[i];
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = cdiv(K, kBK);
    if (nk > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    const int a_row0 = wm * 64 + l32;
    const int b_col0 = wn * 64 + l32;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tile((kt + 1) * kBK);
        const uint16_t *As = lds + buf * (kLdsA + kLdsB);
        const uint16_t *Bs = As + kLdsA;
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            u16x8 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int m = a_row0 + 32 * i;
                af[i] = *reinterpret_cast<const u16x8 *>(As + m * kBK + 8 * swz_a(m, 2 * s + lhi));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    bf[j][e] = Bs[(16 * s + 8 * lhi + e) * kSB + b_col0 + 32 * j];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16<T>(af[i], bf[j], acc[i][j]);
        }
        if (kt + 1 < nk) store_tile(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + b_col0 + 32 * j;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + 32 * i + 8 * (r / 4) + 4 * lhi + (r % 4);
                if (tile_full || (row < M && col < N)) C[(size_t)row * ldc + col] = acc[i][j][r];
            }
        }
    }
}

bool f16_vec(const GemmArgs &g) {
    return rows_aligned16(g.A, g.lda, 2) && rows_aligned16(g.B, g.ldb, 2);
}

template <typename T>
hipError_t launch_t(const GemmArgs &g, hipStream_t s) {
    const dim3 grid(cdiv(g.M, kBM) * cdiv(g.N, kBN));
    const dim3 block(kThreads);
    const uint16_t *A = (const uint16_t *)g.A, *B = (const uint16_t *)g.B;
    if (f16_vec(g))
        hipLaunchKernelGGL((mfma_f16_gemm_kernel<T, true>), grid, block, 0, s, g.M, g.N, g.K, A,
                           g.lda, B, g.ldb, g.C, g.ldc);
    else
        hipLaunchKernelGGL((mfma_f16_gemm_kernel<T, false>), grid, block, 0, s, g.M, g.N, g.K, A,
                           g.lda, B, g.ldb, g.C, g.ldc);
    return hipGetLastError();
}

}  // namespace

const char *desc_mfma_f16(int dtype, const GemmArgs &g) {
    const bool v = f16_vec(g);
    if (dtype == kF16) return v ? "mfma_f16 128x128x32 w2x2 dwordx4" : "mfma_f16 128x128x32 w2x2 u16";
    return v ? "mfma_bf16 128x128x32 w2x2 dwordx4" : "mfma_bf16 128x128x32 w2x2 u16";
}

hipError_t launch_mfma_f16(int dtype, const GemmArgs &g, hipStream_t s) {
    return dtype == kF16 ? launch_t<f16_t>(g, s) : launch_t<bf16_t>(g, s);
}

}  // namespace g355
