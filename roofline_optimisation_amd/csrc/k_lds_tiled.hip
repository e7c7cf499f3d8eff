// LDS-tiled FP32 kernel: a workgroup stages a 32 x 32 slice of A and a 32 x 32 slice
// of B in local data share (LDS), synchronises, and accumulates from LDS; each operand
// element fetched from global memory is reused 32 times.
//
// This is the block-level reuse of "Advanced CUDA features - starting from GEMM"
// (section "Shared Memory Tiling": load a tile of A and of B, barrier, compute from the
// shared copy, repeat along K; global traffic falls by the tile size) and of the
// Level 2 kernel of "Kernel optimisation guide", with the zero-filled out-of-range
// loads and guarded store of the former.
//
// gfx950 mapping (256 threads = 4 waves of 64):
//  * global -> LDS: each thread moves one 16-byte chunk of A and one of B per k-step;
//    eight consecutive lanes cover one 128-byte row segment, so loads are coalesced
//    dwordx4 accesses ("Kernel optimisation guide", vectorised loads and coalescing)
//    and the ds_write_b128 of eight lanes covers all 32 banks once;
//  * compute: lane l owns column l mod 32 and rows (l/32 + 2w) + 8i, i = 0..3, of the
//    tile; per k the wave reads 2 distinct A words (broadcast) and 32 consecutive B
//    words, so the LDS reads are free of bank conflicts without padding;
//  * rows whose start is not 16-byte aligned (odd strides such as lda = 515) take the
//    same path with four dword loads per chunk.
// Accumulation is fmaf in increasing k from +0.0, so each element's rounding sequence
// is the naive kernel's.
#include "common.hpp"
#include "launch.hpp"

namespace g355 {

namespace {

constexpr int kT = 32;  // tile edge (M, N and K)

// Load columns [c, c+4) of one row of a row-major matrix, zero outside [0, ncols) and
// for invalid rows.
template <bool VEC>
__device__ __forceinline__ floatx4 load_chunk(const float *__restrict__ row, int c, int ncols,
                                              bool row_ok) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (!row_ok) return v;
    if (VEC && c + 4 <= ncols) return *reinterpret_cast<const floatx4 *>(row + c);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (c + e < ncols) v[e] = row[c + e];
    return v;
}

template <bool VEC>
__global__ __launch_bounds__(256) void lds_tiled_f32_kernel(int M, int N, int K,
                                                            const float *__restrict__ A, int lda,
                                                            const float *__restrict__ B, int ldb,
                                                            float *__restrict__ C, int ldc) {
    __shared__ __attribute__((aligned(16))) float As[kT][kT];  // [m][k]
    __shared__ __attribute__((aligned(16))) float Bs[kT][kT];  // [k][n]

    const int t = threadIdx.x;
    const int m0 = blockIdx.y * kT;
    const int n0 = blockIdx.x * kT;
    const int lr = t / 8;          // row of the 32 x 32 slice this thread loads
    const int lc = (t % 8) * 4;    // first column of its chunk
    const int tc = t % kT;         // output column
    const int tr = t / kT;         // output rows tr + 8 i

    const bool a_row_ok = m0 + lr < M;
    const float *a_row = A + (size_t)(a_row_ok ? m0 + lr : 0) * lda;

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += kT) {
        const floatx4 av = load_chunk<VEC>(a_row, k0 + lc, K, a_row_ok);
        const bool b_row_ok = k0 + lr < K;
        const float *b_row = B + (size_t)(b_row_ok ? k0 + lr : 0) * ldb;
        const floatx4 bv = load_chunk<VEC>(b_row, n0 + lc, N, b_row_ok);
        *reinterpret_cast<floatx4 *>(&As[lr][lc]) = av;
        *reinterpret_cast<floatx4 *>(&Bs[lr][lc]) = bv;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kT; ++kk) {
            const float b = Bs[kk][tc];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(As[tr + 8 * i][kk], b, acc[i]);
        }
        __syncthreads();
    }
    const int col = n0 + tc;
    if (col < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + tr + 8 * i;
            if (row < M) C[(size_t)row * ldc + col] = acc[i];
        }
    }
}

}  // namespace

static bool tiled_vec(const GemmArgs &g) {
    return rows_aligned16(g.A, g.lda, 4) && rows_aligned16(g.B, g.ldb, 4);
}

const char *desc_lds_tiled_f32(const GemmArgs &g) {
    return tiled_vec(g) ? "lds_tiled_f32 32x32x32 dwordx4" : "lds_tiled_f32 32x32x32 dword";
}

hipError_t launch_lds_tiled_f32(const GemmArgs &g, hipStream_t s) {
    dim3 grid(cdiv(g.N, kT), cdiv(g.M, kT));
    dim3 block(256);
    if (tiled_vec(g))
        hipLaunchKernelGGL(lds_tiled_f32_kernel<true>, grid, block, 0, s, g.M, g.N, g.K,
                           (const float *)g.A, g.lda, (const float *)g.B, g.ldb, g.C, g.ldc);
    else
        hipLaunchKernelGGL(lds_tiled_f32_kernel<false>, grid, block, 0, s, g.M, g.N, g.K,
                           (const float *)g.A, g.lda, (const float *)g.B, g.ldb, g.C, g.ldc);
    return hipGetLastError();
}

}  // namespace g355
