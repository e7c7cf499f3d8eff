// Naive floor kernel: one thread per element of C, every operand fetched from global
// memory, FP32 accumulation in increasing k.
//
// This is the "no reuse" case of "Advanced CUDA features - starting from GEMM"
// (roofline section, case A and case (4): each C_ij reads a row of A and a column of
// B, 2n^3 words in total, intensity 0.25 FLOP/B) and the Level 1 kernel of "Kernel
// optimisation guide".  It is kept as the measured floor of the kernel ladder.
//
// gfx950 mapping: 64 x 4 threads per workgroup, the 64 lanes of a wave along a row of
// C, so each B row segment and each C store is one contiguous 256-byte access and the
// A element is a wave-uniform broadcast.  It also takes the transposed, negated and
// accumulating forms directly (C = sign * op(A) op(B) (+ C)), with C in binary32 or
// (C16) in the operands' 16-bit type.
#include "common.hpp"
#include "launch.hpp"

namespace g355 {

template <typename T, bool C16>
__global__ __launch_bounds__(256) void naive_gemm_kernel(int M, int N, int K,
                                                         const T *__restrict__ A, int lda,
                                                         const T *__restrict__ B, int ldb,
                                                         float *__restrict__ C, int ldc,
                                                         int trans_a, int trans_b, float sign,
                                                         int accumulate) {
    const int col = blockIdx.x * 64 + threadIdx.x;
    const int row = blockIdx.y * 4 + threadIdx.y;
    if (row >= M || col >= N) return;
    // op(A)[row][k] and op(B)[k][col]: a transposed A is stored K x M, a transposed B N x K
    const T *a = trans_a ? A + row : A + (size_t)row * lda;
    const size_t sa = trans_a ? (size_t)lda : 1;
    const T *b = trans_b ? B + (size_t)col * ldb : B + col;
    const size_t sb = trans_b ? 1 : (size_t)ldb;
    float acc = 0.0f;
    for (int k = 0; k < K; ++k)
        acc = __builtin_fmaf(to_float(a[k * sa]), to_float(b[k * sb]), acc);
    const float v = sign * acc;
    if constexpr (C16) {
        uint16_t *c = (uint16_t *)C + (size_t)row * ldc + col;
        *c = to_bits(accumulate ? v + to_float(T{*c}) : v, T{});
    } else {
        float *c = C + (size_t)row * ldc + col;
        *c = accumulate ? v + *c : v;
    }
}

hipError_t launch_naive(int dtype, const GemmArgs &g, hipStream_t s) {
    dim3 block(64, 4);
    dim3 grid(cdiv(g.N, 64), cdiv(g.M, 4));
    if (g.c16) {
        if (dtype == kF16)
            hipLaunchKernelGGL((naive_gemm_kernel<f16_t, true>), grid, block, 0, s, g.M, g.N, g.K,
                               (const f16_t *)g.A, g.lda, (const f16_t *)g.B, g.ldb, g.C, g.ldc,
                               g.trans_a, g.trans_b, g.sign, g.accumulate);
        else
            hipLaunchKernelGGL((naive_gemm_kernel<bf16_t, true>), grid, block, 0, s, g.M, g.N, g.K,
                               (const bf16_t *)g.A, g.lda, (const bf16_t *)g.B, g.ldb, g.C, g.ldc,
                               g.trans_a, g.trans_b, g.sign, g.accumulate);
        return hipGetLastError();
    }
    switch (dtype) {
    case kF32:
        hipLaunchKernelGGL((naive_gemm_kernel<float, false>), grid, block, 0, s, g.M, g.N, g.K,
                           (const float *)g.A, g.lda, (const float *)g.B, g.ldb, g.C, g.ldc,
                           g.trans_a, g.trans_b, g.sign, g.accumulate);
        break;
    case kF16:
        hipLaunchKernelGGL((naive_gemm_kernel<f16_t, false>), grid, block, 0, s, g.M, g.N, g.K,
                           (const f16_t *)g.A, g.lda, (const f16_t *)g.B, g.ldb, g.C, g.ldc,
                           g.trans_a, g.trans_b, g.sign, g.accumulate);
        break;
    default:
        hipLaunchKernelGGL((naive_gemm_kernel<bf16_t, false>), grid, block, 0, s, g.M, g.N, g.K,
                           (const bf16_t *)g.A, g.lda, (const bf16_t *)g.B, g.ldb, g.C, g.ldc,
                           g.trans_a, g.trans_b, g.sign, g.accumulate);
        break;
    }
    return hipGetLastError();
}

}  // namespace g355
