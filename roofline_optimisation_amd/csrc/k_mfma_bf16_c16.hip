// BF16-input GEMM with C stored in the same 16-bit type (C = round16(sign * op(A) op(B)
// (+ C))), every operand layout; kernels in h16_gemm.hpp (epilogue kind 2).
#include "h16_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_bf16_c16(const GemmArgs &g, hipStream_t s) {
    const bool a_mn = g.trans_a != 0, b_mn = g.trans_b == 0;
    if (!a_mn && b_mn) return launch_layout<bf16_t, false, true, 2>(g, s);
    if (a_mn && !b_mn) return launch_layout<bf16_t, true, false, 2>(g, s);
    if (a_mn) return launch_layout<bf16_t, true, true, 2>(g, s);
    return launch_layout<bf16_t, false, false, 2>(g, s);
}

}  // namespace g355
