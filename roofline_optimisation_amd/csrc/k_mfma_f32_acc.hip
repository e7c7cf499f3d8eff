// FP32 GEMM, negated and / or accumulating into C (C = sign * op(A) op(B) (+ C)), every
// operand layout (kernel in f32_gemm.hpp).
#include "f32_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_f32_acc(const GemmArgs &g, hipStream_t s) {
    const bool a_mn = g.trans_a != 0, b_mn = g.trans_b == 0;
    if (!a_mn && b_mn) return launch_f32_layout<false, true, true>(g, s);
    if (a_mn && !b_mn) return launch_f32_layout<true, false, true>(g, s);
    if (a_mn) return launch_f32_layout<true, true, true>(g, s);
    return launch_f32_layout<false, false, true>(g, s);
}

}  // namespace g355
