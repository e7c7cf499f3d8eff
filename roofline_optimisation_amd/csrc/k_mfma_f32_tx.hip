// FP32 GEMM, plain product in the transposed operand layouts (kernel in f32_gemm.hpp).
// A transposed A is stored K x M (m-contiguous, kind MN); a transposed B N x K
// (k-contiguous, kind KM).
#include "f32_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_f32_tx(const GemmArgs &g, hipStream_t s) {
    if (g.trans_a && g.trans_b) return launch_f32_layout<true, false, false>(g, s);
    if (g.trans_a) return launch_f32_layout<true, true, false>(g, s);
    return launch_f32_layout<false, false, false>(g, s);
}

}  // namespace g355
