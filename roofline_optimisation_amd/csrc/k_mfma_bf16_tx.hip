// BF16 GEMM with FP32 accumulation: the plain product in the transposed operand layouts
// (the FP16 operands and the dispatch are in k_mfma_f16_tx.hip; kernels in h16_gemm.hpp).
#include "h16_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_bf16_tx(const GemmArgs &g, hipStream_t s) {
    if (g.trans_a && g.trans_b) return launch_layout<bf16_t, true, false, 0>(g, s);
    if (g.trans_a) return launch_layout<bf16_t, true, true, 0>(g, s);
    return launch_layout<bf16_t, false, false, 0>(g, s);
}

}  // namespace g355
