// FP16 / BF16 GEMM with FP32 accumulation: the plain product in the transposed operand
// layouts, FP16 operands and the dispatch (BF16 operands in k_mfma_bf16_tx.hip, a
// translation unit of its own; kernels in h16_gemm.hpp).  A transposed A is stored K x M,
// so it is m-contiguous (kind MN); a transposed B is stored N x K, so it is k-contiguous
// (KM).
#include "h16_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_bf16_tx(const GemmArgs &g, hipStream_t s);

hipError_t launch_mfma_f16_tx(int dtype, const GemmArgs &g, hipStream_t s) {
    if (dtype != kF16) return launch_mfma_bf16_tx(g, s);
    if (g.trans_a && g.trans_b) return launch_layout<f16_t, true, false, 0>(g, s);
    if (g.trans_a) return launch_layout<f16_t, true, true, 0>(g, s);
    return launch_layout<f16_t, false, false, 0>(g, s);
}

}  // namespace g355
