// FP16-input GEMM negated and / or accumulating into C (C = sign * op(A) op(B) (+ C)),
// A transposed (m-contiguous), B in either layout; the other layouts and the dispatch are
// in k_mfma_f16_acc.hip.  Kernels in h16_gemm.hpp (epilogue kind 1).
#include "h16_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_f16_acc_ta(const GemmArgs &g, hipStream_t s) {
    if (g.trans_b == 0) return launch_layout<f16_t, true, true, 1>(g, s);
    return launch_layout<f16_t, true, false, 1>(g, s);
}

}  // namespace g355
