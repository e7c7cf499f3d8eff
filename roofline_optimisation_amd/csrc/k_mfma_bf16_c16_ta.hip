// BF16-input GEMM with C stored in the same 16-bit type (C = round16(sign * op(A) op(B)
// (+ C))),
// A transposed (m-contiguous), B in either layout; the other layouts and the dispatch are
// in k_mfma_bf16_c16.hip.  Kernels in h16_gemm.hpp (epilogue kind 2).
#include "h16_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_bf16_c16_ta(const GemmArgs &g, hipStream_t s) {
    if (g.trans_b == 0) return launch_layout<bf16_t, true, true, 2>(g, s);
    return launch_layout<bf16_t, true, false, 2>(g, s);
}

}  // namespace g355
