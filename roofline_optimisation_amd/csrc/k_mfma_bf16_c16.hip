// BF16-input GEMM with C stored in the same 16-bit type (C = round16(sign * op(A) op(B)
// (+ C))),
// A k-contiguous, B in either layout, and the dispatch; the layouts with A transposed are
// in k_mfma_bf16_c16_ta.hip (a translation unit of its own, so the two compile in
// parallel).  Kernels in h16_gemm.hpp (epilogue kind 2).
#include "h16_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_bf16_c16_ta(const GemmArgs &g, hipStream_t s);

hipError_t launch_mfma_bf16_c16(const GemmArgs &g, hipStream_t s) {
    if (g.trans_a) return launch_mfma_bf16_c16_ta(g, s);
    if (g.trans_b == 0) return launch_layout<bf16_t, false, true, 2>(g, s);
    return launch_layout<bf16_t, false, false, 2>(g, s);
}

}  // namespace g355
