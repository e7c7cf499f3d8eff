// FP32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32): the plain product in
// the untransposed layout and the dispatch.  The kernel and its design are in
// f32_gemm.hpp; the transposed layouts and the accumulating variants are instantiated
// in k_mfma_f32_tx.hip and k_mfma_f32_acc.hip, so that the units compile in parallel.
#include "f32_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_f32_tx(const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_f32_acc(const GemmArgs &g, hipStream_t s);

const char *desc_mfma_f32(const GemmArgs &g) {
    const F32Pick p = pick_f32(g);
    switch (p.tile) {
    case 192: return p.vec ? "mfma_f32 192x192x32 w2x6 dwordx4" : "mfma_f32 192x192x32 w2x6 dword";
    case 128: return p.vec ? "mfma_f32 128x128x32 w2x4 dwordx4" : "mfma_f32 128x128x32 w2x4 dword";
    case 96: return p.vec ? "mfma_f32 96x96x32 w1x3 dwordx4" : "mfma_f32 96x96x32 w1x3 dword";
    default: return p.vec ? "mfma_f32 64x64x32 w2x2 dwordx4" : "mfma_f32 64x64x32 w2x2 dword";
    }
}

hipError_t launch_mfma_f32(const GemmArgs &g, hipStream_t s) {
    if (g.signed_or_acc()) return launch_mfma_f32_acc(g, s);
    if (g.trans_a || g.trans_b) return launch_mfma_f32_tx(g, s);
    return launch_f32_layout<false, true, false>(g, s);  // A k-contiguous, B n-contiguous
}

}  // namespace g355
