// FP16 / BF16 GEMM with FP32 accumulation on the gfx950 matrix cores: the plain product
// in the untransposed layout (A k-contiguous, B n-contiguous) and the dispatch.  The
// kernels and their design are in h16_gemm.hpp; the transposed layouts, the
// accumulating variants and the 16-bit-C variants are instantiated in k_mfma_f16_tx.hip,
// k_mfma_f16_acc*.hip and k_mfma_*_c16.hip, so that the translation units compile in
// parallel.
#include "h16_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_f16_tx(int dtype, const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_f16_acc(const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_bf16_acc(const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_f16_c16(const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_bf16_c16(const GemmArgs &g, hipStream_t s);

const char *desc_mfma_f16(int dtype, const GemmArgs &g) {
    const bool v = h16_vec(g);
    const bool big = pick_tile(g) == 256;
    if (big && use_dma(g, 256))
        return dtype == kF16 ? "mfma_f16 256x256x32 w2x2 lds-dma" : "mfma_bf16 256x256x32 w2x2 lds-dma";
    const bool narrow = !big && !g.trans_a && !g.signed_or_acc() && !g.c16 && use_128x64(g);
    if (!big && !narrow && use_dma(g, 128))
        return dtype == kF16 ? "mfma_f16 128x128x32 w2x2 lds-dma" : "mfma_bf16 128x128x32 w2x2 lds-dma";
    if (dtype == kF16) {
        if (big) return v ? "mfma_f16 256x256x64 w2x2 dwordx4" : "mfma_f16 256x256x64 w2x2 dwordx4 unaligned";
        if (narrow) return v ? "mfma_f16 128x64x64 w2x2 dwordx4" : "mfma_f16 128x64x64 w2x2 dwordx4 unaligned";
        return v ? "mfma_f16 128x128x64 w2x2 dwordx4" : "mfma_f16 128x128x64 w2x2 dwordx4 unaligned";
    }
    if (big) return v ? "mfma_bf16 256x256x64 w2x2 dwordx4" : "mfma_bf16 256x256x64 w2x2 dwordx4 unaligned";
    if (narrow) return v ? "mfma_bf16 128x64x64 w2x2 dwordx4" : "mfma_bf16 128x64x64 w2x2 dwordx4 unaligned";
    return v ? "mfma_bf16 128x128x64 w2x2 dwordx4" : "mfma_bf16 128x128x64 w2x2 dwordx4 unaligned";
}

hipError_t launch_mfma_f16(int dtype, const GemmArgs &g, hipStream_t s) {
    if (g.c16) return dtype == kF16 ? launch_mfma_f16_c16(g, s) : launch_mfma_bf16_c16(g, s);
    if (g.signed_or_acc()) return dtype == kF16 ? launch_mfma_f16_acc(g, s) : launch_mfma_bf16_acc(g, s);
    if (g.trans_a || g.trans_b) return launch_mfma_f16_tx(dtype, g, s);
    // A is k-contiguous (KM), B n-contiguous (MN)
    return dtype == kF16 ? launch_layout<f16_t, false, true, 0>(g, s)
                         : launch_layout<bf16_t, false, true, 0>(g, s);
}

}  // namespace g355
