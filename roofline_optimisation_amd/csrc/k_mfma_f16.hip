// FP16 / BF16 GEMM with FP32 accumulation on the gfx950 matrix cores: the plain product
// in the untransposed layout (A k-contiguous, B n-contiguous) and the dispatch.  The
// kernels and their design are in h16_gemm.hpp; the transposed layouts, the
// accumulating variants and the 16-bit-C variants are instantiated in k_mfma_f16_tx.hip,
// k_mfma_f16_acc*.hip and k_mfma_*_c16.hip, so that the translation units compile in
// parallel.
#include <string>

#include "h16_gemm.hpp"

namespace g355 {

hipError_t launch_mfma_f16_tx(int dtype, const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_f16_acc(const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_bf16_acc(const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_f16_c16(const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_bf16_c16(const GemmArgs &g, hipStream_t s);

// The instance (and, for the register-staged kernel, the launches of its plan) that
// launch_mfma_f16 picks for these arguments.  The string stays valid until the next call
// on the same thread.
const char *desc_mfma_f16(int dtype, const GemmArgs &g) {
    static thread_local std::string out;
    const bool v = h16_vec(g);
    const bool big = pick_tile(g) == 256;
    const char *name = dtype == kF16 ? "mfma_f16" : "mfma_bf16";
    const int epi = g.c16 ? 2 : (g.signed_or_acc() ? 1 : 0);
    const bool plain_km = !big && !g.trans_a && epi == 0 && staged_small_tiles(g);
    const bool small = plain_km && use_64x64(g);
    const bool narrow = plain_km && !small && use_128x64(g);
    const int bm = big ? 256 : (small ? 64 : 128), bn = big ? 256 : (small || narrow ? 64 : 128);
    out = name;
    const int rect = big ? rect_choice(g) : 256;
    if (!big && use_dma64(g)) {
        out += " 64x64x32 w2x2 lds-dma";
        if (dma_stages(g, 64) == 4) out += " ring4";
        if (dma_ragged_k(g, 64)) out += " k-zero-fill";
        return out.c_str();
    }
    if (rect != 256) {
        out += rect == 192 ? " 192x256x32 w2x2 lds-dma" : " 256x192x32 w2x2 lds-dma";
        if (dma_ragged_k(g, 256)) out += " k-zero-fill";
        return out.c_str();
    }
    const H16Plan p = plan_cfg(bm, bn, g.trans_a != 0, g.trans_b == 0, epi, g);
    if (p.dma) {
        out += big ? " 256x256x32 w2x2 lds-dma" : (small ? " 64x64x32 w2x2 lds-dma" : " 128x128x32 w2x2 lds-dma");
        if (!big && dma_stages(g, bm) == 4) out += " ring4";
        if (dma_ragged_k(g, bm)) out += " k-zero-fill";
        return out.c_str();
    }
    out += big ? " 256x256x64 w2x2 dwordx4"
               : (small ? " 64x64x64 w1x2 dwordx4"
                        : (narrow ? " 128x64x64 w2x2 dwordx4" : " 128x128x64 w2x2 dwordx4"));
    if (!v) out += " unaligned";
    // the launches: [all=...] or [interior=...][edges=...]
    auto edge_name = [&](int mode, bool paired) {
        return mode == 3 ? (paired ? "clamped,paired" : "clamped") : "predicated";
    };
    if (p.all_tiles) {
        out += std::string(" | all=") + edge_name(p.edge, p.edge_paired);
        return out.c_str();
    }
    if (p.interior >= 0)
        out += p.interior == 2 ? (p.interior_paired ? " | interior=buffer,paired" : " | interior=buffer")
                               : " | interior=pointer";
    if (p.edge >= 0) out += std::string(p.interior >= 0 ? " edges=" : " | edges=") + edge_name(p.edge, p.edge_paired);
    return out.c_str();
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
