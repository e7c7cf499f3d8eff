// Other schedules of the FP16 / BF16 direct-to-LDS kernel (h16_dma.hpp), kept so that
// they can be measured against the dispatched one on the same data movement:
//  * split: wave specialisation, the second path of the scheduling section of "Advanced
//    CUDA features - starting from GEMM" (producer warps move the data while consumer
//    warps compute, the two handing stages over through double buffers).  On CDNA4
//    every wave of a kernel gets the same register allocation, so a producer wave
//    beside a compute wave on one SIMD halves the compute wave's registers: the compute
//    waves hold 128 x 64 of C (128 accumulator registers) and the tile is 256 x 128,
//    fed by four producer waves;
//  * w8: the 256 x 256 tile on eight waves, two per SIMD, each 128 x 64 of C, every wave
//    issuing its share of the loads beside its MFMAs (the SIMD interleaves the two
//    waves' instruction streams);
//  * t256x128: 256 x 128 tiles on four waves, every wave loading: twice as many tiles as
//    256 x 256 ones, so a CU's second tile runs while the stores of its first drain.
// Plain products (A k-contiguous, B n-contiguous, FP32 C) of F16 / BF16 operands only.
#include <type_traits>
#include <utility>

#include "../../include/gemm355.h"
#include "h16_gemm.hpp"

namespace g355 {

namespace {

struct SchedShape {
    int em, en, waves;
};

SchedShape shape_of(int variant) {
    switch (variant) {
    case GEMM355_VARIANT_MFMA_SPLIT: return {256, 128, 8};
    case GEMM355_VARIANT_MFMA_W8: return {256, 256, 8};
    default: return {256, 128, 4};
    }
}

template <typename T, int EM, int EN, int WM, int WN, int NS, int PW>
hipError_t launch_sched(const GemmArgs &g, hipStream_t s) {
    hipLaunchKernelGGL((mfma_f16_dma_sched_kernel<T, EM, EN, WM, WN, NS, PW>),
                       dim3(cdiv(g.M, EM) * cdiv(g.N, EN)), dim3(64 * (WM * WN + PW)), 0, s, g.M, g.N,
                       g.K, (const uint16_t *)g.A, g.lda, (const uint16_t *)g.B, g.ldb, g.C, g.ldc);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_sched_t(int variant, const GemmArgs &g, hipStream_t s) {
    switch (variant) {
    case GEMM355_VARIANT_MFMA_SPLIT: return launch_sched<T, 256, 128, 2, 2, 4, 4>(g, s);
    case GEMM355_VARIANT_MFMA_W8: return launch_sched<T, 256, 256, 2, 4, 4, 0>(g, s);
    default: return launch_sched<T, 256, 128, 2, 2, 4, 0>(g, s);
    }
}

}  // namespace

// The shapes these instances take: whole tiles (M, N multiples of the tile extents),
// 16-byte-aligned rows, K a whole number of ring trips (4 stages of 32), every byte
// offset within the 31-bit buffer range; plain products only.
bool mfma_f16_sched_ok(int variant, const GemmArgs &g) {
    const SchedShape sh = shape_of(variant);
    if (g.trans_a || g.trans_b || g.signed_or_acc() || g.c16) return false;
    return h16_vec(g) && g.K > 0 && g.K % (dma::kBK * 4) == 0 && g.M % sh.em == 0 &&
           g.N % sh.en == 0 && op_fits(false, sh.em, g.K, g.lda) && op_fits(true, sh.en, g.K, g.ldb);
}

const char *desc_mfma_f16_sched(int variant, int dtype) {
    const bool f16 = dtype == kF16;
    switch (variant) {
    case GEMM355_VARIANT_MFMA_SPLIT:
        return f16 ? "mfma_f16 256x128x32 w2x2 + 4 producer waves lds-dma"
                   : "mfma_bf16 256x128x32 w2x2 + 4 producer waves lds-dma";
    case GEMM355_VARIANT_MFMA_W8:
        return f16 ? "mfma_f16 256x256x32 w2x4 lds-dma" : "mfma_bf16 256x256x32 w2x4 lds-dma";
    default:
        return f16 ? "mfma_f16 256x128x32 w2x2 lds-dma" : "mfma_bf16 256x128x32 w2x2 lds-dma";
    }
}

hipError_t launch_mfma_f16_sched(int variant, int dtype, const GemmArgs &g, hipStream_t s) {
    if (!mfma_f16_sched_ok(variant, g)) return hipErrorInvalidValue;
    return dtype == kF16 ? launch_sched_t<f16_t>(variant, g, s) : launch_sched_t<bf16_t>(variant, g, s);
}

}  // namespace g355
