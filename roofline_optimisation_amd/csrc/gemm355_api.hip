// C ABI of libgemm355: argument validation, device check and kernel-family dispatch.
//
// The host launcher's job is the one described for launch_matmul_l1 on "Advanced CUDA
// features - starting from GEMM" (section "Shared Memory Tiling", reference
// implementation): size the grid by ceiling division over the output tiles, launch on
// the caller's stream and check the launch.  Here the check returns a status instead
// of aborting the process, and every argument is validated before the first HIP call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gemm355.h"
#include "common.hpp"
#include "launch.hpp"

namespace g355 {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
signed char g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

// True when `dev` is a gfx950 device; queried once per device.
bool device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 0) {
        hipDeviceProp_t p;
        bool ok = false;
        if (hipGetDeviceProperties(&p, dev) == hipSuccess) {
            const char *a = p.gcnArchName;
            ok = a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' &&
                 a[5] == '0' && (a[6] == '\0' || a[6] == ':');
        }
        g_dev_state[dev] = ok ? 1 : -1;
    }
    return g_dev_state[dev] == 1;
}

bool valid_args(int dtype, int M, int N, int K, const void *A, int lda, const void *B, int ldb,
                const void *C, int ldc) {
    if (dtype < kF32 || dtype > kBF16) return false;
    if (M < 0 || N < 0 || K < 0) return false;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1)) return false;
    if ((long)M * K > 0 && A == nullptr) return false;
    if ((long)K * N > 0 && B == nullptr) return false;
    if ((long)M * N > 0 && C == nullptr) return false;
    return true;
}

// Family the typed entry points use.  FP32 GEMMs go to the matrix cores
// (v_mfma_f32_32x32x2_f32 runs at the full FP32 rate); FP16/BF16 likewise.
int auto_variant(int /*dtype*/, const GemmArgs & /*g*/) { return GEMM355_VARIANT_MFMA; }

// The dispatched 16-bit kernels with the 192 x 256 and 256 x 192 tiles turned off.
GemmArgs square(const GemmArgs &g) {
    GemmArgs h = g;
    h.square_tiles = 1;
    return h;
}

// The dispatched 16-bit kernels with the two-per-CU 128 x 128 direct-to-LDS tile turned off.
GemmArgs one_round_128(const GemmArgs &g) {
    GemmArgs h = g;
    h.one_round_128 = 1;
    return h;
}

// The dispatched 16-bit kernels with the direct-to-LDS tiles of small grids turned off.
GemmArgs staged_small(const GemmArgs &g) {
    GemmArgs h = g;
    h.staged_small = 1;
    return h;
}

bool variant_supported(int variant, int dtype) {
    switch (variant) {
    case GEMM355_VARIANT_NAIVE:
    case GEMM355_VARIANT_MFMA: return true;
    case GEMM355_VARIANT_LDS_TILED:
    case GEMM355_VARIANT_REGBLOCK: return dtype == kF32;
    case GEMM355_VARIANT_MFMA_SPLIT:
    case GEMM355_VARIANT_MFMA_W8:
    case GEMM355_VARIANT_MFMA_T256X128:
    case GEMM355_VARIANT_MFMA_T256X256:
    case GEMM355_VARIANT_MFMA_STAGED128:
    case GEMM355_VARIANT_MFMA_STAGED_SMALL: return dtype == kF16 || dtype == kBF16;
    default: return false;
    }
}

hipError_t launch(int variant, int dtype, const GemmArgs &g, hipStream_t s) {
    switch (variant) {
    case GEMM355_VARIANT_NAIVE: return launch_naive(dtype, g, s);
    case GEMM355_VARIANT_LDS_TILED: return launch_lds_tiled_f32(g, s);
    case GEMM355_VARIANT_REGBLOCK: return launch_regblock_f32(g, s);
    case GEMM355_VARIANT_MFMA_SPLIT:
    case GEMM355_VARIANT_MFMA_W8:
    case GEMM355_VARIANT_MFMA_T256X128: return launch_mfma_f16_sched(variant, dtype, g, s);
    case GEMM355_VARIANT_MFMA_T256X256: return launch_mfma_f16(dtype, square(g), s);
    case GEMM355_VARIANT_MFMA_STAGED128: return launch_mfma_f16(dtype, one_round_128(g), s);
    case GEMM355_VARIANT_MFMA_STAGED_SMALL: return launch_mfma_f16(dtype, staged_small(g), s);
    default: return dtype == kF32 ? launch_mfma_f32(g, s) : launch_mfma_f16(dtype, g, s);
    }
}

bool is_sched_variant(int variant) {
    return variant >= GEMM355_VARIANT_MFMA_SPLIT && variant <= GEMM355_VARIANT_MFMA_T256X128;
}

gemm355_status run(int variant, int dtype, int M, int N, int K, const void *A, int lda,
                   const void *B, int ldb, float *C, int ldc, hipStream_t stream) {
    if (!valid_args(dtype, M, N, K, A, lda, B, ldb, C, ldc)) return GEMM355_ERR_INVALID_ARG;
    if (variant < GEMM355_VARIANT_AUTO || variant > GEMM355_VARIANT_MFMA_STAGED_SMALL)
        return GEMM355_ERR_INVALID_ARG;
    const GemmArgs g{M, N, K, A, lda, B, ldb, C, ldc};
    if (variant == GEMM355_VARIANT_AUTO) variant = auto_variant(dtype, g);
    if (!variant_supported(variant, dtype)) return GEMM355_ERR_UNSUPPORTED;
    if (is_sched_variant(variant) && M > 0 && N > 0 && !mfma_f16_sched_ok(variant, g))
        return GEMM355_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return GEMM355_OK;
    if (!device_ok()) return GEMM355_ERR_DEVICE;
    // Every kernel starts its accumulators at +0.0, so K = 0 stores the empty sum.
    return launch(variant, dtype, g, stream) == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

constexpr unsigned kExFlags = GEMM355_TRANS_A | GEMM355_TRANS_B | GEMM355_NEG_A | GEMM355_NEG_B |
                               GEMM355_ACCUMULATE | GEMM355_C_16;

// Validates gemm355_gemm_ex's arguments and fills `g` (variant resolved from AUTO).
gemm355_status ex_args(int &variant, int dtype, unsigned flags, int M, int N, int K, const void *A,
                       int lda, const void *B, int ldb, void *C, int ldc, GemmArgs &g) {
    if ((flags & ~kExFlags) != 0) return GEMM355_ERR_INVALID_ARG;
    const bool c16 = flags & GEMM355_C_16;
    if (c16 && dtype != kF16 && dtype != kBF16) return GEMM355_ERR_INVALID_ARG;
    const bool ta = flags & GEMM355_TRANS_A, tb = flags & GEMM355_TRANS_B;
    const bool acc = flags & GEMM355_ACCUMULATE;
    const bool neg = ((flags & GEMM355_NEG_A) != 0) != ((flags & GEMM355_NEG_B) != 0);
    if (dtype < kF32 || dtype > kBF16) return GEMM355_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return GEMM355_ERR_INVALID_ARG;
    const int min_lda = ta ? M : K, min_ldb = tb ? K : N;
    if (lda < (min_lda > 1 ? min_lda : 1) || ldb < (min_ldb > 1 ? min_ldb : 1) ||
        ldc < (N > 1 ? N : 1))
        return GEMM355_ERR_INVALID_ARG;
    if ((long)M * K > 0 && A == nullptr) return GEMM355_ERR_INVALID_ARG;
    if ((long)K * N > 0 && B == nullptr) return GEMM355_ERR_INVALID_ARG;
    if ((long)M * N > 0 && C == nullptr) return GEMM355_ERR_INVALID_ARG;
    if (variant < GEMM355_VARIANT_AUTO || variant > GEMM355_VARIANT_MFMA_STAGED_SMALL)
        return GEMM355_ERR_INVALID_ARG;
    g = GemmArgs{M, N, K, A, lda, B, ldb, (float *)C, ldc};
    g.c16 = c16;
    g.trans_a = ta;
    g.trans_b = tb;
    g.sign = neg ? -1.0f : 1.0f;
    g.accumulate = acc;
    if (variant == GEMM355_VARIANT_AUTO) variant = auto_variant(dtype, g);
    if (!variant_supported(variant, dtype)) return GEMM355_ERR_UNSUPPORTED;
    if (flags != 0 && variant != GEMM355_VARIANT_NAIVE && variant != GEMM355_VARIANT_MFMA &&
        variant != GEMM355_VARIANT_MFMA_T256X256 && variant != GEMM355_VARIANT_MFMA_STAGED128 &&
        variant != GEMM355_VARIANT_MFMA_STAGED_SMALL)
        return GEMM355_ERR_UNSUPPORTED;
    if (is_sched_variant(variant) && M > 0 && N > 0 && !mfma_f16_sched_ok(variant, g))
        return GEMM355_ERR_UNSUPPORTED;
    return GEMM355_OK;
}

gemm355_status run_ex(int variant, int dtype, unsigned flags, int M, int N, int K, const void *A,
                      int lda, const void *B, int ldb, void *C, int ldc, hipStream_t stream) {
    GemmArgs g{};
    const gemm355_status st = ex_args(variant, dtype, flags, M, N, K, A, lda, B, ldb, C, ldc, g);
    if (st != GEMM355_OK) return st;
    if (M == 0 || N == 0) return GEMM355_OK;
    if (!device_ok()) return GEMM355_ERR_DEVICE;
    if (K == 0 && g.accumulate) return GEMM355_OK;  // adding the empty sum leaves C as it is
    return launch(variant, dtype, g, stream) == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

const char *desc_of(int variant, int dtype, const GemmArgs &g) {
    switch (variant) {
    case GEMM355_VARIANT_NAIVE: return "naive 64x4 threads, one output each";
    case GEMM355_VARIANT_LDS_TILED: return desc_lds_tiled_f32(g);
    case GEMM355_VARIANT_REGBLOCK: return desc_regblock_f32(g);
    case GEMM355_VARIANT_MFMA_SPLIT:
    case GEMM355_VARIANT_MFMA_W8:
    case GEMM355_VARIANT_MFMA_T256X128:
        return mfma_f16_sched_ok(variant, g) ? desc_mfma_f16_sched(variant, dtype) : "invalid";
    case GEMM355_VARIANT_MFMA_T256X256: return desc_mfma_f16(dtype, square(g));
    case GEMM355_VARIANT_MFMA_STAGED128: return desc_mfma_f16(dtype, one_round_128(g));
    case GEMM355_VARIANT_MFMA_STAGED_SMALL: return desc_mfma_f16(dtype, staged_small(g));
    default: return dtype == kF32 ? desc_mfma_f32(g) : desc_mfma_f16(dtype, g);
    }
}

}  // namespace

bool current_device_is_gfx950() { return device_ok(); }

}  // namespace g355

using namespace g355;

extern "C" {

gemm355_status gemm_f32(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                        float *C, int ldc, hipStream_t stream) {
    return run(GEMM355_VARIANT_AUTO, kF32, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

gemm355_status gemm_f16f32acc(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B,
                              int ldb, float *C, int ldc, hipStream_t stream) {
    return run(GEMM355_VARIANT_AUTO, kF16, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

gemm355_status gemm_bf16f32acc(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B,
                               int ldb, float *C, int ldc, hipStream_t stream) {
    return run(GEMM355_VARIANT_AUTO, kBF16, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

gemm355_status gemm355_run_variant(int variant, int dtype, int M, int N, int K, const void *A,
                                   int lda, const void *B, int ldb, float *C, int ldc,
                                   hipStream_t stream) {
    return run(variant, dtype, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

gemm355_status gemm355_gemm_ex(int variant, int dtype, unsigned flags, int M, int N, int K,
                               const void *A, int lda, const void *B, int ldb, void *C, int ldc,
                               hipStream_t stream) {
    return run_ex(variant, dtype, flags, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm355_select_variant(int dtype, int M, int N, int K, const void *A, int lda, const void *B,
                           int ldb, const float *C, int ldc) {
    if (!valid_args(dtype, M, N, K, A, lda, B, ldb, C, ldc)) return -1;
    const GemmArgs g{M, N, K, A, lda, B, ldb, const_cast<float *>(C), ldc};
    return auto_variant(dtype, g);
}

const char *gemm355_kernel_desc(int variant, int dtype, int M, int N, int K, const void *A, int lda,
                                const void *B, int ldb, const float *C, int ldc) {
    if (!valid_args(dtype, M, N, K, A, lda, B, ldb, C, ldc)) return "invalid";
    const GemmArgs g{M, N, K, A, lda, B, ldb, const_cast<float *>(C), ldc};
    if (variant == GEMM355_VARIANT_AUTO) variant = auto_variant(dtype, g);
    if (!variant_supported(variant, dtype)) return "invalid";
    return desc_of(variant, dtype, g);
}

const char *gemm355_kernel_desc_ex(int variant, int dtype, unsigned flags, int M, int N, int K,
                                   const void *A, int lda, const void *B, int ldb, const void *C,
                                   int ldc) {
    GemmArgs g{};
    if (ex_args(variant, dtype, flags, M, N, K, A, lda, B, ldb, const_cast<void *>(C), ldc, g) !=
        GEMM355_OK)
        return "invalid";
    return desc_of(variant, dtype, g);
}

const char *gemm355_status_string(int status) {
    switch (status) {
    case GEMM355_OK: return "ok";
    case GEMM355_ERR_INVALID_ARG: return "invalid argument";
    case GEMM355_ERR_DEVICE: return "no gfx950 device";
    case GEMM355_ERR_LAUNCH: return "kernel launch failed";
    case GEMM355_ERR_UNSUPPORTED: return "variant not available for this dtype";
    default: return "unknown";
    }
}

const char *gemm355_variant_name(int variant) {
    switch (variant) {
    case GEMM355_VARIANT_AUTO: return "auto";
    case GEMM355_VARIANT_NAIVE: return "naive";
    case GEMM355_VARIANT_LDS_TILED: return "lds_tiled";
    case GEMM355_VARIANT_REGBLOCK: return "regblock";
    case GEMM355_VARIANT_MFMA: return "mfma";
    case GEMM355_VARIANT_MFMA_SPLIT: return "mfma_split";
    case GEMM355_VARIANT_MFMA_W8: return "mfma_w8";
    case GEMM355_VARIANT_MFMA_T256X128: return "mfma_t256x128";
    case GEMM355_VARIANT_MFMA_T256X256: return "mfma_t256x256";
    case GEMM355_VARIANT_MFMA_STAGED128: return "mfma_staged128";
    case GEMM355_VARIANT_MFMA_STAGED_SMALL: return "mfma_staged_small";
    default: return "unknown";
    }
}

int gemm355_version(void) { return 100; }

}  // extern "C"
