// Internal launcher declarations of libgemm355 (one per kernel family).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace g355 {

// Each launcher enqueues one kernel on `s` for already-validated arguments with
// M, N > 0 and returns the runtime's launch status.
hipError_t launch_naive(int dtype, const GemmArgs &g, hipStream_t s);
hipError_t launch_lds_tiled_f32(const GemmArgs &g, hipStream_t s);
hipError_t launch_regblock_f32(const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_f32(const GemmArgs &g, hipStream_t s);
hipError_t launch_mfma_f16(int dtype, const GemmArgs &g, hipStream_t s);
// The measurement-only schedules of the FP16/BF16 direct-to-LDS kernel
// (GEMM355_VARIANT_MFMA_SPLIT, _W8, _T256X128): whether one takes these arguments, and
// its launch.
bool mfma_f16_sched_ok(int variant, const GemmArgs &g);
hipError_t launch_mfma_f16_sched(int variant, int dtype, const GemmArgs &g, hipStream_t s);

// Host-side descriptions of the instance each launcher would pick.
const char *desc_lds_tiled_f32(const GemmArgs &g);
const char *desc_regblock_f32(const GemmArgs &g);
const char *desc_mfma_f32(const GemmArgs &g);
const char *desc_mfma_f16(int dtype, const GemmArgs &g);
const char *desc_mfma_f16_sched(int variant, int dtype);

// True when the current HIP device is a gfx950 (queried once per device).
bool current_device_is_gfx950();

// True when every row of a row-major matrix starts on a 16-byte boundary, i.e. the
// base is 16-byte aligned and the row stride is a multiple of 16 bytes.
inline bool rows_aligned16(const void *p, int ld, int elem_bytes) {
    return ((uintptr_t)p % 16 == 0) && (((size_t)ld * elem_bytes) % 16 == 0);
}

}  // namespace g355
