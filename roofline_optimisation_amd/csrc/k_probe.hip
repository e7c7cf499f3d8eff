// Lane-layout probes of the gfx950 matrix-core and LDS transpose-read instructions.
// Each probe runs one instruction on caller-chosen lane data and returns the raw lane
// results, so that tests can pin the layouts the GEMM kernels rely on.
#include <hip/hip_runtime.h>

#include "../../include/gemm355_probe.h"
#include "common.hpp"

namespace g355 {

namespace {

template <int KIND>
__global__ __launch_bounds__(64) void probe_mfma_kernel(const float *__restrict__ a,
                                                        const float *__restrict__ b,
                                                        float *__restrict__ d) {
    const int l = threadIdx.x;
    const size_t base = (size_t)blockIdx.x * 64 + l;
    if constexpr (KIND == 0 || KIND == 1) {
        const float av = a[base], bv = b[base];
        if constexpr (KIND == 0) {
            floatx16 acc = {};
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
            for (int i = 0; i < 16; ++i) d[base * 16 + i] = acc[i];
        } else {
            floatx4 acc = {};
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
            for (int i = 0; i < 4; ++i) d[base * 4 + i] = acc[i];
        }
    } else if constexpr (KIND == 2 || KIND == 3) {
        halfx8 av, bv;
        for (int e = 0; e < 8; ++e) {
            av[e] = (_Float16)a[base * 8 + e];
            bv[e] = (_Float16)b[base * 8 + e];
        }
        if constexpr (KIND == 2) {
            floatx16 acc = {};
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
            for (int i = 0; i < 16; ++i) d[base * 16 + i] = acc[i];
        } else {
            floatx4 acc = {};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
            for (int i = 0; i < 4; ++i) d[base * 4 + i] = acc[i];
        }
    } else {
        bf16x8 av, bv;
        for (int e = 0; e < 8; ++e) {
            av[e] = (__bf16)a[base * 8 + e];
            bv[e] = (__bf16)b[base * 8 + e];
        }
        if constexpr (KIND == 4) {
            floatx16 acc = {};
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
            for (int i = 0; i < 16; ++i) d[base * 16 + i] = acc[i];
        } else {
            floatx4 acc = {};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
            for (int i = 0; i < 4; ++i) d[base * 4 + i] = acc[i];
        }
    }
}

struct LaneAddrs {
    uint32_t a[64];
};

__global__ __launch_bounds__(64) void probe_tr16_kernel(LaneAddrs addrs, uint16_t *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) short lds[2048];
    const int l = threadIdx.x;
    for (int i = l; i < 2048; i += 64) lds[i] = (short)i;
    __syncthreads();
    typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
    const shortx4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_shortx4 *)((__attribute__((address_space(3))) char *)lds + addrs.a[l]));
    for (int e = 0; e < 4; ++e) out[4 * l + e] = (uint16_t)r[e];
}

struct LaneChunks {
    uint32_t c[64];
};

__global__ __launch_bounds__(64) void probe_gll_kernel(const uint32_t *__restrict__ src,
                                                       LaneChunks chunks, uint32_t base,
                                                       uint32_t *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[512];
    const int l = threadIdx.x;
    for (int i = l; i < 512; i += 64) lds[i] = 0;
    __syncthreads();
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void *)(src + 4 * chunks.c[l]),
        (__attribute__((address_space(3))) void *)((__attribute__((address_space(3))) char *)lds + base),
        16, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = l; i < 512; i += 64) out[i] = lds[i];
}

bool is_gfx950() {
    int dev = -1;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess)
        return false;
    const char *a = p.gcnArchName;
    return a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' && a[5] == '0';
}

}  // namespace

}  // namespace g355

using namespace g355;

extern "C" {

int gemm355_probe_mfma_shape(int kind, int *elems_per_lane, int *regs_per_lane) {
    if (kind < 0 || kind > 5) return -1;
    if (elems_per_lane) *elems_per_lane = kind < 2 ? 1 : 8;
    if (regs_per_lane) *regs_per_lane = (kind % 2 == 0) ? 16 : 4;
    return 0;
}

gemm355_status gemm355_probe_mfma(int kind, int nruns, const float *dev_a, const float *dev_b,
                                  float *dev_d, hipStream_t stream) {
    if (kind < 0 || kind > 5 || nruns < 1 || nruns > 65535 || !dev_a || !dev_b || !dev_d)
        return GEMM355_ERR_INVALID_ARG;
    if (!is_gfx950()) return GEMM355_ERR_DEVICE;
    const dim3 grid(nruns), block(64);
    switch (kind) {
    case 0: hipLaunchKernelGGL(probe_mfma_kernel<0>, grid, block, 0, stream, dev_a, dev_b, dev_d); break;
    case 1: hipLaunchKernelGGL(probe_mfma_kernel<1>, grid, block, 0, stream, dev_a, dev_b, dev_d); break;
    case 2: hipLaunchKernelGGL(probe_mfma_kernel<2>, grid, block, 0, stream, dev_a, dev_b, dev_d); break;
    case 3: hipLaunchKernelGGL(probe_mfma_kernel<3>, grid, block, 0, stream, dev_a, dev_b, dev_d); break;
    case 4: hipLaunchKernelGGL(probe_mfma_kernel<4>, grid, block, 0, stream, dev_a, dev_b, dev_d); break;
    default: hipLaunchKernelGGL(probe_mfma_kernel<5>, grid, block, 0, stream, dev_a, dev_b, dev_d); break;
    }
    return hipGetLastError() == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

gemm355_status gemm355_probe_global_load_lds(const uint32_t *dev_src, const uint32_t *host_src_chunk,
                                             uint32_t lds_base, uint32_t *dev_out,
                                             hipStream_t stream) {
    if (!dev_src || !host_src_chunk || !dev_out || lds_base % 16 != 0 || lds_base > 1024)
        return GEMM355_ERR_INVALID_ARG;
    LaneChunks lc;
    for (int l = 0; l < 64; ++l) {
        if (host_src_chunk[l] > 4095) return GEMM355_ERR_INVALID_ARG;
        lc.c[l] = host_src_chunk[l];
    }
    if (!is_gfx950()) return GEMM355_ERR_DEVICE;
    hipLaunchKernelGGL(probe_gll_kernel, dim3(1), dim3(64), 0, stream, dev_src, lc, lds_base,
                       dev_out);
    return hipGetLastError() == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

gemm355_status gemm355_probe_ds_read_tr16(const uint32_t *host_addr, uint16_t *dev_out,
                                          hipStream_t stream) {
    if (!host_addr || !dev_out) return GEMM355_ERR_INVALID_ARG;
    LaneAddrs la;
    for (int l = 0; l < 64; ++l) {
        if (host_addr[l] % 8 != 0 || host_addr[l] > 4096 - 8) return GEMM355_ERR_INVALID_ARG;
        la.a[l] = host_addr[l];
    }
    if (!is_gfx950()) return GEMM355_ERR_DEVICE;
    hipLaunchKernelGGL(probe_tr16_kernel, dim3(1), dim3(64), 0, stream, la, dev_out);
    return hipGetLastError() == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

}  // extern "C"
