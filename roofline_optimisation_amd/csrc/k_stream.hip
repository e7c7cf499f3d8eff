// Memory-slope probes for the Little's-law and occupancy discussion of "Advanced CUDA
// features - starting from GEMM": a streaming kernel whose bytes in flight per wave and
// resident waves per CU the caller sets, and a dependent-load chase that measures the
// latency those bytes must cover.
//
// Streaming: the source is cut into chunks of (threads x vec x unroll) bytes, dealt to
// the workgroups round-robin.  Per chunk every lane issues all `unroll` loads before it
// consumes the first (these are the bytes in flight the page's law counts), and load u
// of the wave covers one contiguous 64 x vec byte span (coalesced).  Occupancy is set as
// the page sets it, through each workgroup's LDS allocation.
#include "../../include/gemm355_stream.h"
#include "common.hpp"
#include "launch.hpp"

namespace g355 {

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int VEC>
struct VecT;
template <>
struct VecT<4> {
    typedef uint32_t type;
    static __device__ __forceinline__ uint32_t fold(uint32_t v) { return v; }
};
template <>
struct VecT<8> {
    typedef u32x2 type;
    static __device__ __forceinline__ uint32_t fold(u32x2 v) { return v[0] ^ v[1]; }
};
template <>
struct VecT<16> {
    typedef u32x4 type;
    static __device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }
};

constexpr int kLdsMax = 160 * 1024;

template <int MODE, int VEC, int U>
__global__ __launch_bounds__(1024) void stream_kernel(const char *__restrict__ src,
                                                      char *__restrict__ dst, int64_t n_bytes) {
    // Dynamic LDS: reserved to limit residency; READ_XOR also uses its first words for
    // the cross-wave reduction.
    extern __shared__ uint32_t lds_reserve[];
    using V = typename VecT<VEC>::type;
    const int t = threadIdx.x, T = blockDim.x;
    const int64_t chunk = (int64_t)T * VEC * U;
    const int64_t nchunks = n_bytes / chunk;
    uint32_t x = 0;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const char *s = src + c * chunk;
        V v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *(const V *)(s + ((int64_t)u * T + t) * VEC);
        if constexpr (MODE != GEMM355_STREAM_READ_XOR) {
            char *d = dst + c * chunk;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                V *p = (V *)(d + ((int64_t)u * T + t) * VEC);
                if constexpr (MODE == GEMM355_STREAM_COPY_NT)
                    __builtin_nontemporal_store(v[u], p);
                else
                    *p = v[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) x ^= VecT<VEC>::fold(v[u]);
        }
    }
    // 32-bit words after the last whole chunk
    const int64_t nw = n_bytes / 4;
    for (int64_t w = nchunks * chunk / 4 + (int64_t)blockIdx.x * T + t; w < nw;
         w += (int64_t)gridDim.x * T) {
        const uint32_t v = ((const uint32_t *)src)[w];
        if constexpr (MODE == GEMM355_STREAM_COPY_NT)
            __builtin_nontemporal_store(v, (uint32_t *)dst + w);
        else if constexpr (MODE == GEMM355_STREAM_COPY)
            ((uint32_t *)dst)[w] = v;
        else
            x ^= v;
    }
    if constexpr (MODE == GEMM355_STREAM_READ_XOR) {
#pragma unroll
        for (int m = 32; m >= 1; m /= 2) x ^= __shfl_xor(x, m, 64);
        const int wave = t / 64, nwaves = T / 64;
        if (t % 64 == 0) lds_reserve[wave] = x;
        __syncthreads();
        if (t == 0) {
            uint32_t r = 0;
            for (int i = 0; i < nwaves; ++i) r ^= lds_reserve[i];
            ((uint32_t *)dst)[blockIdx.x] = r;
        }
    }
}

__global__ __launch_bounds__(64) void chase_kernel(const uint32_t *__restrict__ next, uint32_t last,
                                                   uint32_t start, int hops, uint64_t *out) {
    if (threadIdx.x != 0) return;
    uint32_t cur = start;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int h = 0; h < hops; ++h) cur = min(next[cur], last);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    out[0] = cur;
    out[1] = t1 - t0;
}

template <int MODE, int VEC, int U>
hipError_t launch_stream_k(const void *src, void *dst, int64_t n, int threads, int lds, int grid,
                           hipStream_t s) {
    auto k = stream_kernel<MODE, VEC, U>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3(grid), dim3(threads), lds, s, (const char *)src, (char *)dst, n);
    return hipGetLastError();
}

template <int MODE, int VEC>
hipError_t launch_stream_u(int unroll, const void *src, void *dst, int64_t n, int threads,
                           int lds, int grid, hipStream_t s) {
    switch (unroll) {
    case 1: return launch_stream_k<MODE, VEC, 1>(src, dst, n, threads, lds, grid, s);
    case 2: return launch_stream_k<MODE, VEC, 2>(src, dst, n, threads, lds, grid, s);
    case 4: return launch_stream_k<MODE, VEC, 4>(src, dst, n, threads, lds, grid, s);
    default: return launch_stream_k<MODE, VEC, 8>(src, dst, n, threads, lds, grid, s);
    }
}

template <int MODE>
hipError_t launch_stream_m(int vec, int unroll, const void *src, void *dst, int64_t n,
                           int threads, int lds, int grid, hipStream_t s) {
    switch (vec) {
    case 4: return launch_stream_u<MODE, 4>(unroll, src, dst, n, threads, lds, grid, s);
    case 8: return launch_stream_u<MODE, 8>(unroll, src, dst, n, threads, lds, grid, s);
    default: return launch_stream_u<MODE, 16>(unroll, src, dst, n, threads, lds, grid, s);
    }
}

}  // namespace

}  // namespace g355

using namespace g355;

extern "C" {

gemm355_status gemm355_stream(int mode, const void *src, void *dst, int64_t n_bytes,
                              int vec_bytes, int unroll, int threads, int lds_bytes, int grid,
                              hipStream_t stream) {
    if (mode != GEMM355_STREAM_COPY && mode != GEMM355_STREAM_READ_XOR &&
        mode != GEMM355_STREAM_COPY_NT)
        return GEMM355_ERR_INVALID_ARG;
    if (n_bytes < 0 || n_bytes % 4 != 0) return GEMM355_ERR_INVALID_ARG;
    if (vec_bytes != 4 && vec_bytes != 8 && vec_bytes != 16) return GEMM355_ERR_INVALID_ARG;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return GEMM355_ERR_INVALID_ARG;
    if (threads < 64 || threads > 1024 || threads % 64 != 0) return GEMM355_ERR_INVALID_ARG;
    if (lds_bytes < 0 || lds_bytes > kLdsMax) return GEMM355_ERR_INVALID_ARG;
    if (grid < 1 || grid > (1 << 20)) return GEMM355_ERR_INVALID_ARG;
    const bool copy = mode != GEMM355_STREAM_READ_XOR;
    if (n_bytes > 0 && src == nullptr) return GEMM355_ERR_INVALID_ARG;
    if (dst == nullptr && (!copy || n_bytes > 0)) return GEMM355_ERR_INVALID_ARG;
    if (n_bytes > 0 && (uintptr_t)src % vec_bytes != 0) return GEMM355_ERR_INVALID_ARG;
    if (copy && n_bytes > 0 && (uintptr_t)dst % vec_bytes != 0) return GEMM355_ERR_INVALID_ARG;
    if (!copy && (uintptr_t)dst % 4 != 0) return GEMM355_ERR_INVALID_ARG;
    if (copy && n_bytes > 0) {
        const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
        if (a < b + (uintptr_t)n_bytes && b < a + (uintptr_t)n_bytes) return GEMM355_ERR_INVALID_ARG;
    }
    if (!current_device_is_gfx950()) return GEMM355_ERR_DEVICE;
    if (copy && n_bytes == 0) return GEMM355_OK;
    // READ_XOR keeps one word per wave of the workgroup in the reserved LDS
    const int lds = copy ? lds_bytes : (lds_bytes > 64 ? lds_bytes : 64);
    const hipError_t e =
        mode == GEMM355_STREAM_COPY
            ? launch_stream_m<GEMM355_STREAM_COPY>(vec_bytes, unroll, src, dst, n_bytes, threads,
                                                   lds, grid, stream)
        : mode == GEMM355_STREAM_COPY_NT
            ? launch_stream_m<GEMM355_STREAM_COPY_NT>(vec_bytes, unroll, src, dst, n_bytes,
                                                      threads, lds, grid, stream)
            : launch_stream_m<GEMM355_STREAM_READ_XOR>(vec_bytes, unroll, src, dst, n_bytes,
                                                       threads, lds, grid, stream);
    return e == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

gemm355_status gemm355_chase(const uint32_t *next, int64_t n_words, uint32_t start, int hops,
                             uint64_t *dev_out, hipStream_t stream) {
    if (next == nullptr || dev_out == nullptr) return GEMM355_ERR_INVALID_ARG;
    if (n_words < 1 || n_words > (int64_t(1) << 32)) return GEMM355_ERR_INVALID_ARG;
    if ((int64_t)start >= n_words) return GEMM355_ERR_INVALID_ARG;
    if (hops < 1 || hops > (1 << 30)) return GEMM355_ERR_INVALID_ARG;
    if (!current_device_is_gfx950()) return GEMM355_ERR_DEVICE;
    hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(64), 0, stream, next,
                       (uint32_t)(n_words - 1), start, hops, dev_out);
    return hipGetLastError() == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

}  // extern "C"
