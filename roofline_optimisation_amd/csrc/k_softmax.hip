// Row-wise softmax and row sum in binary32.
//
// The method is the online softmax of "Kernel optimisation guide" (section on softmax
// optimisation): a running maximum m and a running sum l of exp(x - m), the sum
// rescaled by exp(m_old - m_new) whenever the maximum rises, then y = exp(x - m) / l.
// Its section on warp-shuffle reduction supplies the cross-lane combine.
//
// gfx950 mapping (the op is bound by HBM: 4 bytes read and 4 written per element):
//  * A row is held in registers by 64 * WPR lanes, E elements each (WPR waves per row;
//    one wave per row and four waves per workgroup for rows of up to 512, a wave taking
//    two rows of up to 256).  Loads are
//    16-byte vectors when the rows allow it (lane t's vector q covers columns
//    4 (q T + t) .. +3, so each load instruction reads 1 KiB contiguous per wave);
//    every load of the row is issued before the first is used.
//  * Each lane applies the recurrence to its own elements as one block: its maximum m_t,
//    then e_i = exp(x_i - m_t) and l_t = sum e_i, keeping the e_i.
//  * The (m, l) pairs are merged across the wave by register exchange (DPP and swizzle)
//    and across the waves through LDS, each merge being the recurrence's rescale of the
//    pair with the smaller maximum: (m, l) = (m_hi, l_hi + l_lo exp(m_lo - m_hi)).
//  * Each lane then writes y_i = e_i * (exp(m_t - m) / l): one exponential per element,
//    and the row is read from memory once.  The stores are non-temporal (no L2 lines
//    allocated for the results): measured 1-7 % faster than ordinary stores with the data
//    in HBM (20 % for the two-pass rows), 15-30 % when it sits in the last-level cache.
//  * Rows longer than 32768 elements stream: pass 1 applies the recurrence chunk by
//    chunk (16 elements per lane per chunk), pass 2 re-reads the row and writes
//    exp(x - m) * (1 / l).
// The row sum uses the same layout and exchanges with + as the combine.
#include "../../include/gemm355_softmax.h"
#include "common.hpp"
#include "launch.hpp"
#include "wave_reduce.hpp"

namespace g355 {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxResident = 32768;  // longest row held in registers (1024 lanes x 32)
constexpr int kMaxCols = 1 << 30;    // column indexes below plus one chunk stay in int
constexpr int kMaxRows = 1 << 30;    // row indexes (workgroup x 4 + wave) x R stay in int

// Merge (m, l) with another running (maximum, sum) pair: the pair with the smaller
// maximum is rescaled to the larger.  Equal maxima (including two empty pairs, m =
// -infinity) add the sums unscaled.  Commutative, so exchanges leave every lane equal.
__device__ __forceinline__ void merge_ml(float &m, float &l, float mo, float lo) {
    const bool mine = m >= mo;
    const float hi = mine ? m : mo, low = mine ? mo : m;
    const float lhi = mine ? l : lo, llo = mine ? lo : l;
    const float f = (low == hi) ? 1.0f : expf(low - hi);
    m = hi;
    l = lhi + llo * f;
}

struct MergeMl {
    __device__ __forceinline__ void operator()(float &m, float &l, float mo, float lo) const {
        merge_ml(m, l, mo, lo);
    }
};

// Row r's statistics merged over its WPR waves: waves publish their pairs to LDS, then
// every lane merges them in wave order (the same sequence in every lane).
template <int WPR>
__device__ __forceinline__ void block_merge(float &m, float &l, float *sm, float *sl, int wave,
                                            int lane) {
    wave_allreduce2(m, l, MergeMl{});
    if constexpr (WPR > 1) {
        if (lane == 0) {
            sm[wave] = m;
            sl[wave] = l;
        }
        __syncthreads();
        m = sm[0];
        l = sl[0];
#pragma unroll
        for (int w = 1; w < WPR; ++w) merge_ml(m, l, sm[w], sl[w]);
    }
}

template <int WPR>
constexpr int block_threads() { return WPR == 1 ? 256 : 64 * WPR; }

// Results are written with non-temporal stores, which stream past the L2 without
// allocating lines there.
__device__ __forceinline__ void store_nt(float *p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt4(float *p, float a, float b, float c, float d) {
    __builtin_nontemporal_store(f32x4{a, b, c, d}, (f32x4 *)p);
}

// Rows of at most 64 * WPR * E elements, held in registers.  With one wave per row
// (WPR == 1) each wave takes R consecutive rows and issues the loads of all of them
// before it reduces the first.
template <int E, int WPR, int R, bool VEC>
__global__ __launch_bounds__(block_threads<WPR>()) void softmax_rows_kernel(
    int rows, int cols, const float *__restrict__ X, int ldx, float *Y, int ldy) {
    constexpr int T = 64 * WPR;
    static_assert(!VEC || E % 4 == 0, "vector loads take 4 elements");
    static_assert(WPR == 1 || R == 1, "several rows per workgroup only with one wave per row");
    __shared__ float sm[WPR], sl[WPR];
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int row0 = WPR == 1 ? (blockIdx.x * 4 + wave) * R : blockIdx.x;
    const int t = WPR == 1 ? lane : (int)threadIdx.x;
    if (WPR == 1 && row0 >= rows) return;  // a whole wave; no barrier in this shape

    // element e of this lane: column col(e); with vectors, 4 consecutive per vector
    auto col = [&](int e) { return VEC ? 4 * ((e / 4) * T + t) + e % 4 : e * T + t; };
    float v[R][E];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool in = row0 + r < rows;
        const float *x = X + (size_t)(row0 + r) * ldx;
        if constexpr (VEC) {
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                const int c = 4 * (q * T + t);
                float4 f = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
                if (in && c < cols) f = *(const float4 *)(x + c);  // cols % 4 == 0: whole vector in the row
                v[r][4 * q] = f.x;
                v[r][4 * q + 1] = f.y;
                v[r][4 * q + 2] = f.z;
                v[r][4 * q + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int c = col(e);
                v[r][e] = in && c < cols ? x[c] : kNegInf;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float m = kNegInf;
#pragma unroll
        for (int e = 0; e < E; ++e) m = fmaxf(m, v[r][e]);
        // a lane with no element of the row keeps m = -inf and l = 0; shifting by 0 then
        // keeps its exponentials at exp(-inf) = 0
        const float shift = m == kNegInf ? 0.0f : m;
        float l = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            v[r][e] = expf(v[r][e] - shift);
            l += v[r][e];
        }
        float M = m, L = l;
        block_merge<WPR>(M, L, sm, sl, wave, lane);
        const float s = expf(m - M) / L;
        if (row0 + r >= rows) continue;  // past the last row: nothing to write
        float *y = Y + (size_t)(row0 + r) * ldy;
        if constexpr (VEC) {
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                const int c = 4 * (q * T + t);
                if (c < cols)
                    store_nt4(y + c, v[r][4 * q] * s, v[r][4 * q + 1] * s, v[r][4 * q + 2] * s,
                              v[r][4 * q + 3] * s);
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int c = col(e);
                if (c < cols) store_nt(y + c, v[r][e] * s);
            }
        }
    }
}

// Rows longer than the resident limit: one workgroup of 1024 lanes per row, two passes.
template <bool VEC>
__global__ __launch_bounds__(1024) void softmax_long_kernel(int rows, int cols,
                                                            const float *__restrict__ X, int ldx,
                                                            float *Y, int ldy) {
    constexpr int T = 1024, E = 16, CH = T * E;
    __shared__ float sm[16], sl[16];
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, t = threadIdx.x;
    const float *x = X + (size_t)blockIdx.x * ldx;
    float *y = Y + (size_t)blockIdx.x * ldy;
    auto load_chunk = [&](int base, float (&v)[E]) {
        if constexpr (VEC) {
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                const int c = base + 4 * (q * T + t);
                float4 f = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
                if (c < cols) f = *(const float4 *)(x + c);
                v[4 * q] = f.x;
                v[4 * q + 1] = f.y;
                v[4 * q + 2] = f.z;
                v[4 * q + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int c = base + e * T + t;
                v[e] = c < cols ? x[c] : kNegInf;
            }
        }
    };
    // pass 1: the recurrence over this lane's chunks, one chunk at a time
    float m = kNegInf, l = 0.0f;
    for (int base = 0; base < cols; base += CH) {
        float v[E];
        load_chunk(base, v);
        float cm = kNegInf;
#pragma unroll
        for (int e = 0; e < E; ++e) cm = fmaxf(cm, v[e]);
        if (cm > m) {
            l *= expf(m - cm);
            m = cm;
        }
        const float shift = m == kNegInf ? 0.0f : m;
#pragma unroll
        for (int e = 0; e < E; ++e) l += expf(v[e] - shift);
    }
    float M = m, L = l;
    block_merge<16>(M, L, sm, sl, wave, lane);
    const float inv = 1.0f / L;
    // pass 2: normalise
    for (int base = 0; base < cols; base += CH) {
        float v[E];
        load_chunk(base, v);
        if constexpr (VEC) {
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                const int c = base + 4 * (q * T + t);
                if (c < cols)
                    store_nt4(y + c, expf(v[4 * q] - M) * inv, expf(v[4 * q + 1] - M) * inv,
                              expf(v[4 * q + 2] - M) * inv, expf(v[4 * q + 3] - M) * inv);
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int c = base + e * T + t;
                if (c < cols) store_nt(y + c, expf(v[e] - M) * inv);
            }
        }
    }
}

// Row sums: each lane adds its elements in order (U vectors or scalars per lane in
// flight per iteration, loaded non-temporally: each is read once), then the lanes' sums
// are combined across the wave and, in wave order, across the workgroup.
template <int WPR, bool VEC>
__global__ __launch_bounds__(block_threads<WPR>()) void row_sum_kernel(int rows, int cols,
                                                                       const float *__restrict__ X,
                                                                       int ldx, float *out) {
    constexpr int T = 64 * WPR, U = 4;
    __shared__ float ss[WPR];
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int row = WPR == 1 ? blockIdx.x * 4 + wave : blockIdx.x;
    const int t = WPR == 1 ? lane : (int)threadIdx.x;
    if (WPR == 1 && row >= rows) return;
    const float *x = X + (size_t)row * ldx;
    float acc = 0.0f;
    if constexpr (VEC) {
        for (int base = 0; base < cols; base += 4 * T * U) {
            float4 f[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = base + 4 * (u * T + t);
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                if (c < cols) z = __builtin_nontemporal_load((const f32x4 *)(x + c));
                f[u] = make_float4(z[0], z[1], z[2], z[3]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc = ((acc + f[u].x) + f[u].y + f[u].z) + f[u].w;
        }
    } else {
        for (int base = 0; base < cols; base += T * U) {
            float f[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = base + u * T + t;
                f[u] = c < cols ? __builtin_nontemporal_load(x + c) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc += f[u];
        }
    }
    float s = wave_allreduce_sum(acc);
    if constexpr (WPR > 1) {
        if (lane == 0) ss[wave] = s;
        __syncthreads();
        s = ss[0];
#pragma unroll
        for (int w = 1; w < WPR; ++w) s += ss[w];
        if (threadIdx.x == 0) out[row] = s;
    } else {
        if (lane == 0) out[row] = s;
    }
}

template <int E, int WPR, int R, bool VEC>
hipError_t launch_rows(int rows, int cols, const float *X, int ldx, float *Y, int ldy,
                       hipStream_t s) {
    const int grid = WPR == 1 ? cdiv(rows, 4 * R) : rows;
    hipLaunchKernelGGL((softmax_rows_kernel<E, WPR, R, VEC>), dim3(grid),
                       dim3(block_threads<WPR>()), 0, s, rows, cols, X, ldx, Y, ldy);
    return hipGetLastError();
}

template <bool VEC>
hipError_t launch_softmax(int rows, int cols, const float *X, int ldx, float *Y, int ldy,
                          hipStream_t s) {
    // (elements per lane, waves per row, rows per wave) by row length, from a sweep of
    // the 64 Mi-element workloads
    if (cols <= 256) return launch_rows<4, 1, 2, VEC>(rows, cols, X, ldx, Y, ldy, s);
    if (cols <= 512) return launch_rows<8, 1, 1, VEC>(rows, cols, X, ldx, Y, ldy, s);
    if (cols <= 1024) return launch_rows<8, 2, 1, VEC>(rows, cols, X, ldx, Y, ldy, s);
    if (cols <= 2048) return launch_rows<8, 4, 1, VEC>(rows, cols, X, ldx, Y, ldy, s);
    if (cols <= 4096) return launch_rows<32, 2, 1, VEC>(rows, cols, X, ldx, Y, ldy, s);
    if (cols <= 8192) return launch_rows<32, 4, 1, VEC>(rows, cols, X, ldx, Y, ldy, s);
    if (cols <= 16384) return launch_rows<16, 16, 1, VEC>(rows, cols, X, ldx, Y, ldy, s);
    if (cols <= kMaxResident) {
        // one element per load: 64 per lane would need more scalar registers than exist
        if constexpr (VEC) return launch_rows<64, 8, 1, true>(rows, cols, X, ldx, Y, ldy, s);
        else return launch_rows<32, 16, 1, false>(rows, cols, X, ldx, Y, ldy, s);
    }
    hipLaunchKernelGGL((softmax_long_kernel<VEC>), dim3(rows), dim3(1024), 0, s, rows, cols, X,
                       ldx, Y, ldy);
    return hipGetLastError();
}

template <int WPR, bool VEC>
hipError_t launch_sum_w(int rows, int cols, const float *X, int ldx, float *out, hipStream_t s) {
    const int grid = WPR == 1 ? cdiv(rows, 4) : rows;
    hipLaunchKernelGGL((row_sum_kernel<WPR, VEC>), dim3(grid), dim3(block_threads<WPR>()), 0, s,
                       rows, cols, X, ldx, out);
    return hipGetLastError();
}

template <bool VEC>
hipError_t launch_row_sum(int rows, int cols, const float *X, int ldx, float *out,
                          hipStream_t s) {
    if (cols <= 2048) return launch_sum_w<1, VEC>(rows, cols, X, ldx, out, s);
    if (cols <= 16384) return launch_sum_w<4, VEC>(rows, cols, X, ldx, out, s);
    return launch_sum_w<16, VEC>(rows, cols, X, ldx, out, s);
}

// Byte span [first, last) of a rows x cols matrix with row stride ld.
inline void span_of(const void *p, int rows, int cols, int ld, uintptr_t &a, uintptr_t &b) {
    a = (uintptr_t)p;
    b = a + ((size_t)(rows - 1) * ld + cols) * sizeof(float);
}

inline bool vec_ok(const void *p, int ld) { return (uintptr_t)p % 16 == 0 && ld % 4 == 0; }

}  // namespace

}  // namespace g355

using namespace g355;

extern "C" {

gemm355_status gemm355_softmax_f32(int rows, int cols, const float *X, int ldx, float *Y,
                                   int ldy, hipStream_t stream) {
    const int need = cols > 1 ? cols : 1;
    if (rows < 0 || rows > kMaxRows || cols < 0 || cols > kMaxCols || ldx < need || ldy < need)
        return GEMM355_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return GEMM355_OK;
    if (X == nullptr || Y == nullptr) return GEMM355_ERR_INVALID_ARG;
    if ((const void *)X == (const void *)Y) {
        if (ldx != ldy) return GEMM355_ERR_INVALID_ARG;
    } else {
        uintptr_t x0, x1, y0, y1;
        span_of(X, rows, cols, ldx, x0, x1);
        span_of(Y, rows, cols, ldy, y0, y1);
        if (x0 < y1 && y0 < x1) return GEMM355_ERR_INVALID_ARG;
    }
    if (!current_device_is_gfx950()) return GEMM355_ERR_DEVICE;
    const bool vec = cols % 4 == 0 && vec_ok(X, ldx) && vec_ok(Y, ldy);
    const hipError_t e = vec ? launch_softmax<true>(rows, cols, X, ldx, Y, ldy, stream)
                             : launch_softmax<false>(rows, cols, X, ldx, Y, ldy, stream);
    return e == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

gemm355_status gemm355_row_sum_f32(int rows, int cols, const float *X, int ldx, float *out,
                                   hipStream_t stream) {
    if (rows < 0 || rows > kMaxRows || cols < 0 || cols > kMaxCols || ldx < (cols > 1 ? cols : 1))
        return GEMM355_ERR_INVALID_ARG;
    if (rows == 0) return GEMM355_OK;
    if (out == nullptr || (cols > 0 && X == nullptr)) return GEMM355_ERR_INVALID_ARG;
    if (cols > 0) {
        uintptr_t x0, x1;
        span_of(X, rows, cols, ldx, x0, x1);
        const uintptr_t o0 = (uintptr_t)out, o1 = o0 + (size_t)rows * sizeof(float);
        if (x0 < o1 && o0 < x1) return GEMM355_ERR_INVALID_ARG;
    }
    if (!current_device_is_gfx950()) return GEMM355_ERR_DEVICE;
    const bool vec = cols % 4 == 0 && vec_ok(X, ldx);
    const hipError_t e = vec ? launch_row_sum<true>(rows, cols, X, ldx, out, stream)
                             : launch_row_sum<false>(rows, cols, X, ldx, out, stream);
    return e == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

}  // extern "C"
