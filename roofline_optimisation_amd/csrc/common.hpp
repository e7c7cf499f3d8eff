// Internal helpers shared by the gfx950 GEMM kernels of libgemm355.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g355 {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Operand storage types: float, or 16-bit patterns tagged by format.
struct f16_t { uint16_t bits; };
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_float(float x) { return x; }
__device__ __forceinline__ float to_float(f16_t x) {
    return (float)__builtin_bit_cast(_Float16, x.bits);
}
__device__ __forceinline__ float to_float(bf16_t x) {
    return __builtin_bit_cast(float, (uint32_t)x.bits << 16);
}

// Arguments common to every launcher.  Pointers are device pointers; ld* are row
// strides in elements.
struct GemmArgs {
    int M, N, K;
    const void *A;
    int lda;
    const void *B;
    int ldb;
    float *C;
    int ldc;
};

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Workgroups are handed to the 8 XCDs of an MI355X round-robin (workgroup i runs on
// XCD i mod 8).  Renumber so that each XCD receives a contiguous range of logical tile
// ids; combined with the grouped tile order below, the tiles that share A row panels
// and B column panels then share one XCD's L2.
__device__ __forceinline__ int xcd_contiguous_id(int bid, int nblocks) {
    constexpr int kXcd = 8;
    const int full = (nblocks / kXcd) * kXcd;
    if (bid >= full) return bid;
    const int per = full / kXcd;
    return (bid % kXcd) * per + bid / kXcd;
}

// Grouped tile order: walk `group` tile-rows at a time, tile-row fastest, so that
// consecutive ids form compact group x (run) blocks of the tile grid.
__device__ __forceinline__ void grouped_tile(int id, int tiles_m, int tiles_n, int group,
                                             int &tm, int &tn) {
    const int per_group = group * tiles_n;
    const int g = id / per_group;
    const int first_m = g * group;
    const int rows = min(group, tiles_m - first_m);
    const int in = id - g * per_group;
    tm = first_m + in % rows;
    tn = in / rows;
}

}  // namespace g355
