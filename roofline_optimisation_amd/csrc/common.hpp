// Internal helpers shared by the gfx950 GEMM kernels of libgemm355.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace g355 {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
// 16-byte chunks of 16-bit elements at element alignment only (rows whose stride is not
// a multiple of 16 bytes): gfx950 under the HSA ABI runs with unaligned global access
// enabled, so these still load with one global_load_dwordx4.
typedef uint16_t u16x8_ua __attribute__((ext_vector_type(8), aligned(2)));

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

// binary32 -> the 16-bit storage format, to nearest with ties to even.
__device__ __forceinline__ uint16_t to_bits(float v, f16_t) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ uint16_t to_bits(float v, bf16_t) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Arguments common to every launcher.  Pointers are device pointers; ld* are row
// strides in elements.  C = sign * op(A) op(B) (+ C when accumulate), where op(A) is A
// (M x K rows) or, with trans_a, the transpose of the stored K x M matrix, and likewise
// op(B) is B (K x N) or the transpose of the stored N x K matrix.
struct GemmArgs {
    int M, N, K;
    const void *A;
    int lda;
    const void *B;
    int ldb;
    float *C;
    int ldc;
    int trans_a = 0, trans_b = 0;
    float sign = 1.0f;
    int accumulate = 0;
    // C (and the old C when accumulating) is stored in the operands' 16-bit type: C
    // then points to uint16_t patterns and ldc counts those.
    int c16 = 0;
    // Keep the 16-bit kernels' 256 x 256 direct-to-LDS tile where the dispatcher would
    // take the 192 x 256 or 256 x 192 one (a measurement-only variant sets it).
    int square_tiles = 0;
    // Keep the 128 x 128 direct-to-LDS tile to grids of at most 256 tiles (one per CU);
    // larger grids go to the register-staged kernel (a measurement-only variant sets it).
    int one_round_128 = 0;
    int staged_small = 0;
    // The MFMA kernels have plain variants (store the accumulators as they are) and
    // variants that store sign * acc (+ C); the latter serve negated products too.
    bool signed_or_acc() const { return accumulate || sign < 0.0f; }
};

// Stores one 32 x 32 MFMA accumulator block: register r of this lane holds row
// row0 + 8 (r/4) + r%4 (row0 already includes the lane's 4 (l/32)), column col.  EDGE
// guards every access against M x N; NT uses non-temporal stores (C is not re-read).
// The values go out exactly as accumulated, straight from the accumulator registers: the
// plain variants' epilogue.  The signed and accumulating variants apply the sign (and add
// the old C) in their own epilogue, store_block32_acc below, with no extra pass.
template <bool EDGE, bool NT>
__device__ __forceinline__ void store_block32(const floatx16 &acc, float *__restrict__ C, int ldc,
                                              int row0, int col, int M, int N) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = row0 + 8 * (r / 4) + r % 4;
        float *c = C + (size_t)row * ldc + col;
        if (!EDGE || (row < M && col < N)) {
            if (NT) __builtin_nontemporal_store(acc[r], c);
            else *c = acc[r];
        }
    }
}

// The same block for the variants that apply a sign or accumulate: c = sign * acc
// (+ c when use_old; sign = +1 or -1).  The block is done in two halves of 8 rows; the
// fences keep each half's loads
// together and apart from the rest, so that few old values are live at a time.  AREAD:
// the accumulators live in the AGPR file; each is read with its own v_accvgpr_read at
// its point of use (otherwise the compiler copies all of them to VGPRs at once when the
// loop ends, which does not fit next to the loop's other registers).
template <bool EDGE, bool NT, bool AREAD>
__device__ __forceinline__ void store_block32_acc(const floatx16 &acc, float *__restrict__ C,
                                                  int ldc, int row0, int col, int M, int N,
                                                  float sign, int use_old) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __builtin_amdgcn_sched_barrier(0);
        float old[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 8 * h + q;
            const int row = row0 + 8 * (r / 4) + r % 4;
            const bool ok = use_old && (!EDGE || (row < M && col < N));
            old[q] = ok ? C[(size_t)(ok ? row : 0) * ldc + (ok ? col : 0)] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 8 * h + q;
            const int row = row0 + 8 * (r / 4) + r % 4;
            float *c = C + (size_t)row * ldc + col;
            if (!EDGE || (row < M && col < N)) {
                float a;
                if constexpr (AREAD)
                    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a) : "a"(acc[r]));
                else
                    a = acc[r];
                const float v = sign * a + old[q];
                if (NT) __builtin_nontemporal_store(v, c);
                else *c = v;
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// The same block with C in the 16-bit type T: c = round16(sign * acc (+ old c widened
// to binary32)), rounded to nearest with ties to even; two halves of 8 rows as above,
// one 2-byte access per element.  `flags` bit 0 adds the old C.
template <bool EDGE, typename T, bool AREAD>
__device__ __forceinline__ void store_block32_c16(const floatx16 &acc, uint16_t *__restrict__ C,
                                                  int ldc, int row0, int col, int M, int N,
                                                  float sign, int flags) {
    const bool use_old = flags & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __builtin_amdgcn_sched_barrier(0);
        float old[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 8 * h + q;
            const int row = row0 + 8 * (r / 4) + r % 4;
            const bool ok = use_old && (!EDGE || (row < M && col < N));
            old[q] = ok ? to_float(T{C[(size_t)(ok ? row : 0) * ldc + (ok ? col : 0)]}) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 8 * h + q;
            const int row = row0 + 8 * (r / 4) + r % 4;
            if (!EDGE || (row < M && col < N)) {
                float a;
                if constexpr (AREAD)
                    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a) : "a"(acc[r]));
                else
                    a = acc[r];
                __builtin_nontemporal_store(to_bits(sign * a + old[q], T{}),
                                            C + (size_t)row * ldc + col);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Two horizontally adjacent 32 x 32 blocks (columns col0 .. col0+63, lane l holding
// column l%32 of each) with C in the 16-bit type T.  With `flags` bit 1 (set by the host
// when ldc is even and C 4-byte aligned) each row of the pair is written as one whole
// 128-byte line: lanes 2j and 2j+1 exchange one register per row (DPP quad permute
// [1,0,3,2]; the even lane sends its block-1 value, the odd lane its block-0 value), so
// the even lane holds columns 2j, 2j+1 of block 0 and the odd lane columns 2j, 2j+1 of
// block 1, and each lane reads the old C and writes the result 4 bytes at a time.  The
// exchange runs in every lane (full EXEC) before the guarded accesses.  Without bit 1
// each block takes store_block32_c16.
template <bool EDGE, typename T, bool AREAD>
__device__ __forceinline__ void store_pair32_c16(const floatx16 &acc0, const floatx16 &acc1,
                                                 uint16_t *__restrict__ C, int ldc, int row0,
                                                 int col0, int M, int N, float sign, int flags) {
    const int lane = threadIdx.x & 63;
    if (!(flags & 2)) {
        store_block32_c16<EDGE, T, AREAD>(acc0, C, ldc, row0, col0 + (lane & 31), M, N, sign, flags);
        store_block32_c16<EDGE, T, AREAD>(acc1, C, ldc, row0, col0 + 32 + (lane & 31), M, N, sign,
                                          flags);
        return;
    }
    const bool use_old = flags & 1;
    const int odd = lane & 1;
    const int cw = col0 + (lane & 30) + 32 * odd;  // first of the two columns this lane writes
    auto rd = [&](const floatx16 &acc, int r) {
        float a;
        if constexpr (AREAD)
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a) : "a"(acc[r]));
        else
            a = acc[r];
        return a;
    };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __builtin_amdgcn_sched_barrier(0);
        float old_lo[8], old_hi[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 8 * h + q;
            const int row = row0 + 8 * (r / 4) + r % 4;
            const bool in = !EDGE || (row < M && cw < N);
            const bool both = !EDGE || cw + 1 < N;
            uint32_t w = 0;
            if (use_old && in) {
                const uint16_t *c = C + (size_t)row * ldc + cw;
                w = both ? *(const uint32_t *)c : (uint32_t)c[0];
            }
            old_lo[q] = use_old ? to_float(T{(uint16_t)(w & 0xFFFF)}) : 0.f;
            old_hi[q] = use_old ? to_float(T{(uint16_t)(w >> 16)}) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 8 * h + q;
            const float a0 = rd(acc0, r), a1 = rd(acc1, r);
            const float send = odd ? a0 : a1;
            const float recv = __builtin_bit_cast(
                float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF,
                                                   false));
            const float lo = odd ? recv : a0, hi = odd ? a1 : recv;
            const int row = row0 + 8 * (r / 4) + r % 4;
            const uint32_t w = (uint32_t)to_bits(sign * lo + old_lo[q], T{}) |
                               ((uint32_t)to_bits(sign * hi + old_hi[q], T{}) << 16);
            uint16_t *c = C + (size_t)row * ldc + cw;
            if (!EDGE || (row < M && cw + 1 < N))
                __builtin_nontemporal_store(w, (uint32_t *)c);
            else if (row < M && cw < N)
                __builtin_nontemporal_store((uint16_t)(w & 0xFFFF), c);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// One 16 x 16 accumulator quad with a sign and optional accumulation: register r of this
// lane holds row row0 + r (row0 already includes the lane's 4 (l/16)), column col;
// c = sign * acc (+ c when use_old); EDGE guards every access against M x N.  Each
// register is read from the AGPR file at its point of use (see store_block32_acc).
// Ordinary stores: a store writes 64-byte pieces of lines, which the L2 merges.
template <bool EDGE>
__device__ __forceinline__ void store_quad16_acc(const floatx4 &acc, float *__restrict__ C, int ldc,
                                                 int row0, int col, int M, int N, float sign,
                                                 bool use_old) {
    __builtin_amdgcn_sched_barrier(0);
    float old[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool ok = !EDGE || (row0 + r < M && col < N);
        old[r] = use_old && ok ? C[(size_t)(row0 + r) * ldc + col] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float a;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a) : "a"(acc[r]));
        if (!EDGE || (row0 + r < M && col < N)) C[(size_t)(row0 + r) * ldc + col] = sign * a + old[r];
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Two horizontally adjacent 16 x 16 quads (columns col0 .. col0+31, lane l holding column
// l%16 of each, rows row0 + r) with C in the 16-bit type T, c = round16(sign * acc (+ old
// c)).  With `flags` bit 1 (ldc even, C 4-byte aligned) lanes 2m and 2m+1 exchange one
// register per row as in store_pair32_c16, so the even lane writes columns 2m, 2m+1 of
// quad 0 and the odd lane those of quad 1, 4 bytes at a time; otherwise every element is
// one 2-byte access.  `flags` bit 0 adds the old C.  EDGE guards every access against
// M x N (a pair whose second column is outside is read and written 2 bytes at a time;
// the exchange itself runs in every lane).  `lane` is this lane's index in the wave.
// One row of such a pair in paired mode: the 4-byte word this lane writes, from its own
// values a0 (quad 0) and a1 (quad 1) of the row and the old word (two 16-bit values) when
// use_old.  The exchange between lanes 2m and 2m+1 runs in every lane.
template <typename T>
__device__ __forceinline__ uint32_t pair16_word(float a0, float a1, int odd, float sign, uint32_t oldw,
                                                bool use_old) {
    const float send = odd ? a0 : a1;
    const float recv = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
    const float lo = odd ? recv : a0, hi = odd ? a1 : recv;
    const float olo = use_old ? to_float(T{(uint16_t)(oldw & 0xFFFF)}) : 0.f;
    const float ohi = use_old ? to_float(T{(uint16_t)(oldw >> 16)}) : 0.f;
    return (uint32_t)to_bits(sign * lo + olo, T{}) | ((uint32_t)to_bits(sign * hi + ohi, T{}) << 16);
}

template <bool EDGE, typename T>
__device__ __forceinline__ void store_pair16_c16(const floatx4 &acc0, const floatx4 &acc1,
                                                 uint16_t *__restrict__ C, int ldc, int row0,
                                                 int col0, int M, int N, float sign, int flags,
                                                 int lane) {
    const bool use_old = flags & 1;
    auto rd = [&](const floatx4 &acc, int r) {
        float a;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a) : "a"(acc[r]));
        return a;
    };
    __builtin_amdgcn_sched_barrier(0);
    if (!(flags & 2)) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = col0 + 16 * q + (lane & 15);
                const bool ok = !EDGE || (row0 + r < M && col < N);
                uint16_t *c = C + (size_t)(row0 + r) * ldc + col;
                const float old = use_old && ok ? to_float(T{*c}) : 0.f;
                const uint16_t v = to_bits(sign * rd(q ? acc1 : acc0, r) + old, T{});
                if (ok) *c = v;
            }
        __builtin_amdgcn_sched_barrier(0);
        return;
    }
    const int odd = lane & 1;
    const int cw = col0 + (lane & 14) + 16 * odd;  // first of the two columns this lane writes
    uint32_t oldw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint16_t *c = C + (size_t)(row0 + r) * ldc + cw;
        const bool in = !EDGE || (row0 + r < M && cw < N), both = !EDGE || cw + 1 < N;
        oldw[r] = use_old && in ? (both ? *(const uint32_t *)c : (uint32_t)c[0]) : 0u;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t w = pair16_word<T>(rd(acc0, r), rd(acc1, r), odd, sign, oldw[r], use_old);
        uint16_t *c = C + (size_t)(row0 + r) * ldc + cw;
        if (!EDGE || (row0 + r < M && cw + 1 < N)) *(uint32_t *)c = w;
        else if (row0 + r < M && cw < N) *c = (uint16_t)(w & 0xFFFF);
    }
    __builtin_amdgcn_sched_barrier(0);
}

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
