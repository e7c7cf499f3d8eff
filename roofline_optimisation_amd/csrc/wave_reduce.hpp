// Reductions across the 64 lanes of a wave by register exchange (CDNA4).
//
// "Kernel optimisation guide" (section on warp-shuffle reduction) sums a value over a
// 32-lane warp by adding, at halving distances, the value another lane holds.  On a
// 64-lane gfx950 wave the exchanges that need no memory are:
//  * DPP operand modifiers, which let a VALU instruction read its operand from another
//    lane of the same row of 16: quad permutes (partner lane l ^ 1, l ^ 2), the half-row
//    mirror (lane i of each 8 reads lane 7 - i) and the row mirror (i reads 15 - i);
//  * ds_swizzle in bit-mask mode, which swaps the two 16-lane halves of each 32 lanes
//    through the LDS crossbar without touching LDS memory;
//  * v_readlane, which reads lane 0 and lane 32 into scalar registers.
// The mirrors are not exchanges at a fixed distance, but once every quad (then every 8,
// then every 16) holds one value, a mirror pairs each lane with a lane of the other quad
// (8, 16), which is all a reduction needs.  With a commutative combine (IEEE + and max
// are) every lane ends with the same bits.  All 64 lanes must be active.
#pragma once

#include <hip/hip_runtime.h>

namespace g355 {

template <int CTRL>
struct DppXchg {
    static __device__ __forceinline__ float get(float v) {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
    }
};

struct SwapHalves16 {
    // bit-mask swizzle: and_mask 0x1F, or_mask 0, xor_mask 0x10
    static __device__ __forceinline__ float get(float v) {
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    }
};

__device__ __forceinline__ float read_lane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Combine a pair of values (a, b) over the wave with `op(a, b, a_other, b_other)`, which
// updates (a, b) in place and must be commutative in its two pairs.
template <class X, class Op>
__device__ __forceinline__ void xchg_step(float &a, float &b, Op op) {
    const float ao = X::get(a), bo = X::get(b);
    op(a, b, ao, bo);
}

template <class Op>
__device__ __forceinline__ void wave_allreduce2(float &a, float &b, Op op) {
    xchg_step<DppXchg<kDppQuadXor1>>(a, b, op);
    xchg_step<DppXchg<kDppQuadXor2>>(a, b, op);
    xchg_step<DppXchg<kDppRowHalfMirror>>(a, b, op);
    xchg_step<DppXchg<kDppRowMirror>>(a, b, op);
    xchg_step<SwapHalves16>(a, b, op);
    float a0 = read_lane(a, 0), b0 = read_lane(b, 0);
    op(a0, b0, read_lane(a, 32), read_lane(b, 32));
    a = a0;
    b = b0;
}

// Sum over the 64 lanes; every lane returns the same value.
__device__ __forceinline__ float wave_allreduce_sum(float v) {
    v += DppXchg<kDppQuadXor1>::get(v);
    v += DppXchg<kDppQuadXor2>::get(v);
    v += DppXchg<kDppRowHalfMirror>::get(v);
    v += DppXchg<kDppRowMirror>::get(v);
    v += SwapHalves16::get(v);
    return read_lane(v, 0) + read_lane(v, 32);
}

}  // namespace g355
