// FP16 / BF16 GEMM with FP32 accumulation on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_f16 / _bf16): the AMD counterpart of the tensor-core level of
// "Kernel optimisation guide" (Level 4: 16-bit A and B fragments, FP32 accumulator
// fragments, one matrix multiply-accumulate per fragment step) and of the tensor-core
// section of "Advanced CUDA features - starting from GEMM" (a wave-cooperative
// D = A.B + C unit whose register layout the data movement has to match; its table of
// tensor-core instructions lists transposed and negated operands and D scaled by 0 or 1,
// which the operand kinds and the epilogue below provide).
//
// Structure:
//  * a workgroup of WM x WN waves owns a BM x BN tile of C and walks K in steps of
//    BK = 64 with two LDS stages: the dwordx4 loads of step t+1 are in flight while
//    step t is multiplied, then written to the other stage before the one barrier of
//    the step (the double buffer of "Kernel optimisation guide", Level 3);
//  * each wave owns (BM/WM) x (BN/WN) of C as 32 x 32 FP32 accumulator blocks;
//  * the MFMA wants, per lane l of a fragment, 8 consecutive k of row (A) or column (B)
//    l%32 at k = 8(l/32) .. +7 of a 16-wide k step.  An operand stored with k
//    contiguous (kind KM: A of C = A.B, or a transposed B) is kept [m or n][k] in LDS
//    with rows padded to 144 bytes and read with one ds_read_b128 per fragment (the 32
//    rows one instruction touches fall on distinct bank groups).  An operand stored
//    with m or n contiguous (kind MN: B, or a transposed A) stays [k][m or n] in LDS as
//    loaded, rows padded to 2*extent + 64 bytes, and two ds_read_b64_tr_b16 per
//    fragment transpose it on the way out.  Within each 16-lane group that instruction
//    hands output lane j, as its element e, halfword j%4 of the 8 bytes read by source
//    lane 4e + (j%16)/4; so source lane 4e + q addresses row k+e, columns c + 4q ..
//    c + 4q + 3, and output lane j receives column c + j%16 for rows k .. k+3;
//  * interior tiles (inside M x N, K a multiple of BK) run a straight-line kernel; the
//    ragged strips run a predicated one that zero-fills loads and guards stores;
//  * C = sign * op(A) op(B) (+ C): the epilogue kind EPI selects what the stores do:
//    0 stores the FP32 accumulators as they are; 1 stores sign * acc in FP32, adding the
//    old C (loaded block by block in the epilogue) when accumulating; 2 does the same
//    with C in the operands' 16-bit type (old C widened, result rounded to nearest even).
//
// Square 256 x 256, 128 x 128 or 64 x 64 tiles (and 192 x 256, 256 x 192) take a second
// design (dma_tile in h16_dma.hpp) when K is a multiple of 8 and at least one trip of its
// ring (128 or 256), rows are 16-byte aligned and the m/n-contiguous
// extents are multiples of 8; ragged tiles included: the tiles go from memory straight
// into LDS (buffer_load_dwordx4 ... lds) through a ring of k-steps, so no registers stage
// them and no LDS store instructions are issued; LDS rows are XOR-swizzled instead of
// padded; the arithmetic is v_mfma_f32_16x16x32 on 16 x 16 accumulator quads.  Its MFMAs
// sum each 32-wide k-step in one instruction where this kernel's take two 16-wide ones,
// so the two kernels' results may differ in rounding (both are within the
// FP32-accumulation tolerance; on integer-valued inputs both are exact).
#pragma once

#include <type_traits>
#include <utility>

#include "common.hpp"
#include "launch.hpp"

namespace g355 {

namespace {

constexpr int kBK = 64;
constexpr int kSA = kBK + 8;  // KM operand LDS row stride in halves (144 bytes)

// One operand of the product as the staged kernel holds it.  MN: rows are k (kBK of
// them), E halves each; KM: rows are m or n (E of them), kBK halves each.
template <bool MN, int E, int TT>
struct H16Op {
    static constexpr int kStride = MN ? E + 32 : kSA;          // LDS row stride (halves)
    static constexpr int kRows = MN ? kBK : E;
    static constexpr int kLds = kRows * kStride;               // halves per stage
    static constexpr int kPerRow = (MN ? E : kBK) / 8;         // 16-byte chunks per row
    static constexpr int kChunks = kRows * kPerRow / TT;       // per thread
    static constexpr int kRowStep = TT / kPerRow;
    static constexpr int kPieces = MN ? 2 : 1;                 // LDS reads per fragment
    static_assert((kRows * kPerRow) % TT == 0 && TT % kPerRow == 0,
                  "tile chunks must divide over the threads");
};

template <int BM, int BN, int WM, int WN, bool A_MN, bool B_MN>
struct H16Cfg {
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kTM = BM / WM, kTN = BN / WN;
    static constexpr int kMB = kTM / 32, kNB = kTN / 32;
    using OA = H16Op<A_MN, BM, kThreads>;
    using OB = H16Op<B_MN, BN, kThreads>;
    static constexpr int kLdsA = OA::kLds, kLdsB = OB::kLds;   // halves per stage
    static constexpr int kLdsBytes = 2 * (kLdsA + kLdsB) * 2;
    static_assert(kTM % 32 == 0 && kTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

template <typename T>
__device__ __forceinline__ floatx16 mfma32x32x16(u16x8 a, u16x8 b, floatx16 c);
template <>
__device__ __forceinline__ floatx16 mfma32x32x16<f16_t>(u16x8 a, u16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                  __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ floatx16 mfma32x32x16<bf16_t>(u16x8 a, u16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) u16x8 lds_u16x8;

// An LDS address held in its own VGPR: the empty asm hides its relation to other
// addresses, so the compiler keeps one base per (stage, region) and addresses every
// access as base + immediate (DS immediates are 16 bits) instead of adding large
// constants to a shared base inside the loop.
__device__ __forceinline__ lds_u16 *lds_base(lds_u16 *p) {
    uint32_t a = (uint32_t)(uintptr_t)p;
    asm volatile("" : "+v"(a));
    return (lds_u16 *)(uintptr_t)a;
}

__device__ __forceinline__ u16x8 join(shortx4 lo, shortx4 hi) {
    return __builtin_bit_cast(u16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Columns [c, c+8) of one row.  EDGE: zero outside [0, ncols) and for invalid rows;
// otherwise the chunk is known to be inside the matrix.
template <bool VEC, bool EDGE>
__device__ __forceinline__ u16x8 ld_chunk8(const uint16_t *__restrict__ row, int c, int ncols,
                                           bool row_ok) {
    if (!EDGE || (row_ok && c + 8 <= ncols))
        return VEC ? *reinterpret_cast<const u16x8 *>(row + c)
                   : *reinterpret_cast<const u16x8_ua *>(row + c);
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (!row_ok) return v;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (!EDGE || c + e < ncols) v[e] = row[c + e];
    return v;
}

// Ragged-tile chunks without branches: the load reads the 8 elements at column
// min(c, ncols - 8) of row min(r, nrows - 1), always inside the matrix (ncols >= 8), and
// the staging to LDS moves element c + e down to slot e (shift d = c - clamped column)
// and zeroes the slots past the row's end or of a row past the matrix (nv = elements
// kept).  Loads and fix-ups are apart in time, so the loads stay in flight like the
// interior kernel's.
struct ChunkPos { int row, col, nrows, ncols; };

__device__ __forceinline__ u16x8 fix_chunk8(u16x8 v, int d, int nv) {
    const u32x4 w = __builtin_bit_cast(u32x4, v);
    const int q = min(d, 7) >> 1;
    const bool h = (d & 1) != 0;
    uint32_t x[5];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        x[i] = i + q >= 3 ? w[3] : i + q == 2 ? w[2] : i + q == 1 ? w[1] : w[0];
    x[4] = w[3];
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t sh = __builtin_amdgcn_alignbit(x[i + 1], x[i], 16);
        const uint32_t m = 2 * i + 1 < nv ? 0xffffffffu : 2 * i < nv ? 0x0000ffffu : 0u;
        y[i] = (h ? sh : x[i]) & m;
    }
    return __builtin_bit_cast(u16x8, y);
}

// Fragment registers of one operand: a KM fragment is one ds_read_b128, an MN fragment
// the two halves of two ds_read_b64_tr_b16.
template <bool MN, int NBLK>
struct H16Frag {
    u16x8 f[2][NBLK];
    __device__ __forceinline__ u16x8 get(int slot, int b) const { return f[slot][b]; }
};
template <int NBLK>
struct H16Frag<true, NBLK> {
    shortx4 f[2][NBLK][2];
    __device__ __forceinline__ u16x8 get(int slot, int b) const {
        return join(f[slot][b][0], f[slot][b][1]);
    }
};

// LOAD: 0 = dwordx4 at 2-byte alignment (rows not 16-byte aligned), 1 = dwordx4
// through pointers, 2 = dwordx4 through buffer resources (interior tiles, offsets
// below 2^31 bytes), 3 (ragged tiles, contiguous extents of at least 8) = dwordx4 at
// 2-byte alignment clamped into the matrix, fixed up when staged (fix_chunk8); the
// predicated ragged kernel (EDGE with LOAD 0 or 1) branches per element instead.
template <typename T, int BM, int BN, int WM, int WN, int LOAD, bool EDGE, bool PAIRED,
          bool A_MN, bool B_MN, int EPI>
__device__ __forceinline__ void h16_tile(int M, int N, int K, const uint16_t *__restrict__ A,
                                         int lda, const uint16_t *__restrict__ B, int ldb,
                                         float *__restrict__ C, int ldc, float sign,
                                         int use_old, int m0, int n0, uint16_t *lds) {
    using Cfg = H16Cfg<BM, BN, WM, WN, A_MN, B_MN>;
    using OA = typename Cfg::OA;
    using OB = typename Cfg::OB;
    constexpr int MB = Cfg::kMB, NB = Cfg::kNB;
    constexpr int kAC = OA::kChunks, kBC = OB::kChunks;

    const int t = threadIdx.x;
    const int lane = t % 64, wave = t / 64;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane % 32, lhi = lane / 32;
    // Chunk i of a thread: row r0 + kRowStep i, column c0 of the operand's LDS image.
    const int a_r0 = t / OA::kPerRow, a_c0 = (t % OA::kPerRow) * 8;
    const int b_r0 = t / OB::kPerRow, b_c0 = (t % OB::kPerRow) * 8;

    // Global addressing of chunk (r, c) of a k-step at k0.  KM: row mn0 + r, column
    // k0 + c; MN: row k0 + r, column mn0 + c.  Interior tiles read through buffer
    // resources based at the tile's first row (KM) or first column (MN): one VGPR
    // offset per operand, the chunk and k-step parts in SGPRs.
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A_MN ? A + m0 : A + (size_t)m0 * lda), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(B_MN ? B + n0 : B + (size_t)n0 * ldb), (short)0, 0x7fffffff, 0x00020000);
    const int va = (a_r0 * lda + a_c0) * 2, vb = (b_r0 * ldb + b_c0) * 2;

    // Two staging register sets: the loads of k-step t+3 are issued while step t is
    // multiplied and written to LDS two steps later.
    u16x8 sa[2][kAC], sb[2][kBC];
    // Global -> register staging, one 16-byte chunk per call (chunk w < kAC is A's,
    // the rest B's).
    auto op_chunk = [&](auto mn_c, const uint16_t *__restrict__ X, int ld, int mn0, int MNext,
                        int r, int c, int k0) -> u16x8 {
        constexpr bool kMN = decltype(mn_c)::value;
        const int row = kMN ? k0 + r : mn0 + r;
        const int col = kMN ? mn0 + c : k0 + c;
        const bool ok = !EDGE || row < (kMN ? K : MNext);
        return ld_chunk8<LOAD == 1, EDGE>(X + (size_t)(ok ? row : 0) * ld, col,
                                          kMN ? MNext : K, ok);
    };
    // LOAD 3: chunk (r, c) of the k-step at k0 as a position in its operand.
    auto chunk_pos = [&](auto mn_c, int mn0, int MNext, int r, int c, int k0) -> ChunkPos {
        constexpr bool kMN = decltype(mn_c)::value;
        return kMN ? ChunkPos{k0 + r, mn0 + c, K, MNext} : ChunkPos{mn0 + r, k0 + c, MNext, K};
    };
    auto pos_of = [&](int w, int k0) -> ChunkPos {
        if (w < kAC)
            return chunk_pos(std::integral_constant<bool, A_MN>{}, m0, M, a_r0 + w * OA::kRowStep, a_c0, k0);
        return chunk_pos(std::integral_constant<bool, B_MN>{}, n0, N,
                         b_r0 + (w - kAC) * OB::kRowStep, b_c0, k0);
    };
    auto load_one = [&](auto set_c, int k0, int w) {
        constexpr int S = decltype(set_c)::value;
        if constexpr (LOAD == 3) {
            const ChunkPos p = pos_of(w, k0);
            const uint16_t *X = w < kAC ? A : B;
            const int ld = w < kAC ? lda : ldb;
            const u16x8 v = *reinterpret_cast<const u16x8_ua *>(
                X + (size_t)min(p.row, p.nrows - 1) * ld + min(p.col, p.ncols - 8));
            if (w < kAC) sa[S][w] = v;
            else sb[S][w - kAC] = v;
        } else if constexpr (LOAD == 2) {
            if (w < kAC) {
                const int so = A_MN ? (k0 + w * OA::kRowStep) * lda * 2
                                    : (w * OA::kRowStep * lda + k0) * 2;
                sa[S][w] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(ra, va, so, 0));
            } else {
                const int i = w - kAC;
                const int so = B_MN ? (k0 + i * OB::kRowStep) * ldb * 2
                                    : (i * OB::kRowStep * ldb + k0) * 2;
                sb[S][i] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rb, vb, so, 0));
            }
        } else {
            if (w < kAC)
                sa[S][w] = op_chunk(std::integral_constant<bool, A_MN>{}, A, lda, m0, M,
                                    a_r0 + w * OA::kRowStep, a_c0, k0);
            else
                sb[S][w - kAC] = op_chunk(std::integral_constant<bool, B_MN>{}, B, ldb, n0, N,
                                          b_r0 + (w - kAC) * OB::kRowStep, b_c0, k0);
        }
    };
    // Per-lane LDS bases for the staged writes, one per stage and operand.
    constexpr int kStage = Cfg::kLdsA + Cfg::kLdsB;
    lds_u16 *const L = (lds_u16 *)lds;
    lds_u16 *const a_wr[2] = {lds_base(L + a_r0 * OA::kStride + a_c0),
                              lds_base(L + kStage + a_r0 * OA::kStride + a_c0)};
    lds_u16 *const b_wr[2] = {lds_base(L + Cfg::kLdsA + b_r0 * OB::kStride + b_c0),
                              lds_base(L + kStage + Cfg::kLdsA + b_r0 * OB::kStride + b_c0)};
    // k0: the first k of the staged k-step (LOAD 3 recomputes the chunk's fix-up from it)
    auto store_one = [&](auto set_c, int buf, int w, int k0) {
        constexpr int S = decltype(set_c)::value;
        u16x8 v = w < kAC ? sa[S][w] : sb[S][w - kAC];
        if constexpr (LOAD == 3) {
            const ChunkPos p = pos_of(w, k0);
            const int nv = p.row < p.nrows ? min(max(p.ncols - p.col, 0), 8) : 0;
            v = fix_chunk8(v, p.col - min(p.col, p.ncols - 8), nv);
        } else {
            (void)k0;
        }
        if (w < kAC)
            *(lds_u16x8 *)(a_wr[buf] + w * OA::kRowStep * OA::kStride) = v;
        else
            *(lds_u16x8 *)(b_wr[buf] + (w - kAC) * OB::kRowStep * OB::kStride) = v;
    };

    floatx16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Per-lane fragment offsets within a stage, for the wave's first block (wb = the
    // wave's first row or column).  KM: row wb + l%32, k 8 (l/32) (+ 32 b rows, + 16 s).
    // MN: lane (g = l/16, s16 = l%16) reads row 8 (g/2) + s16/4, column wb + 16 (g%2) +
    // 4 (s16%4) (+ 16 s rows, + 4 h rows, + 32 b columns).
    const int g16 = lane / 16, s16 = lane % 16;
    auto frag_off = [&](auto mn_c, int stride, int wb) {
        constexpr bool kMN = decltype(mn_c)::value;
        if constexpr (kMN)
            return (8 * (g16 / 2) + s16 / 4) * stride + wb + 16 * (g16 % 2) + 4 * (s16 % 4);
        else
            return (wb + l32) * stride + 8 * lhi;
    };
    const int a_off = frag_off(std::integral_constant<bool, A_MN>{}, OA::kStride, wm * Cfg::kTM);
    const int b_off = frag_off(std::integral_constant<bool, B_MN>{}, OB::kStride, wn * Cfg::kTN);
    constexpr int kSteps = kBK / 16;
    constexpr int kRA = MB * OA::kPieces;
    constexpr int kR = kRA + NB * OB::kPieces;  // fragment reads per sub-step
    H16Frag<A_MN, MB> af;
    H16Frag<B_MN, NB> bf;
    lds_u16 *const a_rd[2] = {lds_base(L + a_off), lds_base(L + kStage + a_off)};
    lds_u16 *const b_rd[2] = {lds_base(L + Cfg::kLdsA + b_off),
                              lds_base(L + kStage + Cfg::kLdsA + b_off)};
    // Fragment read `p` of sub-step s into slot: the A pieces first, block-major, then B's.
    auto read_op = [&](auto mn_c, auto &fr, lds_u16 *base, int stride, int s, int slot, int p) {
        constexpr bool kMN = decltype(mn_c)::value;
        if constexpr (kMN) {
            const int b = p / 2, h = p % 2;
            fr.f[slot][b][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_shortx4 *)(base + 16 * s * stride + 32 * b + 4 * h * stride));
        } else {
            fr.f[slot][p] = *(const lds_u16x8 *)(base + 32 * p * stride + 16 * s);
        }
    };
    auto read_piece = [&](int buf, int s, int slot, int p) {
        if (p < kRA)
            read_op(std::integral_constant<bool, A_MN>{}, af, a_rd[buf], OA::kStride, s, slot, p);
        else
            read_op(std::integral_constant<bool, B_MN>{}, bf, b_rd[buf], OB::kStride, s, slot, p - kRA);
    };
    auto mfma_one = [&](int slot, int q) {
        const int i = q / NB, j = q % NB;
        acc[i][j] = mfma32x32x16<T>(af.get(slot, i), bf.get(slot, j), acc[i][j]);
    };
    constexpr int kMf = MB * NB;                  // MFMAs per sub-step
    constexpr int kPre = (kMf * 3 + 7) / 8;       // of those, issued before the barrier
    constexpr int kWr = kAC + kBC;                // staged chunks per k-step
    static_assert(kR <= 2 * kMf, "a sub-step's fragment reads go two per MFMA of the one before");

    // Events of one k-step are spread over its kSteps * kMf MFMA slots: event e of n
    // spread over slots [lo, hi) goes after the MFMA of slot lo + ceil-spread(e).
    constexpr int kSlots = kSteps * kMf;
    auto ev_begin = [](int q, int n, int lo, int hi) {  // first event at or after slot q
        if (q <= lo) return 0;
        if (q >= hi) return n;
        return ((q - lo) * n + (hi - lo) - 1) / (hi - lo);
    };
    // Store window: the idle stage is free from the start of the k-step, so the staged
    // chunks of k-step t+1 are written over every slot before the barrier.  Paired loads
    // of k-step t+2 (into the other, already written-out set) go over the first half.
    constexpr int kBarrier = (kSteps - 1) * kMf + kPre;   // barrier after this many slots
    constexpr int kStoreLo = 0, kStoreHi = kBarrier;
    constexpr int kLoadLo = 0, kLoadHi = kSlots / 2;

    // One k-step t on stage buf.  Every memory instruction is issued between MFMAs so
    // that no burst blocks the in-order issue of the MFMAs behind it:
    //  * sub-step s < last reads the fragments of s+1 (slot (s+1) % 2) two per MFMA
    //    after its first MFMAs;
    //  * the staged chunks of k-step t+1 (set S) are written to the idle stage, spread
    //    over all slots before the barrier; paired variant: the loads of k-step t+2 go
    //    into the other set O over the first half; unpaired variant: chunk w of t+2 is
    //    loaded into S right after chunk w of t+1 was written;
    //  * after the barrier, the first fragments of t+1 are read between the last MFMAs.
    // The body has no branches (a branch makes the compiler wait for every outstanding
    // LDS read at the join): near the end the loads re-read the last k-step and the idle
    // stage takes dummies.
    const int nk = cdiv(K, kBK);
    auto kstep = [&](auto set_c, auto other_c, int kt, int buf) {
        const int kload = min(kt + 2, nk - 1) * kBK;
        const int kstore = min(kt + 1, nk - 1) * kBK;  // the k-step held in set S
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
#pragma unroll
          for (int q = 0; q < kMf; ++q) {
            const int qs = s * kMf + q;
            if (qs >= kBarrier) {
                // after the barrier: next k-step's first fragments before each MFMA
                const int r_lo = ev_begin(qs, kR, kBarrier, kSlots);
                const int r_hi = ev_begin(qs + 1, kR, kBarrier, kSlots);
#pragma unroll
                for (int o = r_lo; o < r_hi; ++o) read_piece(buf ^ 1, 0, 0, o);
            }
            mfma_one(s & 1, q);
            if (s + 1 < kSteps) {
#pragma unroll
                for (int p = 2 * q; p < 2 * q + 2; ++p)
                    if (p < kR) read_piece(buf, s + 1, (s + 1) & 1, p);
            }
            if (qs < kBarrier) {
                const int w_lo = ev_begin(qs, kWr, kStoreLo, kStoreHi);
                const int w_hi = ev_begin(qs + 1, kWr, kStoreLo, kStoreHi);
#pragma unroll
                for (int w = w_lo; w < w_hi; ++w) {
                    store_one(set_c, buf ^ 1, w, kstore);
                    if constexpr (!PAIRED) load_one(set_c, kload, w);
                }
            }
            if constexpr (PAIRED) {
                const int l_lo = ev_begin(qs, kWr, kLoadLo, kLoadHi);
                const int l_hi = ev_begin(qs + 1, kWr, kLoadLo, kLoadHi);
#pragma unroll
                for (int w = l_lo; w < l_hi; ++w) load_one(other_c, kload, w);
            }
            if (qs == kBarrier - 1) __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
          }
        }
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    if (nk > 0) {
#pragma unroll
        for (int w = 0; w < kWr; ++w) load_one(S0{}, 0, w);
#pragma unroll
        for (int w = 0; w < kWr; ++w) store_one(S0{}, 0, w, 0);
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWr; ++w) load_one(S1{}, min(1, nk - 1) * kBK, w);
#pragma unroll
        for (int p = 0; p < kR; ++p) read_piece(0, 0, 0, p);
        if constexpr (PAIRED) {
            // nk is even: k-steps in pairs, staging sets alternating statically
            for (int kt = 0; kt < nk; kt += 2) {
                kstep(S1{}, S0{}, kt, 0);      // loads kt+2 into set 0, stores kt+1 (set 1)
                kstep(S0{}, S1{}, kt + 1, 1);  // loads kt+3 into set 1, stores kt+2 (set 0)
            }
        } else {
            // any nk: one staging set, loads issued one k-step ahead
            for (int kt = 0; kt < nk; ++kt) kstep(S1{}, S1{}, kt, kt & 1);
        }
    }

    // 32x32 accumulator layout: register r of lane l holds row 8(r/4) + 4(l/32) + r%4,
    // column l%32 of the block.  Streaming stores: C is not re-read by this kernel.
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
        {
            const int row0 = m0 + wm * Cfg::kTM + 32 * i + 4 * lhi;
            const int col = n0 + wn * Cfg::kTN + 32 * j + l32;
            if constexpr (EPI == 2) {
                static_assert(NB % 2 == 0, "16-bit C stores block pairs");
                if (j % 2 == 0)
                    store_pair32_c16<EDGE, T, (MB * NB > 8)>(acc[i][j], acc[i][j + 1], (uint16_t *)C, ldc,
                                                             row0, col - l32, M, N, sign, use_old);
            } else if constexpr (EPI == 1) store_block32_acc<EDGE, true, (MB * NB > 8)>(acc[i][j], C, ldc, row0, col, M, N, sign, use_old);
            else store_block32<EDGE, true>(acc[i][j], C, ldc, row0, col, M, N);
        }
}

// Same tile-numbering scheme as the FP32 kernel: interior launches walk the full tiles
// in XCD-contiguous grouped order; edge launches take the ragged right strip, then the
// ragged bottom strip (or every tile when K is ragged).
template <bool EDGE>
__device__ __forceinline__ void h16_tile_of(int bid, int nblocks, int tiles_m, int tiles_n,
                                            bool ragged_n, bool all_tiles, int &tm, int &tn) {
    if (!EDGE || all_tiles) {
        grouped_tile(xcd_contiguous_id(bid, nblocks), tiles_m, tiles_n, 4, tm, tn);
        return;
    }
    const int right = ragged_n ? tiles_m : 0;
    if (bid < right) {
        tm = bid;
        tn = tiles_n - 1;
    } else {
        tm = tiles_m - 1;
        tn = bid - right;
    }
}

template <typename T, int BM, int BN, int WM, int WN, int MINW, int LOAD, bool EDGE, bool PAIRED,
          bool A_MN, bool B_MN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(MINW)))
void mfma_f16_gemm_kernel(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                          const uint16_t *__restrict__ B, int ldb, float *__restrict__ C, int ldc,
                          float sign, int use_old, int all_tiles) {
    using Cfg = H16Cfg<BM, BN, WM, WN, A_MN, B_MN>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (Cfg::kLdsA + Cfg::kLdsB)];
    const int tiles_m = EDGE ? cdiv(M, BM) : M / BM;
    const int tiles_n = EDGE ? cdiv(N, BN) : N / BN;
    int tm, tn;
    h16_tile_of<EDGE>(blockIdx.x, gridDim.x, tiles_m, tiles_n, N % BN != 0, all_tiles != 0, tm, tn);
    h16_tile<T, BM, BN, WM, WN, LOAD, EDGE, PAIRED, A_MN, B_MN, EPI>(
        M, N, K, A, lda, B, ldb, C, ldc, sign, use_old, tm * BM, tn * BN, lds);
}

// Every row of both operands starts on a 16-byte boundary.
inline bool h16_vec(const GemmArgs &g) {
    return rows_aligned16(g.A, g.lda, 2) && rows_aligned16(g.B, g.ldb, 2);
}

#include "h16_dma.hpp"

// Byte offsets below 2^31 for every chunk of a 256-extent tile of the operand.
inline bool op_fits(bool mn, int ext, int K, int ld) {
    return mn ? ((long)K * ld + ext) * 2 < (1L << 31) : ((long)ext * ld + K) * 2 < (1L << 31);
}

// Ring stages of the direct-load kernel for this call: 256-wide tiles 4; 128-wide tiles 8
// (128 KiB, one per CU) when the grid fits one round of 256, else 4 (64 KiB, two per CU:
// grids of more than 256 tiles then run at most ceil(tiles / 512) rounds, where one
// workgroup per CU would take ceil(tiles / 256); with one tile per CU the deeper ring is
// the faster one, 2048^3 FP16 19.5 against 24.7 us).  64-wide tiles 8 (64 KiB).  A K below
// an 8-stage trip (128 <= K < 256) takes the 4-stage ring, one trip of 128, on 128- and
// 64-wide tiles alike.
inline int dma_stages(const GemmArgs &g, int tile) {
    if (tile == 128 && (long)cdiv(g.M, 128) * cdiv(g.N, 128) > 256) return 4;
    if (tile != 256 && g.K < dma::kBK * 8) return 4;
    return dma::ring_stages(tile);
}

// The direct-load kernel takes every tile (ragged ones included) of a 256 x 256, 128 x 128
// or 64 x 64 configuration when rows are 16-byte aligned, K is a multiple of 8 and at least
// one trip round the ring (32 x the ring stages: 128 or 256; a K that is not a whole
// number of trips runs to the next trip with the chunks past K loaded as zeros), and every
// byte offset up to that trip fits the 31-bit buffer range.  At 128 x 128 the tile's loads
// (16 KiB per k-step per tile against 256 cycles of MFMAs) run at the CU's load-path rate,
// so the kernel is load-bound there; it still beats the register-staged kernel: by 10-20 %
// at 2048^2 (one tile per CU), by 5-17 % from 2304^2 to 2816^2 (two per CU).
inline bool use_dma(const GemmArgs &g, int tile) {
    const int trip = dma::kBK * dma_stages(g, tile);
    if (tile == 128 && g.one_round_128 && (long)cdiv(g.M, 128) * cdiv(g.N, 128) > 256) return false;
    // an m/n-contiguous operand's extent is a whole number of 16-byte chunks, so no
    // load straddles the end of its last row
    if ((g.trans_a && g.M % 8 != 0) || (!g.trans_b && g.N % 8 != 0)) return false;
    // K from 128 to 255 on a tile that takes the 8-stage ring otherwise (64 wide, or 128 wide
    // one per CU) runs on the 4-stage ring, except for plain products with K a whole number of
    // 64-wide k-steps, whose register-staged interior tiles (two staging sets, no predicates)
    // were as fast or faster: BF16 2048^2 x 128 6.25 against 7.19 us, FP16 1536^2 x 192 6.57
    // against 6.81; elsewhere the ring won (1024^2 x 200 with A transposed 4.96 against 8.21,
    // 2048^2 x 136 8.16 against 10.81, 2048^2 x 192 accumulating 8.32 against 9.29)
    const bool two_per_cu = tile == 128 && (long)cdiv(g.M, 128) * cdiv(g.N, 128) > 256;
    if (tile != 256 && !two_per_cu && g.K < dma::kBK * 8 && g.K % 64 == 0 && !g.trans_a &&
        !g.signed_or_acc() && !g.c16)
        return false;
    // staged_small (a measurement variant): neither the 64 x 64 tile nor the 4-stage ring on
    // tiles that otherwise take the 8-stage one
    if (g.staged_small && (tile == 64 || (tile == 128 && !two_per_cu && g.K < dma::kBK * 8))) return false;
    const int kpad = cdiv(g.K, trip) * trip;
    return (tile == 256 || tile == 128 || tile == 64) && h16_vec(g) && g.K >= trip && g.K % 8 == 0 &&
           g.M >= tile && g.N >= tile && op_fits(g.trans_a != 0, tile, kpad, g.lda) &&
           op_fits(g.trans_b == 0, tile, kpad, g.ldb);
}

// The EM x EN direct-load tile with one extent of 192 (192 x 256 or 256 x 192, any layout
// and epilogue) on the same terms as the 256 x 256 one: rows 16-byte aligned, K a multiple
// of 8 and at least one ring trip, every byte offset within 31 bits, and an m/n-contiguous
// operand's extent a multiple of 8.
inline bool use_dma_rect(const GemmArgs &g, int em, int en) {
    if ((g.trans_a && g.M % 8 != 0) || (!g.trans_b && g.N % 8 != 0)) return false;
    const int trip = dma::kBK * dma::ring_stages(256);
    const int kpad = cdiv(g.K, trip) * trip;
    return h16_vec(g) && g.K >= trip && g.K % 8 == 0 && g.M >= em && g.N >= en &&
           op_fits(g.trans_a != 0, em, kpad, g.lda) && op_fits(g.trans_b == 0, en, kpad, g.ldb);
}

// Which tile a product headed for 256 x 256 tiles takes: 256 (the square tile), 192 (192 x
// 256) or -192 (256 x 192), by rounds of resident tiles (one per CU) times tile area, a
// tile with a 192 extent at 0.87 of the square one's rate per unit of area (FP16 3072^3:
// 50.8 against 57.0 us, 192 against 144 tiles; 6144 x 6144 x 4096: 229.6 against 263.0 us,
// 768 against 576), or 0.85 when its 192 side is an m/n-contiguous operand, so that between
// otherwise equal grids the tile whose 192 side is k-contiguous wins (A and B both
// transposed, K-contiguous 192 side against m/n-contiguous: FP16 3072^2 x 4096 65.1 against
// 67.3 us, BF16 61.7 against 65.3, BF16 3000^2 x 1000 accumulating 31.5 against 35.5).
// Ties keep the square tile, then 192 x 256.
inline int rect_choice(const GemmArgs &g) {
    if (g.square_tiles) return 256;
    const auto cost = [&](int em, int en) {
        const long t = (long)cdiv(g.M, em) * cdiv(g.N, en);
        const bool mn192 = em == 192 ? g.trans_a != 0 : g.trans_b == 0;  // 192 side m/n-contiguous
        return (double)((t + 255) / 256) * em * en / (em == en ? 1.0 : mn192 ? 0.85 : 0.87);
    };
    int best = 256;
    double c = cost(256, 256);
    if (use_dma_rect(g, 192, 256) && cost(192, 256) < c) {
        best = 192;
        c = cost(192, 256);
    }
    if (use_dma_rect(g, 256, 192) && cost(256, 192) < c) best = -192;
    return best;
}

// K is not a whole number of the direct-load kernel's ring trips.
inline bool dma_ragged_k(const GemmArgs &g, int tile) {
    return g.K % (dma::kBK * dma_stages(g, tile)) != 0;
}

// The epilogue's flags argument: bit 0 adds the old C; with 16-bit C, bit 1 selects
// 4-byte accesses that write whole lines (possible when ldc is even and C 4-byte
// aligned).
template <int EPI>
inline int epi_flags(const GemmArgs &g) {
    int f = g.accumulate ? 1 : 0;
    if (EPI == 2 && g.ldc % 2 == 0 && (uintptr_t)g.C % 4 == 0) f |= 2;
    return f;
}

template <typename T, int BM, int BN, int WM, int WN, int MINW, int LOAD, bool EDGE, bool PAIRED,
          bool A_MN, bool B_MN, int EPI>
hipError_t launch_one(const GemmArgs &g, int tiles, int all_flag, hipStream_t s) {
    hipLaunchKernelGGL((mfma_f16_gemm_kernel<T, BM, BN, WM, WN, MINW, LOAD, EDGE, PAIRED, A_MN, B_MN, EPI>),
                       dim3(tiles), dim3(64 * WM * WN), 0, s, g.M, g.N, g.K,
                       (const uint16_t *)g.A, g.lda, (const uint16_t *)g.B, g.ldb, g.C, g.ldc,
                       g.sign, epi_flags<EPI>(g), all_flag);
    return hipGetLastError();
}

// The launches one configuration makes.  Interior tiles: direct-to-LDS loads (256 x 256,
// K % 128 == 0), else buffer loads when rows are 16-byte aligned and every offset fits in
// 31 bits, with the two-set pipeline when the number of k-steps is even; ragged strips:
// clamped loads fixed up when staged (predicated element loads when a contiguous extent is
// below 8).  The signed / accumulating epilogues (EPI 1, 2) keep to the direct-to-LDS and
// pointer-load kernels, which bounds the number of instances.
struct H16Plan {
    bool dma = false;         // the direct-to-LDS kernel takes every tile
    bool all_tiles = false;   // one clamped launch over every tile (edge_paired applies)
    int interior = -1;        // interior launch: load mode 2 buffer, 1 pointer, 0 pointer at
                              // element alignment; -1 none
    bool interior_paired = false;
    int edge = -1;            // ragged strips (or every tile when K is ragged): 3 clamped,
                              // 1 / 0 predicated (aligned / unaligned rows); -1 none
    bool edge_paired = false;
};

inline H16Plan plan_cfg(int BM, int BN, bool a_mn, bool b_mn, int epi, const GemmArgs &g) {
    H16Plan p;
    if (BM == BN && use_dma(g, BM)) {
        p.dma = true;
        return p;
    }
    const bool vec = h16_vec(g);
    const bool kfull = g.K % kBK == 0;
    const int full_tiles = kfull ? (g.M / BM) * (g.N / BN) : 0;
    const int edge_tiles = cdiv(g.M, BM) * cdiv(g.N, BN) - full_tiles;
    const bool fits = op_fits(a_mn, BM, g.K, g.lda) && op_fits(b_mn, BN, g.K, g.ldb);
    // Clamped loads need 8 elements along each operand's contiguous extent.  With them
    // the ragged-tile kernel can take every tile in one launch; its tiles run about 1.5x
    // as long as interior ones (one staging set, fix-ups), so it does when that takes
    // less time than the interior launch followed by the ragged strips' launch.  (EPI 0
    // with an even number of k-steps: the two-set pipeline.)
    const bool clamp = (a_mn ? g.M : g.K) >= 8 && (b_mn ? g.N : g.K) >= 8;
    const bool clamp_paired = epi == 0 && cdiv(g.K, kBK) % 2 == 0;
    if (clamp && full_tiles > 0 && edge_tiles > 0) {
        const int all = full_tiles + edge_tiles;
        if (cdiv(all, 256) * 3 < cdiv(full_tiles, 256) * 2 + cdiv(edge_tiles, 256) * 3) {
            p.all_tiles = true;
            p.edge = 3;
            p.edge_paired = clamp_paired;
            return p;
        }
    }
    if (full_tiles > 0) {
        if (epi == 0 && vec && fits) {
            p.interior = 2;
            p.interior_paired = (g.K / kBK) % 2 == 0;
        } else {
            p.interior = vec ? 1 : 0;
        }
    }
    if (edge_tiles > 0) {
        // Whole tiles with only K ragged (by a multiple of 8) and aligned rows never take
        // the predicated loads' element paths, which then run faster than the fix-ups
        // (4096 x 4096 x 4000 BF16: 142 against 174 us); any row or column past the
        // matrix makes them the slower ones (4000^3: 298 against 178 us).
        const bool whole = vec && g.M % BM == 0 && g.N % BN == 0 && g.K % 8 == 0;
        if (clamp && !whole) {
            p.edge = 3;
            p.edge_paired = clamp_paired;
        } else {
            p.edge = vec ? 1 : 0;
        }
    }
    return p;
}

template <typename T, bool A_MN, bool B_MN, int EPI, int E, int NS>
hipError_t launch_dma(const GemmArgs &g, hipStream_t s) {
    const dim3 grid(cdiv(g.M, E) * cdiv(g.N, E));
    if (dma_ragged_k(g, E))
        hipLaunchKernelGGL((mfma_f16_dma_kernel<T, A_MN, B_MN, EPI, E, true, NS>), grid, dim3(256), 0, s, g.M,
                           g.N, g.K, (const uint16_t *)g.A, g.lda, (const uint16_t *)g.B, g.ldb, g.C, g.ldc,
                           g.sign, epi_flags<EPI>(g));
    else
        hipLaunchKernelGGL((mfma_f16_dma_kernel<T, A_MN, B_MN, EPI, E, false, NS>), grid, dim3(256), 0, s, g.M,
                           g.N, g.K, (const uint16_t *)g.A, g.lda, (const uint16_t *)g.B, g.ldb, g.C, g.ldc,
                           g.sign, epi_flags<EPI>(g));
    return hipGetLastError();
}

template <typename T, int BM, int BN, int WM, int WN, int MINW, bool A_MN, bool B_MN, int EPI>
hipError_t launch_cfg(const GemmArgs &g, hipStream_t s) {
    const H16Plan p = plan_cfg(BM, BN, A_MN, B_MN, EPI, g);
    if constexpr (BM == BN && BM >= 64) {
        if (p.dma) {
            if constexpr (BM == 128 || BM == 64)
                if (dma_stages(g, BM) == 4) return launch_dma<T, A_MN, B_MN, EPI, BM, 4>(g, s);
            return launch_dma<T, A_MN, B_MN, EPI, BM, dma::ring_stages(BM)>(g, s);
        }
    }
    if (p.dma) return hipErrorInvalidValue;
    const bool kfull = g.K % kBK == 0;
    const int full_tiles = kfull ? (g.M / BM) * (g.N / BN) : 0;
    const int edge_tiles = cdiv(g.M, BM) * cdiv(g.N, BN) - full_tiles;
    const int all_flag = kfull ? 0 : 1;
    auto launch_clamped = [&](int tiles, int flag) {
        if constexpr (EPI == 0) {
            if (p.edge_paired)
                return launch_one<T, BM, BN, WM, WN, MINW, 3, true, true, A_MN, B_MN, EPI>(g, tiles, flag, s);
        }
        return launch_one<T, BM, BN, WM, WN, MINW, 3, true, false, A_MN, B_MN, EPI>(g, tiles, flag, s);
    };
    if (p.all_tiles) return launch_clamped(full_tiles + edge_tiles, 1);
    if (p.interior >= 0) {
        hipError_t e = hipSuccess;
        if (p.interior == 2) {
            if constexpr (EPI == 0) {
                if (p.interior_paired)
                    e = launch_one<T, BM, BN, WM, WN, MINW, 2, false, true, A_MN, B_MN, EPI>(g, full_tiles, all_flag, s);
                else
                    e = launch_one<T, BM, BN, WM, WN, MINW, 2, false, false, A_MN, B_MN, EPI>(g, full_tiles, all_flag, s);
            }
        } else if (p.interior == 1) {
            e = launch_one<T, BM, BN, WM, WN, MINW, 1, false, false, A_MN, B_MN, EPI>(g, full_tiles, all_flag, s);
        } else {
            e = launch_one<T, BM, BN, WM, WN, MINW, 0, false, false, A_MN, B_MN, EPI>(g, full_tiles, all_flag, s);
        }
        if (e != hipSuccess) return e;
    }
    if (p.edge == 3) return launch_clamped(edge_tiles, all_flag);
    if (p.edge == 1) return launch_one<T, BM, BN, WM, WN, MINW, 1, true, false, A_MN, B_MN, EPI>(g, edge_tiles, all_flag, s);
    if (p.edge == 0) return launch_one<T, BM, BN, WM, WN, MINW, 0, true, false, A_MN, B_MN, EPI>(g, edge_tiles, all_flag, s);
    return hipSuccess;
}

// Cost model as for FP32: with w resident workgroups per CU a config needs
// ceil(tiles / (256 w)) rounds of w * BM * BN work each, divided by the tile's measured
// efficiency: per unit of work the 256 x 256 direct-to-LDS tile runs about 1.8x faster
// than two 128 x 128 tiles per CU (4096^3 FP16: 256^2 x 4096 per CU in 100 us;
// 4096 x 4104 on 128-wide tiles: two 128^2 x 4096 per CU in 96 us per round), so 128-wide
// tiles count 1/0.55 of their area.  Ties go to the larger tile.
inline int pick_tile(const GemmArgs &g) {
    struct Opt { int tile, per_cu; double eff; };
    const Opt opts[] = {{256, 1, 1.0}, {128, 2, 0.55}};
    double best = -1;
    int tile = 128;
    for (const Opt &o : opts) {
        const long tiles = (long)cdiv(g.M, o.tile) * cdiv(g.N, o.tile);
        const long slots = 256L * o.per_cu;
        const double cost = (double)((tiles + slots - 1) / slots * o.per_cu * (long)o.tile * o.tile) / o.eff;
        if (best < 0 || cost < best) {
            best = cost;
            tile = o.tile;
        }
    }
    return tile;
}

// Plain products with A k-contiguous whose 128 x 128 tiling leaves CUs idle (fewer tiles
// than CUs) take 128 x 64 tiles (twice as many); measured faster at n = 512 and 1024.
// (With A m-contiguous the 64 x 32 wave tile would read more fragments per sub-step
// than its MFMAs carry.)
inline bool use_128x64(const GemmArgs &g) {
    return (long)cdiv(g.M, 128) * cdiv(g.N, 128) < 256;
}

// When even the 128 x 64 tiling leaves CUs idle, 64 x 64 tiles on two waves (64 x 32 of C
// each): half the operand bytes per CU, and at these sizes the CU's load path, not its
// matrix cores, sets the time (BF16 1024^3: 7.2 against 7.9 us; 512^3: 4.8 against 5.3).
// The register-staged kernel's tile, for the calls the direct-to-LDS 64 x 64 tile does not
// take (rows not 16-byte aligned, K not a multiple of 8 or below 256).
inline bool use_64x64(const GemmArgs &g) {
    return (long)cdiv(g.M, 128) * cdiv(g.N, 64) < 256;
}

// The 64 x 64 direct-to-LDS tile (8-stage ring, 64 KiB of LDS, up to two per CU), any layout
// and epilogue, where the 128 x 128 tiling leaves CUs idle and the 64 x 64 grid fits one
// round of two per CU (at most 512 tiles).  Against the 128 x 128 direct-to-LDS tile (FP16 /
// BF16, µs, transposed, accumulating, negated or 16-bit-C products): 1024^3 5.8-6.0 against
// 9.2-10.4 (64 CUs busy), 1152^3 9.7 against 12.4, 1280^3 11.1 against 13.2, 1408^3 12.1
// against 14.6 (484 tiles); from 576 tiles the larger tile wins (1536^3 16.9-18.4 against
// 14.2-14.6, 1600^3 18.1 against 16.5, 1536^2 x 4096 38.5 against 27.8).
inline bool use_dma64(const GemmArgs &g) {
    return (long)cdiv(g.M, 128) * cdiv(g.N, 128) < 256 && (long)cdiv(g.M, 64) * cdiv(g.N, 64) <= 512 &&
           use_dma(g, 64);
}

// Plain products with A k-contiguous take the register-staged 128 x 64 and 64 x 64 tiles
// only where the 128 x 128 direct-to-LDS tile cannot run (rows not 16-byte aligned, K not a
// multiple of 8 or below 256): that tile, on the CUs it leaves idle, is faster than either
// once the 64 x 64 one no longer fits one round.
inline bool staged_small_tiles(const GemmArgs &g) { return g.staged_small || !use_dma(g, 128); }

template <typename T, bool A_MN, bool B_MN, int EPI, int EM, int EN>
hipError_t launch_rect(const GemmArgs &g, hipStream_t s) {
    const dim3 grid(cdiv(g.M, EM) * cdiv(g.N, EN));
    if (dma_ragged_k(g, 256))
        hipLaunchKernelGGL((mfma_f16_dma_rect_kernel<T, A_MN, B_MN, EPI, EM, EN, true>), grid, dim3(256), 0, s,
                           g.M, g.N, g.K, (const uint16_t *)g.A, g.lda, (const uint16_t *)g.B, g.ldb, g.C,
                           g.ldc, g.sign, epi_flags<EPI>(g));
    else
        hipLaunchKernelGGL((mfma_f16_dma_rect_kernel<T, A_MN, B_MN, EPI, EM, EN>), grid, dim3(256), 0, s, g.M,
                           g.N, g.K, (const uint16_t *)g.A, g.lda, (const uint16_t *)g.B, g.ldb, g.C, g.ldc,
                           g.sign, epi_flags<EPI>(g));
    return hipGetLastError();
}

template <typename T, bool A_MN, bool B_MN, int EPI>
hipError_t launch_layout(const GemmArgs &g, hipStream_t s) {
    if (pick_tile(g) == 256) {
        const int rect = rect_choice(g);
        if (rect == 192) return launch_rect<T, A_MN, B_MN, EPI, 192, 256>(g, s);
        if (rect == -192) return launch_rect<T, A_MN, B_MN, EPI, 256, 192>(g, s);
        return launch_cfg<T, 256, 256, 2, 2, 1, A_MN, B_MN, EPI>(g, s);
    }
    if (use_dma64(g)) {
        if (dma_stages(g, 64) == 4) return launch_dma<T, A_MN, B_MN, EPI, 64, 4>(g, s);
        return launch_dma<T, A_MN, B_MN, EPI, 64, dma::ring_stages(64)>(g, s);
    }
    if constexpr (!A_MN && EPI == 0) {
        if (staged_small_tiles(g)) {
            if (use_64x64(g)) return launch_cfg<T, 64, 64, 1, 2, 4, A_MN, B_MN, EPI>(g, s);
            if (use_128x64(g)) return launch_cfg<T, 128, 64, 2, 2, 2, A_MN, B_MN, EPI>(g, s);
        }
    }
    return launch_cfg<T, 128, 128, 2, 2, 2, A_MN, B_MN, EPI>(g, s);
}

}  // namespace

}  // namespace g355
