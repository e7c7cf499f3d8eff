// FP32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32), FP32 products and
// FP32 accumulation.
//
// Structure (the reuse hierarchy of "Advanced CUDA features - starting from GEMM":
// shared-memory tiling for block-level reuse, register tiling for thread-level reuse,
// and batched, overlapped global loads from its scheduling section; the double buffer
// of "Kernel optimisation guide", Level 3):
//  * a workgroup of WM x WN waves owns a BM x BN tile of C and walks K in steps of
//    BK = 32, with two LDS stages: while the matrix cores consume stage t, the dwordx4
//    loads of step t+1 are in flight into registers and are written to the other stage
//    before the single barrier of the step;
//  * each wave owns a (BM/WM) x (BN/WN) sub-tile held as 32 x 32 MFMA accumulator
//    blocks (the register tile); one A fragment feeds BN/WN/32 MFMAs and one B fragment
//    BM/WM/32 MFMAs;
//  * LDS layouts: A is kept [m][k] with a row stride of BK+4 words, so the ds_read_b128
//    of lanes on consecutive rows land on distinct bank groups; B is kept [k][n] with a
//    row stride of BN+8 words, so the two k rows one ds_read_b32 touches fall in
//    opposite halves of the banks;
//  * fragment k order: lane l reads A[m][k0+4(l/32) .. +3] with one ds_read_b128 and
//    feeds element s to MFMA step s, paired with B[k0+4(l/32)+s][n]; each MFMA then
//    sums k0+s and k0+4+s, and steps s = 0..3 cover k0..k0+7;
//  * edges: when rows are 16-byte aligned, m/n-contiguous extents are multiples of 4
//    and K of BK, the unpredicated kernel takes every tile, its chunk coordinates
//    clamped to the matrix and its stores guarded where a tile crosses M or N; with K a
//    multiple of 4 but not of BK an instance (KT) also zero-fills the last k-step;
//    otherwise tiles that cross M, N or the K tail load with per-element predicates and
//    zero fill, store with a guard, and run as a second launch;
//  * launch order: tiles are renumbered so each XCD receives a contiguous range, walked
//    in groups of 4 tile-rows, which keeps shared A and B panels in that XCD's L2;
//  * operand layouts (the transposed and negated operands and the D-scaled-by-0-or-1 of
//    the tensor-core instruction table of "Advanced CUDA features - starting from
//    GEMM"): an operand stored with k contiguous (kind KM: A, or a transposed B) takes
//    the A path above, one stored with m or n contiguous (kind MN: B, or a transposed
//    A) the B path; the plain kernels store the accumulators as they are, the signed /
//    accumulating variants (ACC) store sign * acc, plus the old C when accumulating.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace g355 {

namespace {

constexpr int kBK = 32;
constexpr int kSA = kBK + 4;  // A LDS row stride (words)

// One operand as the kernel holds it.  KM: E rows (m or n) of kBK words, row stride
// kSA; MN: kBK rows (k) of E words, row stride E + 8.
template <bool MN, int E, int TT>
struct F32Op {
    static constexpr int kStride = MN ? E + 8 : kSA;
    static constexpr int kRows = MN ? kBK : E;
    static constexpr int kLds = kRows * kStride;             // words per stage
    static constexpr int kPerRow = (MN ? E : kBK) / 4;       // 16-byte chunks per row
    static constexpr int kChunks = kRows * kPerRow / TT;     // per thread
    static constexpr int kPieces = MN ? 4 : 1;               // LDS reads per block per group
    static_assert((kRows * kPerRow) % TT == 0, "tile chunks must divide over the threads");
};

template <int BM, int BN, int WM, int WN, bool A_MN, bool B_MN>
struct F32Cfg {
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kTM = BM / WM, kTN = BN / WN;
    static constexpr int kMB = kTM / 32, kNB = kTN / 32;
    using OA = F32Op<A_MN, BM, kThreads>;
    using OB = F32Op<B_MN, BN, kThreads>;
    static constexpr int kAChunks = OA::kChunks, kBChunks = OB::kChunks;
    static constexpr int kLdsA = OA::kLds, kLdsB = OB::kLds;
    static constexpr int kLdsBytes = 2 * (kLdsA + kLdsB) * 4;
    static_assert(kTM % 32 == 0 && kTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// Fragment registers of one operand for one 8-wide k group: a KM fragment is one
// ds_read_b128 (k0 + 4(l/32) .. +3), an MN fragment four ds_read_b32 (one per step).
template <bool MN, int NBLK>
struct F32Frag {
    floatx4 f[2][NBLK];
    __device__ __forceinline__ float get(int slot, int b, int s) const { return f[slot][b][s]; }
};
template <int NBLK>
struct F32Frag<true, NBLK> {
    float f[2][NBLK][4];
    __device__ __forceinline__ float get(int slot, int b, int s) const { return f[slot][b][s]; }
};

// Columns [c, c+4) of one row.  EDGE: zero outside [0, ncols) and for invalid rows;
// otherwise the caller guarantees the chunk is inside the matrix.
template <bool VEC, bool EDGE>
__device__ __forceinline__ floatx4 ld_chunk(const float *__restrict__ row, int c, int ncols,
                                            bool row_ok) {
    if (!EDGE) {
        if (VEC) return *reinterpret_cast<const floatx4 *>(row + c);
        return floatx4{row[c], row[c + 1], row[c + 2], row[c + 3]};
    }
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (!row_ok) return v;
    if (VEC && c + 4 <= ncols) return *reinterpret_cast<const floatx4 *>(row + c);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (c + e < ncols) v[e] = row[c + e];
    return v;
}

// One BM x BN tile of C.  LOAD: 0 = dword loads (rows not 16-byte aligned), 1 = dwordx4
// through pointers, 2 = dwordx4 through buffer resources (interior tiles, offsets below
// 2^31 bytes).  EDGE selects the predicated loads and guarded stores.  (Clamped loads
// fixed up when staged, as in the 16-bit kernel, and 16-byte loads at 4-byte alignment
// both measured slower here than these loads.)
// KT (unpredicated, LOAD 2 or 0): K is not a multiple of BK but of 4; the last k-step's
// chunks past K load from inside the matrix (a row clamped to K-1, or 4 columns clamped
// to K-4) and are zeroed when staged to LDS.  With LOAD 0 (rows not 16-byte aligned) each
// chunk is four dword buffer loads at the same offsets.
template <int BM, int BN, int WM, int WN, int LOAD, bool EDGE, bool PAIRED, bool A_MN, bool B_MN,
          bool ACC, bool KT = false>
__device__ __forceinline__ void f32_tile(int M, int N, int K, const float *__restrict__ A, int lda,
                                         const float *__restrict__ B, int ldb,
                                         float *__restrict__ C, int ldc, float sign,
                                         int use_old, int m0, int n0, float *lds) {
    using Cfg = F32Cfg<BM, BN, WM, WN, A_MN, B_MN>;
    using OA = typename Cfg::OA;
    using OB = typename Cfg::OB;
    constexpr int T = Cfg::kThreads;
    constexpr int MB = Cfg::kMB, NB = Cfg::kNB;
    constexpr int kAC = Cfg::kAChunks, kBC = Cfg::kBChunks, kWr = kAC + kBC;

    const int t = threadIdx.x;
    const int lane = t % 64, wave = t / 64;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane % 32, lhi = lane / 32;

    // Per-thread chunk coordinates (fixed across k-steps): chunk q = t + T i of an
    // operand's LDS image, row q / kPerRow, column 4 (q % kPerRow).  KM: rows are m (or
    // n), columns k; MN: rows are k, columns m (or n).
    int a_r[kAC], a_c[kAC], b_r[kBC], b_c[kBC];
#pragma unroll
    for (int i = 0; i < kAC; ++i) {
        const int q = t + T * i;
        a_r[i] = q / OA::kPerRow;
        a_c[i] = (q % OA::kPerRow) * 4;
    }
#pragma unroll
    for (int i = 0; i < kBC; ++i) {
        const int q = t + T * i;
        b_r[i] = q / OB::kPerRow;
        b_c[i] = (q % OB::kPerRow) * 4;
    }
    // An unpredicated tile that reaches past row M or column N (launched when the host
    // lets this kernel take every tile: K % kBK == 0, an m/n-contiguous extent a multiple
    // of 4): a chunk whose row (KM) or 4 columns (MN) lie past the matrix loads the last
    // one inside instead, so every load stays within the operand; its products only
    // reach outputs past row M or column N, whose stores are guarded below.
    if constexpr (!EDGE) {
#pragma unroll
        for (int i = 0; i < kAC; ++i) {
            if (A_MN) a_c[i] = min(a_c[i], M - m0 - 4);
            else a_r[i] = min(a_r[i], M - m0 - 1);
        }
#pragma unroll
        for (int i = 0; i < kBC; ++i) {
            if (B_MN) b_c[i] = min(b_c[i], N - n0 - 4);
            else b_r[i] = min(b_r[i], N - n0 - 1);
        }
    }
    // Buffer resources based at the tile's first row (KM) or first column (MN).
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A_MN ? A + m0 : A + (size_t)m0 * lda), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(B_MN ? B + n0 : B + (size_t)n0 * ldb), (short)0, 0x7fffffff, 0x00020000);
    // Chunk (r, c) of the k-step at k0 through pointers: KM: row mn0 + r, column k0 + c;
    // MN: row k0 + r, column mn0 + c.
    auto op_chunk = [&](auto mn_c, const float *__restrict__ X, int ld, int mn0, int MNext,
                        int r, int c, int k0) -> floatx4 {
        constexpr bool kMN = decltype(mn_c)::value;
        const int row = kMN ? k0 + r : mn0 + r;
        const int col = kMN ? mn0 + c : k0 + c;
        const bool ok = !EDGE || row < (kMN ? K : MNext);
        return ld_chunk<LOAD == 1, EDGE>(X + (size_t)(ok ? row : 0) * ld, col, kMN ? MNext : K, ok);
    };

    floatx4 st[kWr];  // staged chunks of the next k-step (A chunks first)
    static_assert(!KT || (LOAD != 1 && !EDGE), "the K tail rides on the unpredicated buffer loads");
    auto load_one = [&](int k0, int w) {
        if constexpr (KT) {
            // one chunk at byte offset off of a buffer: one dwordx4 (LOAD 2) or four dwords
            const auto buf_chunk = [](__amdgpu_buffer_rsrc_t r, int off) {
                if constexpr (LOAD == 2)
                    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
                floatx4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * e, 0, 0));
                return v;
            };
            // the offset carries the k position, clamped into the matrix
            if (w < kAC) {
                const int r = A_MN ? min(k0 + a_r[w], K - 1) : a_r[w];
                const int c = A_MN ? a_c[w] : min(k0 + a_c[w], K - 4);
                st[w] = buf_chunk(ra, (r * lda + c) * 4);
            } else {
                const int v = w - kAC;
                const int r = B_MN ? min(k0 + b_r[v], K - 1) : b_r[v];
                const int c = B_MN ? b_c[v] : min(k0 + b_c[v], K - 4);
                st[w] = buf_chunk(rb, (r * ldb + c) * 4);
            }
        } else if constexpr (LOAD == 2) {
            if (w < kAC)
                st[w] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        ra, (a_r[w] * lda + a_c[w]) * 4,
                                                        A_MN ? k0 * lda * 4 : k0 * 4, 0));
            else
                st[w] = __builtin_bit_cast(
                    floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                 rb, (b_r[w - kAC] * ldb + b_c[w - kAC]) * 4,
                                 B_MN ? k0 * ldb * 4 : k0 * 4, 0));
        } else {
            if (w < kAC)
                st[w] = op_chunk(std::integral_constant<bool, A_MN>{}, A, lda, m0, M, a_r[w], a_c[w], k0);
            else
                st[w] = op_chunk(std::integral_constant<bool, B_MN>{}, B, ldb, n0, N, b_r[w - kAC],
                                 b_c[w - kAC], k0);
        }
    };
    // k0: the first k of the staged k-step (for KT: chunks at or past K are stored as 0)
    auto store_one = [&](int buf, int w, int k0) {
        float *As = lds + buf * (Cfg::kLdsA + Cfg::kLdsB);
        float *Bs = As + Cfg::kLdsA;
        floatx4 v = st[w];
        if constexpr (KT) {
            const int kk = w < kAC ? k0 + (A_MN ? a_r[w] : a_c[w])
                                   : k0 + (B_MN ? b_r[w - kAC] : b_c[w - kAC]);
            if (kk >= K) v = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        if (w < kAC)
            *reinterpret_cast<floatx4 *>(As + a_r[w] * OA::kStride + a_c[w]) = v;
        else
            *reinterpret_cast<floatx4 *>(Bs + b_r[w - kAC] * OB::kStride + b_c[w - kAC]) = v;
    };

    floatx16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Fragments of one 8-wide k group: lane l needs, for block row or column
    // wb + 32 b + l%32, k0+4(l/32)+s for steps s = 0..3 (MFMA step s then sums k0+s and
    // k0+4+s).  KM: one ds_read_b128 of the row; MN: one ds_read_b32 per step.  Pieces
    // are the A reads then the B reads; an MN operand's are step-major.
    const int a_rc0 = wm * Cfg::kTM + l32;  // + 32 i
    const int b_rc0 = wn * Cfg::kTN + l32;  // + 32 j
    constexpr int kGroups = kBK / 8;
    constexpr int kRA = MB * OA::kPieces;
    constexpr int kR = kRA + NB * OB::kPieces;  // fragment reads per group
    constexpr int kMf = 4 * MB * NB;            // MFMAs per group
    static_assert(kR <= 2 * kMf, "a group's fragment reads go two per MFMA of the one before");
    F32Frag<A_MN, MB> af;
    F32Frag<B_MN, NB> bf;
    auto read_op = [&](auto mn_c, auto &fr, const float *X, int stride, int rc0, int nblk, int kq,
                       int slot, int p) {
        constexpr bool kMN = decltype(mn_c)::value;
        if constexpr (kMN) {
            const int s = p / nblk, b = p % nblk;
            fr.f[slot][b][s] = X[(kq + s) * stride + rc0 + 32 * b];
        } else {
            fr.f[slot][p] = *reinterpret_cast<const floatx4 *>(X + (rc0 + 32 * p) * stride + kq);
        }
    };
    auto read_piece = [&](int buf, int g, int slot, int p) {
        const float *As = lds + buf * (Cfg::kLdsA + Cfg::kLdsB);
        const float *Bs = As + Cfg::kLdsA;
        const int kq = g * 8 + 4 * lhi;
        if (p < kRA)
            read_op(std::integral_constant<bool, A_MN>{}, af, As, OA::kStride, a_rc0, MB, kq, slot, p);
        else
            read_op(std::integral_constant<bool, B_MN>{}, bf, Bs, OB::kStride, b_rc0, NB, kq, slot, p - kRA);
    };
    auto mfma_one = [&](int slot, int q) {  // step-major: q = (s, i, j)
        const int s = q / (MB * NB), i = (q / NB) % MB, j = q % NB;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af.get(slot, i, s), bf.get(slot, j, s),
                                                         acc[i][j], 0, 0, 0);
    };
    constexpr int kPre = (kMf * 2) / 3;  // MFMAs of the last group issued before the barrier

    // Software pipeline (the same shape as the 16-bit kernel): group g reads the
    // fragments of g+1 between its first MFMAs; the last group writes the staged k-step
    // t+1 to the idle stage between its first kPre MFMAs, then the barrier, then the
    // global loads of t+2 and the first fragments of t+1 go between its remaining MFMAs.
    // No branches in the body; near the end the loads re-read the last k-step.
    const int nk = cdiv(K, kBK);
    if (nk > 0) {
#pragma unroll
        for (int w = 0; w < kWr; ++w) load_one(0, w);
#pragma unroll
        for (int w = 0; w < kWr; ++w) store_one(0, w, 0);
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWr; ++w) load_one(min(1, nk - 1) * kBK, w);
#pragma unroll
        for (int p = 0; p < kR; ++p) read_piece(0, 0, 0, p);
        // One k-step t on stage buf (a compile-time constant in the unrolled pair, so
        // every LDS address is a register base plus an immediate offset).
        auto kstep = [&](auto buf_c, int kt) {
            constexpr int buf = decltype(buf_c)::value;
#pragma unroll
            for (int g = 0; g < kGroups - 1; ++g) {
#pragma unroll
                for (int q = 0; q < kMf; ++q) {
                    mfma_one(g & 1, q);
#pragma unroll
                    for (int p = 2 * q; p < 2 * q + 2; ++p)
                        if (p < kR) read_piece(buf, g + 1, (g + 1) & 1, p);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            constexpr int sl = (kGroups - 1) & 1;
#pragma unroll
            for (int q = 0; q < kPre; ++q) {
                mfma_one(sl, q);
#pragma unroll
                for (int w = q * kWr / kPre; w < (q + 1) * kWr / kPre; ++w)
                    store_one(buf ^ 1, w, min(kt + 1, nk - 1) * kBK);
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
            const int kload = min(kt + 2, nk - 1) * kBK;
            constexpr int kPost = kMf - kPre;
            constexpr int nops = kR + kWr;
#pragma unroll
            for (int q = kPre; q < kMf; ++q) {
                const int qq = q - kPre;
                const int o_lo = qq * nops / kPost, o_hi = (qq + 1) * nops / kPost;
#pragma unroll
                for (int o = o_lo; o < o_hi; ++o) {
                    if (o < kR) read_piece(buf ^ 1, 0, 0, o);
                    else load_one(kload, o - kR);
                }
                mfma_one(sl, q);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        if constexpr (PAIRED) {
            for (int kt = 0; kt < nk; kt += 2) {  // nk is even
                kstep(B0{}, kt);
                kstep(B1{}, kt + 1);
            }
        } else {
            for (int kt = 0; kt < nk; kt += 2) {
                kstep(B0{}, kt);
                if (kt + 1 < nk) kstep(B1{}, kt + 1);
            }
        }
    }

    // 32x32 accumulator layout: register r of lane l holds row 8(r/4) + 4(l/32) + r%4,
    // column l%32 of the block.  Guarded stores for predicated tiles and for unpredicated
    // ones that reach past M x N.
    auto store_all = [&](auto guard_c) {
        constexpr bool G = decltype(guard_c)::value;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int row0 = m0 + wm * Cfg::kTM + 32 * i + 4 * lhi, col = n0 + b_rc0 + 32 * j;
                if constexpr (ACC) store_block32_acc<G, false, false>(acc[i][j], C, ldc, row0, col, M, N, sign, use_old);
                else store_block32<G, false>(acc[i][j], C, ldc, row0, col, M, N);
            }
    };
    if (EDGE || m0 + BM > M || n0 + BN > N) store_all(std::true_type{});
    else store_all(std::false_type{});
}

// Tile coordinates of workgroup `bid`.  Unpredicated launches (EDGE false) cover, in
// XCD-contiguous grouped order, the tiles that lie inside M x N, or with all_tiles every
// tile (ragged ones clamped as above).  Edge launches cover either every tile
// (all_tiles: K is not a multiple of BK) or only the ragged right column strip followed
// by the ragged bottom row strip.
template <bool EDGE>
__device__ __forceinline__ void tile_of(int bid, int nblocks, int tiles_m, int tiles_n,
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

template <int BM, int BN, int WM, int WN, int MINW, int LOAD, bool EDGE, bool PAIRED, bool A_MN,
          bool B_MN, bool ACC, bool KT = false>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(MINW)))
void mfma_f32_gemm_kernel(int M, int N, int K, const float *__restrict__ A, int lda,
                          const float *__restrict__ B, int ldb, float *__restrict__ C, int ldc,
                          float sign, int use_old, int all_tiles) {
    using Cfg = F32Cfg<BM, BN, WM, WN, A_MN, B_MN>;
    __shared__ __attribute__((aligned(16))) float lds[2 * (Cfg::kLdsA + Cfg::kLdsB)];
    const int tiles_m = EDGE || all_tiles ? cdiv(M, BM) : M / BM;
    const int tiles_n = EDGE || all_tiles ? cdiv(N, BN) : N / BN;
    int tm, tn;
    tile_of<EDGE>(blockIdx.x, gridDim.x, tiles_m, tiles_n, N % BN != 0, all_tiles != 0, tm, tn);
    f32_tile<BM, BN, WM, WN, LOAD, EDGE, PAIRED, A_MN, B_MN, ACC, KT>(M, N, K, A, lda, B, ldb, C, ldc,
                                                                 sign, use_old, tm * BM, tn * BN,
                                                                 lds);
}

struct F32Pick {
    int tile;  // 192, 128 or 64
    bool vec;
};

// Whether the unpredicated kernel may take every tile, ragged ones included: K a whole
// number of k-steps and m/n-contiguous extents whole 4-element chunks (rows 16-byte
// aligned load each chunk with one dwordx4, other rows with four dword loads).
inline bool f32_cover_all(const GemmArgs &g) {
    return g.K % kBK == 0 && (!g.trans_a || g.M % 4 == 0) && (g.trans_b || g.N % 4 == 0);
}

// The same with a K tail (K a multiple of 4 but not of BK): the KT kernel.
inline bool f32_ktail(const GemmArgs &g) {
    return g.K % kBK != 0 && g.K % 4 == 0 && (!g.trans_a || g.M % 4 == 0) && (g.trans_b || g.N % 4 == 0);
}

// Cost model: tiles are spread over the 256 CUs, so a config finishes after
// ceil(tiles / 256) tile-times per CU, each proportional to the tile's area over the
// efficiency measured for that tile shape on full tiles (64: 0.85, 128 and 192: 0.95 of
// the MFMA rate); ragged strips run as a second launch at about half that efficiency,
// unless the unpredicated kernel takes every tile.
inline F32Pick pick_f32(const GemmArgs &g) {
    struct Opt { int tile; double eff; };
    const Opt opts[] = {{192, 0.95}, {128, 0.95}, {96, 0.93}, {64, 0.85}};
    const bool vec = rows_aligned16(g.A, g.lda, 4) && rows_aligned16(g.B, g.ldb, 4);
    const bool cover = f32_cover_all(g) || f32_ktail(g);
    double best = -1.0;
    int tile = 64;
    for (const Opt &o : opts) {
        const long full = (long)(g.M / o.tile) * (g.N / o.tile);
        const long all = (long)cdiv(g.M, o.tile) * cdiv(g.N, o.tile);
        const long edge = cover ? 0 : (g.K % kBK == 0 ? all - full : all);
        const double area = (double)o.tile * o.tile;
        const double cost = (double)((all - edge + 255) / 256) * area / o.eff +
                            (double)((edge + 255) / 256) * area / (0.5 * o.eff);
        if (best < 0 || cost < best) {
            best = cost;
            tile = o.tile;
        }
    }
    return {tile, vec};
}

template <int BM, int BN, int WM, int WN, int MINW, int LOAD, bool EDGE, bool PAIRED, bool A_MN,
          bool B_MN, bool ACC, bool KT = false>
hipError_t launch_one(const GemmArgs &g, int tiles, int all_flag, hipStream_t s) {
    hipLaunchKernelGGL((mfma_f32_gemm_kernel<BM, BN, WM, WN, MINW, LOAD, EDGE, PAIRED, A_MN, B_MN, ACC, KT>),
                       dim3(tiles), dim3(64 * WM * WN), 0, s, g.M, g.N, g.K, (const float *)g.A,
                       g.lda, (const float *)g.B, g.ldb, g.C, g.ldc, g.sign, g.accumulate, all_flag);
    return hipGetLastError();
}

// Byte offsets below 2^31 for every chunk of an extent-E tile of the operand.
inline bool f32_fits(bool mn, int ext, int K, int ld) {
    return mn ? ((long)K * ld + ext) * 4 < (1L << 31) : ((long)ext * ld + K) * 4 < (1L << 31);
}

// MINW: waves per SIMD the register budget must allow (resident workgroups per CU
// times waves per workgroup / 4).  Full interior tiles go to the straight-line kernel
// (buffer loads when rows are 16-byte aligned and offsets fit in 31 bits); ragged
// strips (or every tile, when K is not a multiple of BK) to the predicated one.  ACC:
// the variants that store sign * acc (+ C).
// INTERIOR: the caller guarantees whole tiles and K % BK == 0, and only the unpaired
// interior kernels are instantiated (for configurations whose paired and predicated
// kernels do not fit in the register budget).
template <int BM, int BN, int WM, int WN, int MINW, bool A_MN, bool B_MN, bool ACC,
          bool INTERIOR = false>
hipError_t launch_cfg(const GemmArgs &g, bool vec, hipStream_t s) {
    const bool kfull = g.K % kBK == 0;
    const int full_tiles = kfull ? (g.M / BM) * (g.N / BN) : 0;
    const int edge_tiles = cdiv(g.M, BM) * cdiv(g.N, BN) - full_tiles;
    const int all_flag = kfull ? 0 : 1;
    const bool fits = f32_fits(A_MN, BM, g.K, g.lda) && f32_fits(B_MN, BN, g.K, g.ldb);
    if constexpr (!INTERIOR) {
        if (f32_ktail(g) && fits) {  // every tile, K tail included, in one launch
            if (vec)
                return launch_one<BM, BN, WM, WN, MINW, 2, false, false, A_MN, B_MN, ACC, true>(
                    g, cdiv(g.M, BM) * cdiv(g.N, BN), 1, s);
            return launch_one<BM, BN, WM, WN, MINW, 0, false, false, A_MN, B_MN, ACC, true>(
                g, cdiv(g.M, BM) * cdiv(g.N, BN), 1, s);
        }
    }
    if (!INTERIOR && f32_cover_all(g) && edge_tiles > 0) {
        // every tile in one unpredicated launch (ragged tiles clamped, stores guarded)
        if constexpr (!INTERIOR) {
            const int all = cdiv(g.M, BM) * cdiv(g.N, BN);
            if (!vec) return launch_one<BM, BN, WM, WN, MINW, 0, false, false, A_MN, B_MN, ACC>(g, all, 1, s);
            if (fits && (g.K / kBK) % 2 == 0)
                return launch_one<BM, BN, WM, WN, MINW, 2, false, true, A_MN, B_MN, ACC>(g, all, 1, s);
            if (fits) return launch_one<BM, BN, WM, WN, MINW, 2, false, false, A_MN, B_MN, ACC>(g, all, 1, s);
            return launch_one<BM, BN, WM, WN, MINW, 1, false, false, A_MN, B_MN, ACC>(g, all, 1, s);
        }
    }
    if constexpr (!INTERIOR) {
        // Ragged strips that would take a launch (a round) of their own go with the
        // interior tiles into one launch of the predicated kernel when that takes fewer
        // rounds at its slower pace (up to 1.5x an interior tile's time): FP32
        // 1000 x 1000 x 1024 with lda 1025 61 -> 40 us; 3000 x 3000 x 3008 and 4000^3
        // (lda + 1) measured 3 % slower in one launch and keep two.
        if (full_tiles > 0 && edge_tiles > 0) {
            const int all = full_tiles + edge_tiles;
            if (cdiv(all, 256) * 3 < cdiv(full_tiles, 256) * 2 + cdiv(edge_tiles, 256) * 3) {
                if (vec) return launch_one<BM, BN, WM, WN, MINW, 1, true, false, A_MN, B_MN, ACC>(g, all, 1, s);
                return launch_one<BM, BN, WM, WN, MINW, 0, true, false, A_MN, B_MN, ACC>(g, all, 1, s);
            }
        }
    }
    if (full_tiles > 0) {
        hipError_t e = hipSuccess;
        if (!INTERIOR && vec && fits && (g.K / kBK) % 2 == 0) {
            if constexpr (!INTERIOR)
                e = launch_one<BM, BN, WM, WN, MINW, 2, false, true, A_MN, B_MN, ACC>(g, full_tiles, all_flag, s);
        } else if (vec && fits)
            e = launch_one<BM, BN, WM, WN, MINW, 2, false, false, A_MN, B_MN, ACC>(g, full_tiles, all_flag, s);
        else if (vec)
            e = launch_one<BM, BN, WM, WN, MINW, 1, false, false, A_MN, B_MN, ACC>(g, full_tiles, all_flag, s);
        else
            e = launch_one<BM, BN, WM, WN, MINW, 0, false, false, A_MN, B_MN, ACC>(g, full_tiles, all_flag, s);
        if (e != hipSuccess) return e;
    }
    if (edge_tiles > 0) {
        if constexpr (INTERIOR) {
            return hipErrorInvalidValue;  // excluded by the caller
        } else {
            if (vec) return launch_one<BM, BN, WM, WN, MINW, 1, true, false, A_MN, B_MN, ACC>(g, edge_tiles, all_flag, s);
            return launch_one<BM, BN, WM, WN, MINW, 0, true, false, A_MN, B_MN, ACC>(g, edge_tiles, all_flag, s);
        }
    }
    return hipSuccess;
}

// With both operands m/n-contiguous every fragment takes four ds_read_b32 per group; in
// the 12-wave 192 x 192 tile (168 registers per wave) only the unpaired interior kernels
// hold that, so this layout takes the 192 tile when M and N are multiples of 192 and K of
// 32 (no edge tiles) and the 128 x 128 tile otherwise.
template <bool A_MN, bool B_MN, bool ACC>
hipError_t launch_f32_layout(const GemmArgs &g, hipStream_t s) {
    const F32Pick p = pick_f32(g);
    const bool whole192 = g.M % 192 == 0 && g.N % 192 == 0 && g.K % kBK == 0;
    const int tile = (A_MN && B_MN && p.tile == 192 && !whole192) ? 128 : p.tile;
    switch (tile) {
    case 192:
        if constexpr (!(A_MN && B_MN)) return launch_cfg<192, 192, 2, 6, 3, A_MN, B_MN, ACC>(g, p.vec, s);
        else return launch_cfg<192, 192, 2, 6, 3, A_MN, B_MN, ACC, true>(g, p.vec, s);
    case 128: return launch_cfg<128, 128, 2, 4, 2, A_MN, B_MN, ACC>(g, p.vec, s);
    case 96: return launch_cfg<96, 96, 1, 3, 3, A_MN, B_MN, ACC>(g, p.vec, s);
    default: return launch_cfg<64, 64, 2, 2, 4, A_MN, B_MN, ACC>(g, p.vec, s);
    }
}

}  // namespace

}  // namespace g355
