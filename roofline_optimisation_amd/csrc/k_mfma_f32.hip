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
//  * edges: tiles that cross M, N or the K tail load with per-element predicates and
//    zero fill and store with a guard; interior tiles take the unpredicated path;
//  * launch order: tiles are renumbered so each XCD receives a contiguous range, walked
//    in groups of 4 tile-rows, which keeps shared A and B panels in that XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace g355 {

namespace {

constexpr int kBK = 32;
constexpr int kSA = kBK + 4;  // A LDS row stride (words)

template <int BM, int BN, int WM, int WN>
struct F32Cfg {
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kTM = BM / WM, kTN = BN / WN;
    static constexpr int kMB = kTM / 32, kNB = kTN / 32;
    static constexpr int kSB = BN + 8;  // B LDS row stride (words)
    static constexpr int kAChunks = BM * kBK / 4 / kThreads;
    static constexpr int kBChunks = kBK * BN / 4 / kThreads;
    static constexpr int kLdsA = BM * kSA;
    static constexpr int kLdsB = kBK * kSB;
    static constexpr int kLdsBytes = 2 * (kLdsA + kLdsB) * 4;
    static_assert(kTM % 32 == 0 && kTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert((BM * kBK / 4) % kThreads == 0 && (kBK * BN / 4) % kThreads == 0,
                  "tile chunks must divide over the threads");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
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

// One BM x BN tile of C.  EDGE selects the predicated loads and guarded stores; the
// interior instance (tile inside M x N, K a multiple of BK) is straight-line code, so
// the dwordx4 loads of a k-step issue back to back.
template <int BM, int BN, int WM, int WN, bool VEC, bool EDGE>
__device__ __forceinline__ void f32_tile(int M, int N, int K, const float *__restrict__ A, int lda,
                                         const float *__restrict__ B, int ldb,
                                         float *__restrict__ C, int ldc, int m0, int n0,
                                         float *lds) {
    using Cfg = F32Cfg<BM, BN, WM, WN>;
    constexpr int T = Cfg::kThreads;
    constexpr int MB = Cfg::kMB, NB = Cfg::kNB;
    constexpr int SB = Cfg::kSB;

    const int t = threadIdx.x;
    const int lane = t % 64, wave = t / 64;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane % 32, lhi = lane / 32;

    // Per-thread global chunk coordinates (fixed across k-steps).
    int a_r[Cfg::kAChunks], a_c[Cfg::kAChunks];
    int b_r[Cfg::kBChunks], b_c[Cfg::kBChunks];
#pragma unroll
    for (int i = 0; i < Cfg::kAChunks; ++i) {
        const int q = t + T * i;
        a_r[i] = q / (kBK / 4);
        a_c[i] = (q % (kBK / 4)) * 4;
    }
#pragma unroll
    for (int i = 0; i < Cfg::kBChunks; ++i) {
        const int q = t + T * i;
        b_r[i] = q / (BN / 4);
        b_c[i] = (q % (BN / 4)) * 4;
    }

    floatx4 sa[Cfg::kAChunks], sb[Cfg::kBChunks];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < Cfg::kAChunks; ++i) {
            const int r = m0 + a_r[i];
            const bool ok = !EDGE || r < M;
            sa[i] = ld_chunk<VEC, EDGE>(A + (size_t)(ok ? r : 0) * lda, k0 + a_c[i], K, ok);
        }
#pragma unroll
        for (int i = 0; i < Cfg::kBChunks; ++i) {
            const int r = k0 + b_r[i];
            const bool ok = !EDGE || r < K;
            sb[i] = ld_chunk<VEC, EDGE>(B + (size_t)(ok ? r : 0) * ldb, n0 + b_c[i], N, ok);
        }
    };
    auto store_tile = [&](int buf) {
        float *As = lds + buf * (Cfg::kLdsA + Cfg::kLdsB);
        float *Bs = As + Cfg::kLdsA;
#pragma unroll
        for (int i = 0; i < Cfg::kAChunks; ++i)
            *reinterpret_cast<floatx4 *>(As + a_r[i] * kSA + a_c[i]) = sa[i];
#pragma unroll
        for (int i = 0; i < Cfg::kBChunks; ++i)
            *reinterpret_cast<floatx4 *>(Bs + b_r[i] * SB + b_c[i]) = sb[i];
    };

    floatx16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = cdiv(K, kBK);
    if (nk > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    const int a_row0 = wm * Cfg::kTM + l32;  // + 32 mb
    const int b_col0 = wn * Cfg::kTN + l32;  // + 32 nb
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tile((kt + 1) * kBK);
        const float *As = lds + buf * (Cfg::kLdsA + Cfg::kLdsB);
        const float *Bs = As + Cfg::kLdsA;
#pragma unroll
        for (int kg = 0; kg < kBK / 8; ++kg) {
            const int kq = kg * 8 + 4 * lhi;
            floatx4 af[MB];
            float bf[NB][4];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                af[i] = *reinterpret_cast<const floatx4 *>(As + (a_row0 + 32 * i) * kSA + kq);
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int s = 0; s < 4; ++s) bf[j][s] = Bs[(kq + s) * SB + b_col0 + 32 * j];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][s], bf[j][s],
                                                                         acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tile(buf ^ 1);
        __syncthreads();
    }

    // 32x32 accumulator layout: register r of lane l holds row 8(r/4) + 4(l/32) + r%4,
    // column l%32 of the block.
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int col = n0 + b_col0 + 32 * j;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * Cfg::kTM + 32 * i + 8 * (r / 4) + 4 * lhi + (r % 4);
                if (!EDGE || (row < M && col < N)) C[(size_t)row * ldc + col] = acc[i][j][r];
            }
        }
    }
}

// Tile coordinates of workgroup `bid`.  Interior launches (EDGE false) cover the
// tiles_m_full x tiles_n_full tiles that lie inside M x N, in XCD-contiguous grouped
// order.  Edge launches cover either every tile (all_tiles: K is not a multiple of BK)
// or only the ragged right column strip followed by the ragged bottom row strip.
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

template <int BM, int BN, int WM, int WN, int MINW, bool VEC, bool EDGE>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(MINW)))
void mfma_f32_gemm_kernel(int M, int N, int K, const float *__restrict__ A, int lda,
                          const float *__restrict__ B, int ldb, float *__restrict__ C, int ldc,
                          int all_tiles) {
    using Cfg = F32Cfg<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(16))) float lds[2 * (Cfg::kLdsA + Cfg::kLdsB)];
    const int tiles_m = EDGE ? cdiv(M, BM) : M / BM;
    const int tiles_n = EDGE ? cdiv(N, BN) : N / BN;
    int tm, tn;
    tile_of<EDGE>(blockIdx.x, gridDim.x, tiles_m, tiles_n, N % BN != 0, all_tiles != 0, tm, tn);
    f32_tile<BM, BN, WM, WN, VEC, EDGE>(M, N, K, A, lda, B, ldb, C, ldc, tm * BM, tn * BN, lds);
}

struct F32Pick {
    int tile;  // 192, 128 or 64
    bool vec;
};

// Cost model: a tile config with w resident workgroups per CU finishes in
// ceil(tiles / (256 w)) rounds of w * BM * BN work each; pick the cheapest, larger
// tiles first on ties (less L2 traffic per FLOP).
F32Pick pick_f32(const GemmArgs &g) {
    struct Opt { int tile, per_cu; };
    const Opt opts[] = {{192, 1}, {128, 2}, {64, 4}};
    long best = -1;
    int tile = 64;
    for (const Opt &o : opts) {
        const long tiles = (long)cdiv(g.M, o.tile) * cdiv(g.N, o.tile);
        const long slots = 256L * o.per_cu;
        const long rounds = (tiles + slots - 1) / slots;
        const long cost = rounds * o.per_cu * (long)o.tile * o.tile;
        if (best < 0 || cost < best) {
            best = cost;
            tile = o.tile;
        }
    }
    const bool vec = rows_aligned16(g.A, g.lda, 4) && rows_aligned16(g.B, g.ldb, 4);
    return {tile, vec};
}

// MINW: waves per SIMD the register budget must allow (resident workgroups per CU
// times waves per workgroup / 4).  Full interior tiles go to the straight-line kernel;
// ragged strips (or every tile, when K is not a multiple of BK) to the predicated one.
template <int BM, int BN, int WM, int WN, int MINW>
hipError_t launch_cfg(const GemmArgs &g, bool vec, hipStream_t s) {
    const dim3 block(64 * WM * WN);
    const bool kfull = g.K % kBK == 0;
    const int full_tiles = kfull ? (g.M / BM) * (g.N / BN) : 0;
    const int all = cdiv(g.M, BM) * cdiv(g.N, BN);
    const int edge_tiles = all - full_tiles;
    const int all_flag = kfull ? 0 : 1;
    const float *A = (const float *)g.A, *B = (const float *)g.B;
    if (full_tiles > 0) {
        if (vec)
            hipLaunchKernelGGL((mfma_f32_gemm_kernel<BM, BN, WM, WN, MINW, true, false>),
                               dim3(full_tiles), block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb,
                               g.C, g.ldc, all_flag);
        else
            hipLaunchKernelGGL((mfma_f32_gemm_kernel<BM, BN, WM, WN, MINW, false, false>),
                               dim3(full_tiles), block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb,
                               g.C, g.ldc, all_flag);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (edge_tiles > 0) {
        if (vec)
            hipLaunchKernelGGL((mfma_f32_gemm_kernel<BM, BN, WM, WN, MINW, true, true>),
                               dim3(edge_tiles), block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb,
                               g.C, g.ldc, all_flag);
        else
            hipLaunchKernelGGL((mfma_f32_gemm_kernel<BM, BN, WM, WN, MINW, false, true>),
                               dim3(edge_tiles), block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb,
                               g.C, g.ldc, all_flag);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

const char *desc_mfma_f32(const GemmArgs &g) {
    const F32Pick p = pick_f32(g);
    switch (p.tile) {
    case 192: return p.vec ? "mfma_f32 192x192x32 w2x2 dwordx4" : "mfma_f32 192x192x32 w2x2 dword";
    case 128: return p.vec ? "mfma_f32 128x128x32 w2x2 dwordx4" : "mfma_f32 128x128x32 w2x2 dword";
    default: return p.vec ? "mfma_f32 64x64x32 w2x2 dwordx4" : "mfma_f32 64x64x32 w2x2 dword";
    }
}

hipError_t launch_mfma_f32(const GemmArgs &g, hipStream_t s) {
    const F32Pick p = pick_f32(g);
    switch (p.tile) {
    case 192: return launch_cfg<192, 192, 2, 2, 1>(g, p.vec, s);
    case 128: return launch_cfg<128, 128, 2, 2, 2>(g, p.vec, s);
    default: return launch_cfg<64, 64, 2, 2, 4>(g, p.vec, s);
    }
}

}  // namespace g355
