// 256 x 256 and 128 x 128 interior tiles of the FP16 / BF16 GEMM fed by direct global
// -> LDS loads and multiplied with v_mfma_f32_16x16x32_{f16,bf16}.  Included by
// h16_gemm.hpp.
//
// Data movement ("Kernel optimisation guide", Level 3 double buffering, extended to a
// ring; the overlap of loads and arithmetic in the scheduling section of "Advanced
// CUDA features - starting from GEMM"):
//  * K is walked in steps of 32.  An m/n-contiguous operand goes through a ring of kNs
//    stages (4 of 16 KiB for 256-wide tiles, 8 of 8 KiB for 128-wide ones), its loads of
//    k-step t + kNs - 1 issued while step t is multiplied, into the stage step t-1 has
//    released; a k-contiguous operand goes through kNs/2 slots of a 64-wide double step,
//    loaded every other k-step, so that its loads read whole 128-byte lines (with
//    32-wide steps each line would be fetched twice, half of it each time);
//  * a load is buffer_load_dwordx4 with the lds flag: lane l's 16 bytes land at
//    m0 + 16 l, so one instruction fills 1 KiB of LDS (8 rows of a KM operand, 2 or 4
//    rows of an MN operand) and the lane -> source mapping chooses where each 16-byte
//    chunk goes;
//  * a KM operand's rows are 128 bytes, chunk c of row r stored in slot c ^ ((r / 2) %
//    8); an MN operand's rows are 2 E bytes (E = 256 or 128), chunk c of row k in slot
//    c ^ 4 (k % 4) ^ 2 ((k / 8) % 2).  With these the fragment reads (ds_read_b128 for
//    KM, ds_read_b64_tr_b16 for MN) touch distinct banks within every 16 lanes of a
//    b128 read and every 32 lanes of a b64 read, i.e. no bank conflicts, without padding
//    (which a contiguous 1 KiB load cannot skip);
//  * each wave waits for its own loads of step t+1 (vmcnt), then one barrier per
//    k-step publishes them to all four waves.
//
// Arithmetic: each wave owns E/2 x E/2 of C as blocks of 16 x 16 (E = 256: 8 x 8 FP32
// accumulator quads, 256 accumulator registers) and multiplies a whole 32-wide k-step
// per instruction.  The 16x16x32 form was chosen over 32x32x16 (same arithmetic per
// k-step, same fragment bytes) because the part sustains a higher clock on it under the
// same operands: on register-resident U[-1,1] binary16 data 1.97 against 1.72 GHz.  Per
// lane l a fragment holds 8 consecutive k (8 (l/16) .. +7) of row (A) or column (B)
// l%16; the accumulator quad holds column l%16, rows 4 (l/16) .. +3.
//
// The loads are issued from inline assembly (m0 holds the LDS destination), so the
// compiler neither tracks them nor waits for them; the kernel's own s_waitcnt vmcnt
// instructions do, and no other code of this kernel uses m0.
#pragma once

namespace dma {

constexpr int kBK = 32;
constexpr int kWM = 2, kWN = 2, kWaves = kWM * kWN;

// Geometry of an E x E tile (E = 256 or 128; both operands have extent E).  A 128-wide
// tile's k-step is a quarter of a 256-wide one's arithmetic (16 MFMAs, ~130 ns), so its
// ring has kNs = 8 stages instead of 4 to keep the loads as far ahead in time.
template <int E>
struct Geo {
    static constexpr int kNs = E == 256 ? 4 : 8;  // ring stages (k-steps)
    static constexpr int kTM = E / kWM, kTN = E / kWN;     // wave tile
    static constexpr int kMB = kTM / 16, kNB = kTN / 16;    // accumulator quads per wave
    static constexpr int kStage = E * kBK * 2;   // bytes per operand per stage (E x 32)
    static constexpr int kBOff = kNs * kStage;   // the B ring follows the A ring
    static constexpr int kLds = 2 * kNs * kStage;
    static constexpr int kI = kStage / 1024 / kWaves;  // MN: 1 KiB loads per wave per k-step
    static constexpr int kRowB = 2 * E;          // MN: bytes per LDS row (one k)
    static constexpr int kRpi = 1024 / kRowB;    // MN: rows one load instruction fills
    static constexpr int kKMRows = E / kWaves;   // KM: rows one wave fills
    // MFMAs per k-step, the step's wait and barrier after kBarrier of them, its loads
    // spread over the first kLoadHi
    static constexpr int kMf = kMB * kNB;
    static constexpr int kBarrier = E == 256 ? 40 : 10;
    static constexpr int kLoadHi = E == 256 ? 32 : 8;
    static_assert(E == 256 || E == 128, "tile extents");
    static_assert(kLds <= 160 * 1024, "LDS budget");
    static_assert(kI * kRpi == 8, "an MN operand's wave fills 8 rows, all of one (k / 8) parity");
    static_assert(kKMRows / 8 == 2 * kI, "a KM double step takes twice an MN step's loads");
    // every ds_read immediate (slot / stage + block / row offsets) stays below 64 KiB
    static_assert((kNs / 2 - 1) * 2 * kStage + (kMB - 1) * 2048 < 65536, "KM read offsets");
    static_assert((kNs - 1) * kStage + 4 * kRowB < 65536, "MN read offsets");
    static_assert(kLoadHi <= kBarrier && kBarrier < kMf, "the step's loads precede its wait");
};

typedef int int4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// D = A.B + C on one 16 x 16 accumulator quad, C and D in the same accumulator
// registers.  Inline assembly ties the accumulator to one AGPR quad for the whole loop
// (with the builtin the register allocator moved accumulators between register files
// at every k-step); the caller keeps the wait states the compiler does not see.
template <typename T>
__device__ __forceinline__ floatx4 mfma16(u16x8 a, u16x8 b, floatx4 c);
template <>
__device__ __forceinline__ floatx4 mfma16<f16_t>(u16x8 a, u16x8 b, floatx4 c) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
}
template <>
__device__ __forceinline__ floatx4 mfma16<bf16_t>(u16x8 a, u16x8 b, floatx4 c) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
}

// A raw buffer resource over `p` (2^31 - 1 bytes; the host checks every offset fits).
__device__ __forceinline__ int4v rsrc_of(const void *p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    int4v r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    r[2] = 0x7fffffff;
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from the buffer at voff + soff into LDS at lds_dst + 16 * lane.
// m0 must be written right before the load; one wait state separates the two.
__device__ __forceinline__ void load_lds16(uint32_t lds_dst, uint32_t voff, int4v rsrc,
                                           uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_dst), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ lds_char *lds_reg(lds_char *p) {
    uint32_t a = (uint32_t)(uintptr_t)p;
    asm volatile("" : "+v"(a));
    return (lds_char *)(uintptr_t)a;
}

// Loads and fragment reads of one operand of extent E in its region at byte offset
// `roff` (4 E x 32 x 2 bytes: 64 KiB for E = 256).
//  * MN (m/n-contiguous): a ring of kNs stages of one 32-wide k-step (E x 32 halves,
//    rows of 2 E bytes).  Wave w fills rows [8 w, +8): instruction i rows
//    8 w + R i + l / (64 / R) with R = 1024 / (2 E) rows per instruction, lane slot
//    l % (64 / R) taking chunk slot ^ 4 (row % 4) ^ 2 ((row / 8) % 2), where
//    (row / 8) % 2 = w % 2 and row % 4 = l/32 + 2 (i % 2) (E = 256) or l/16 (E = 128).
//  * KM (k-contiguous): kNs / 2 slots of one 64-wide double step (E rows of 128 bytes),
//    so that every load reads whole 128-byte lines; k-step t uses half t % 2 of slot
//    (t / 2) % (kNs / 2).  Wave w fills rows [E/4 w, +E/4), instruction i rows 8 i + l/8, lane
//    slot l%8 taking chunk slot ^ ((row / 2) % 8), where (row / 2) % 8 =
//    4 (i % 2) + l/16.
template <bool MN, int E>
struct DmaOp {
    using G = Geo<E>;
    static constexpr int NB = E / 32;                // quads along this operand per wave
    static constexpr int kSlot = 2 * G::kStage;      // KM slot bytes
    static constexpr int kPieces = MN ? 2 : 1;       // LDS reads per fragment
    int4v rsrc;
    uint32_t voff[MN ? 2 : 2 * G::kI];   // per lane: MN by instruction parity, KM by instruction
    lds_char *rd[MN ? NB : 2];
    H16Frag<MN, NB> fr;

    // X: the operand, whose rows (KM) or columns (MN) number ext (a multiple of 8 for
    // MN); mn0: the tile's first row (KM) or column (MN); wb: the wave's first row or
    // column within the tile.  In a ragged tile a lane whose source row (KM) or 16-byte
    // column chunk (MN) lies beyond ext loads the last one inside instead, so every load
    // stays within the operand; what it puts in LDS only reaches outputs beyond row M or
    // column N, which are never stored.
    __device__ __forceinline__ void init(const uint16_t *X, int ld, int ext, int mn0, int wave,
                                         int lane, lds_char *L, int roff, int wb) {
        if constexpr (MN) {
            constexpr int lpr = 64 / G::kRpi;        // lanes per row of one load
            rsrc = rsrc_of(X + mn0);
            const int rl = lane / lpr, row = 8 * wave + rl, slot = lane % lpr;
            const int kx = 2 * (wave & 1), last = (ext - mn0) / 8 - 1;
#pragma unroll
            for (int p = 0; p < 2; ++p)
                voff[p] = (uint32_t)((row * ld + 8 * min(slot ^ (4 * ((G::kRpi * p + rl) % 4)) ^ kx, last)) * 2);
            // block b, piece h: lane (g = l/16, e = (l%16)/4, q = l%4) reads row 8 g + 4 h +
            // e, chunk wb/8 + 2 b + q/2, byte 8 (q%2) of it; that row's swizzle key is
            // 4 e ^ 2 (g%2)
            const int g = lane >> 4, e = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                rd[b] = lds_reg(L + roff + (8 * g + e) * G::kRowB +
                                16 * ((wb / 8 + 2 * b + (q >> 1)) ^ (4 * e) ^ (2 * (g & 1))) +
                                8 * (q & 1));
        } else {
            rsrc = rsrc_of(X + (size_t)mn0 * ld);
            const int row = G::kKMRows * wave + lane / 8, slot = lane & 7, last = ext - mn0 - 1;
#pragma unroll
            for (int i = 0; i < 2 * G::kI; ++i)
                voff[i] = (uint32_t)((min(row + 8 * i, last) * ld +
                                      8 * (slot ^ ((4 * (i % 2) + lane / 16) & 7))) * 2);
            // block b, half h of the slot: row wb + 16 b + l%16, chunk 4 h + l/16, whose
            // swizzle key ((l%16) / 2) % 8 does not depend on b
            const int l16 = lane & 15, lq = lane >> 4;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                rd[h] = lds_reg(L + roff + (wb + l16) * 128 + 16 * ((4 * h + lq) ^ (l16 >> 1)));
        }
    }
    // Load instruction i of one issue: MN: k-step at k0 into stage `place`; KM: the
    // double step at k0 into slot `place`.
    __device__ __forceinline__ void issue(uint32_t lds0, int roff, int wave, int ld, int place,
                                          int k0, int i) {
        if constexpr (MN) {
            const uint32_t dst = lds0 + roff + place * G::kStage + (wave * G::kI + i) * 1024;
            load_lds16(dst, voff[i & 1], rsrc, (uint32_t)((k0 + G::kRpi * i) * ld * 2));
        } else {
            const uint32_t dst = lds0 + roff + place * kSlot + (wave * 2 * G::kI + i) * 1024;
            load_lds16(dst, voff[i], rsrc, (uint32_t)(k0 * 2));
        }
    }
    // Piece h of block b of k-step u (u = t % kNs, so the MN stage is u, the KM slot
    // u / 2 and the KM half u % 2) into fragment slot `fslot`.
    __device__ __forceinline__ void read(int u, int fslot, int b, int h) {
        if constexpr (MN) {
            fr.f[fslot][b][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_shortx4 *)(rd[b] + u * G::kStage + 4 * h * G::kRowB));
        } else {
            fr.f[fslot][b] = *(const lds_u16x8 *)(rd[u % 2] + (u / 2) * kSlot + b * 2048);
        }
    }
};

// The order in which a k-step's fragment pieces are read: A block 0, then the B blocks,
// then the other A blocks, i.e. in the order the MFMAs (A block outer, B block inner,
// odd rows walking the B blocks backwards) first use them.
template <bool A_MN, bool B_MN, int E>
struct PieceOrder {
    static constexpr int kMB = Geo<E>::kMB, kNB = Geo<E>::kNB;
    static constexpr int kPA = A_MN ? 2 : 1, kPB = B_MN ? 2 : 1;
    static constexpr int kR = kMB * kPA + kNB * kPB;
    // piece p -> (operand 0 = A / 1 = B, block, half)
    static constexpr int op(int p) { return p < kPA ? 0 : (p < kPA + kNB * kPB ? 1 : 0); }
    static constexpr int blk(int p) {
        return p < kPA ? 0 : (p < kPA + kNB * kPB ? (p - kPA) / kPB : 1 + (p - kPA - kNB * kPB) / kPA);
    }
    static constexpr int half(int p) {
        return p < kPA ? p : (p < kPA + kNB * kPB ? (p - kPA) % kPB : (p - kPA - kNB * kPB) % kPA);
    }
};

// kstep(kt, integral_constant<u>) for u = 0 .. kNs-1 in order.
template <typename F, int... U>
__device__ __forceinline__ void for_steps(F &kstep, int kt, std::integer_sequence<int, U...>) {
    (kstep(kt, std::integral_constant<int, U>{}), ...);
}

// Empty volatile statements that take every accumulator quad in and out of an AGPR:
// code that defines the accumulators stays before them and code that reads them after,
// so they order the accumulators' writes and reads with respect to the explicit wait
// states around the inline-assembly MFMAs.
template <int kMB, int kNB>
__device__ __forceinline__ void pin_acc(floatx4 (&acc)[kMB][kNB]) {
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// The FP32 accumulator quads of one wave, stored to C: quad (i, j) holds rows
// row0 + 16 i + 4 (l/16) + r, column col0 + 16 j + l%16.  EDGE (a tile reaching past
// row M or column N) guards every access.  For each row the eight quads of
// a block row go out back to back, so every 128-byte line of C is written whole by two
// consecutive stores.  The stores are ordinary (cached) ones: each instruction writes
// half lines, which the L2 merges; as non-temporal stores the same pattern took 40 %
// longer (64 MiB from 256 workgroups: 15.8 against 11.2 us).
template <int EPI, typename T, bool EDGE, int kMB, int kNB>
__device__ __forceinline__ void store_tile(floatx4 (&acc)[kMB][kNB], float *__restrict__ C, int ldc,
                                           int row0, int col0, int M, int N, float sign, int flags) {
    const int lane = threadIdx.x & 63;
    const int rl = row0 + 4 * (lane >> 4);
    if constexpr (EPI == 0) {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < kNB; ++j) {
                    const int row = rl + 16 * i + r, col = col0 + 16 * j + (lane & 15);
                    if (!EDGE || (row < M && col < N)) C[(size_t)row * ldc + col] = acc[i][j][r];
                }
    } else if constexpr (EPI == 1) {
        const bool use_old = flags & 1;
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                store_quad16_acc<EDGE>(acc[i][j], C, ldc, rl + 16 * i, col0 + 16 * j + (lane & 15),
                                       M, N, sign, use_old);
    } else {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kNB; j += 2)
                store_pair16_c16<EDGE, T>(acc[i][j], acc[i][j + 1], (uint16_t *)C, ldc, rl + 16 * i,
                                          col0 + 16 * j, M, N, sign, flags);
    }
}

template <typename T, bool A_MN, bool B_MN, int EPI, int E>
__device__ __forceinline__ void dma_tile(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                                         const uint16_t *__restrict__ B, int ldb,
                                         float *__restrict__ C, int ldc, float sign,
                                         int flags, int m0, int n0, char *lds_raw) {
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int wm = wave / kWN, wn = wave % kWN;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char *)lds_raw;
    lds_char *const L = (lds_char *)lds_raw;

    using G = Geo<E>;
    constexpr int kMB = G::kMB, kNB = G::kNB, kI = G::kI, kBOff = G::kBOff, kNs = G::kNs;
    using OA = DmaOp<A_MN, E>;
    using OB = DmaOp<B_MN, E>;
    using PO = PieceOrder<A_MN, B_MN, E>;
    OA oa;
    OB ob;
    oa.init(A, lda, M, m0, wave, lane, L, 0, wm * G::kTM);
    ob.init(B, ldb, N, n0, wave, lane, L, kBOff, wn * G::kTN);
    // Loads per wave: nMN every k-step (the MN operands' next stage), nKM every other
    // k-step (the KM operands' next double step), MN loads first.
    constexpr int nMN = (A_MN ? kI : 0) + (B_MN ? kI : 0);
    constexpr int nKM = (A_MN ? 0 : 2 * kI) + (B_MN ? 0 : 2 * kI);
    // issue w of an MN batch (k-step at k0 into stage st) / of a KM batch (double step at
    // k0 into slot sl)
    auto issue_mn = [&](int st, int k0, int w) {
        if constexpr (A_MN) {
            if (w < kI) { oa.issue(lds0, 0, wave, lda, st, k0, w); return; }
            w -= kI;
        }
        if constexpr (B_MN) ob.issue(lds0, kBOff, wave, ldb, st, k0, w);
    };
    auto issue_km = [&](int sl, int k0, int w) {
        if constexpr (!A_MN) {
            if (w < 2 * kI) { oa.issue(lds0, 0, wave, lda, sl, k0, w); return; }
            w -= 2 * kI;
        }
        if constexpr (!B_MN) ob.issue(lds0, kBOff, wave, ldb, sl, k0, w);
    };
    constexpr int kR = PO::kR;
    auto read_piece = [&](int u, int fslot, int p) {
        if (PO::op(p) == 0) oa.read(u, fslot, PO::blk(p), PO::half(p));
        else ob.read(u, fslot, PO::blk(p), PO::half(p));
    };

    floatx4 acc[kMB][kNB];

    // One k-step t = kt + u (u = t % kNs is a compile-time constant): kMf MFMAs on the
    // fragments in slot u % 2.  The step's loads (MN: k-step t + kNs - 1 into stage
    // (u - 1) % kNs; on even steps KM: double step t/2 + kNs/2 - 1 into the slot of double
    // step t/2 - 1) are spread over the first kLoadHi MFMAs; after kBarrier MFMAs the wave
    // waits until the loads step t+1 needs are done, then the barrier publishes them and
    // the fragments of t+1 are read into the other slot under the remaining MFMAs, in the
    // order of their first use.  Loads are issued in step order (a step's MN loads, then
    // its KM loads), the prologue's included, so the wait counts are the loads of the
    // steps after the one that issued what step t+1 needs: on an even step t both of its
    // operands' loads came from step t - kNs + 2, so the loads of the kNs - 2 steps after
    // it may stay in flight; on an odd step its KM loads came from step t - kNs + 3
    // (those of kNs - 3 later steps may stay), its MN loads alone from t - kNs + 2.  No
    // branches: near the end the loads repeat the last k-step or double step into free
    // stages or slots.
    constexpr int kMf = G::kMf, kBarrier = G::kBarrier, kLoadHi = G::kLoadHi;
    auto ev_begin = [](int qs, int n, int lo, int hi) {
        if (qs <= lo) return 0;
        if (qs >= hi) return n;
        return ((qs - lo) * n + (hi - lo) - 1) / (hi - lo);
    };
    const int nk = K / kBK;
    auto kstep = [&](int kt, auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int u1 = (u + 1) % kNs;
        constexpr int f = u % 2;
        constexpr bool even = u % 2 == 0;
        constexpr int nLd = nMN + (even ? nKM : 0);
        constexpr int kWait = even ? (kNs - 2) * nMN + (kNs - 2) / 2 * nKM
                                   : (nKM ? (kNs - 3) * nMN + (kNs - 4) / 2 * nKM : (kNs - 2) * nMN);
        static_assert(kWait < 64, "vmcnt range");
        const int t = kt + u;
        const int k_mn = min(t + kNs - 1, nk - 1) * kBK;
        const int k_km = min(t / 2 + kNs / 2 - 1, nk / 2 - 1) * 2 * kBK;
#pragma unroll
        for (int qs = 0; qs < kMf; ++qs) {
            // snake order: odd block rows walk the B blocks backwards, so consecutive
            // MFMAs change one operand (measured 2 % faster on register-resident data:
            // the operands' bit changes are what the part's power limit charges for)
            const int i = qs / kNB, j = (i & 1) ? kNB - 1 - qs % kNB : qs % kNB;
            acc[i][j] = mfma16<T>(oa.fr.get(f, i), ob.fr.get(f, j), acc[i][j]);
            if (qs >= kBarrier) {
                const int lo = ev_begin(qs - kBarrier, kR, 0, kMf - kBarrier);
                const int hi = ev_begin(qs - kBarrier + 1, kR, 0, kMf - kBarrier);
#pragma unroll
                for (int o = lo; o < hi; ++o) read_piece(u1, 1 - f, o);
            }
            {
                const int lo = ev_begin(qs, nLd, 0, kLoadHi);
                const int hi = ev_begin(qs + 1, nLd, 0, kLoadHi);
#pragma unroll
                for (int w = lo; w < hi; ++w) {
                    if (w < nMN) issue_mn((u + kNs - 1) % kNs, k_mn, w);
                    else issue_km((u / 2 + kNs / 2 - 1) % (kNs / 2), k_km, w - nMN);
                }
            }
            if (qs == kBarrier - 1) {
                wait_vmcnt<kWait>();
                __syncthreads();
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue, in the order the steps before step 0 would have issued it: KM double step
    // 0, then MN k-steps 0 .. kNs-2 into stages 0 .. kNs-2, KM double step d after MN
    // k-step 2d + 1 (d = 1 .. kNs/2 - 2); wait for step 0's data (everything after MN
    // k-step 0 may stay in flight), read its fragments
#pragma unroll
    for (int w = 0; w < nKM; ++w) issue_km(0, 0, w);
#pragma unroll
    for (int p = 0; p < kNs - 1; ++p) {
#pragma unroll
        for (int w = 0; w < nMN; ++w) issue_mn(p, min(p, nk - 1) * kBK, w);
        if (p % 2 == 1 && p >= 3) {
#pragma unroll
            for (int w = 0; w < nKM; ++w)
                issue_km((p - 1) / 2, min((p - 1) / 2, nk / 2 - 1) * 2 * kBK, w);
        }
    }
    wait_vmcnt<(kNs - 2) * nMN + (kNs / 2 - 2) * nKM>();
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kR; ++p) read_piece(0, 0, p);
    // The MFMAs are inline assembly, so the compiler inserts no wait states for them:
    // the accumulators are zeroed here, at least 16 wait states before the first MFMA
    // reads them, and the epilogue reads them at least 32 wait states after the last
    // MFMA (an 8-pass MFMA's result may be read 11 wait states after it issues).
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    pin_acc(acc);
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    for (int kt = 0; kt < nk; kt += kNs)
        for_steps(kstep, kt, std::make_integer_sequence<int, kNs>{});
    // nothing may still write this workgroup's LDS when it exits
    wait_vmcnt<0>();
    pin_acc(acc);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    pin_acc(acc);
    if (m0 + E <= M && n0 + E <= N)
        store_tile<EPI, T, false>(acc, C, ldc, m0 + wm * G::kTM, n0 + wn * G::kTN, M, N, sign, flags);
    else
        store_tile<EPI, T, true>(acc, C, ldc, m0 + wm * G::kTM, n0 + wn * G::kTN, M, N, sign, flags);
}

}  // namespace dma

// One workgroup per CU (128 KiB of LDS for either tile; E = 256 also takes all 256
// accumulator registers of a lane).
template <typename T, bool A_MN, bool B_MN, int EPI, int E>
__global__ __launch_bounds__(64 * dma::kWaves) __attribute__((amdgpu_waves_per_eu(1)))
void mfma_f16_dma_kernel(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                         const uint16_t *__restrict__ B, int ldb, float *__restrict__ C,
                         int ldc, float sign, int flags) {
    __shared__ __attribute__((aligned(1024))) char lds[dma::Geo<E>::kLds];
    int tm, tn;
    grouped_tile(xcd_contiguous_id(blockIdx.x, gridDim.x), cdiv(M, E), cdiv(N, E), 4, tm, tn);
    dma::dma_tile<T, A_MN, B_MN, EPI, E>(M, N, K, A, lda, B, ldb, C, ldc, sign, flags, tm * E, tn * E,
                                         lds);
}
