// 256 x 256 interior tiles of the FP16 / BF16 GEMM fed by direct global -> LDS loads and
// multiplied with v_mfma_f32_16x16x32_{f16,bf16}.  Included by h16_gemm.hpp.
//
// Data movement ("Kernel optimisation guide", Level 3 double buffering, extended to a
// ring; the overlap of loads and arithmetic in the scheduling section of "Advanced
// CUDA features - starting from GEMM"):
//  * K is walked in steps of 32.  An m/n-contiguous operand goes through a ring of
//    kNs = 4 stages (16 KiB each), its loads of k-step t+3 issued while step t is
//    multiplied, into the stage step t-1 has released; a k-contiguous operand goes through
//    two slots of a 64-wide double step (32 KiB each), loaded every other k-step, so that
//    its loads read whole 128-byte lines (with 32-wide steps each line would be fetched
//    twice, half of it each time);
//  * a load is buffer_load_dwordx4 with the lds flag: lane l's 16 bytes land at
//    m0 + 16 l, so one instruction fills 1 KiB of LDS (8 rows of a KM operand or 2 rows
//    of an MN operand) and the lane -> source mapping chooses where each 16-byte chunk
//    goes;
//  * a KM operand's rows are 128 bytes, chunk c of row r stored in slot c ^ ((r / 2) %
//    8); an MN operand's rows are 512 bytes, chunk c of row k in slot
//    c ^ 4 (k % 4) ^ 2 ((k / 8) % 2).  With these the fragment reads (ds_read_b128 for
//    KM, ds_read_b64_tr_b16 for MN) touch distinct banks within every 16 lanes of a
//    b128 read and every 32 lanes of a b64 read, i.e. no bank conflicts, without padding
//    (which a contiguous 1 KiB load cannot skip);
//  * each wave waits for its own loads of step t+1 (vmcnt), then one barrier per
//    k-step publishes them to all four waves.
//
// Arithmetic: each wave owns 128 x 128 of C as 8 x 8 blocks of 16 x 16 (64 FP32
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

constexpr int kBM = 256, kBN = 256, kBK = 32, kNs = 4;
constexpr int kWM = 2, kWN = 2, kWaves = kWM * kWN;
constexpr int kTM = kBM / kWM, kTN = kBN / kWN, kMB = kTM / 16, kNB = kTN / 16;
constexpr int kStage = kBM * kBK * 2;        // bytes per operand per stage (both 256 x 32)
constexpr int kBOff = kNs * kStage;          // the B ring follows the A ring
constexpr int kLds = 2 * kNs * kStage;
constexpr int kI = kStage / 1024 / kWaves;   // 1 KiB loads per wave per operand per k-step
static_assert(kBM == kBN, "both operands share the ring geometry");
static_assert(kLds <= 160 * 1024, "LDS budget");
static_assert(kI == 4, "an MN operand's wave fills 8 rows, all of one (k / 8) parity");
// every ds_read immediate (slot / stage + block / row offsets) stays below 64 KiB
static_assert(2 * kStage + (kMB - 1) * 2048 < 65536, "KM read offsets");
static_assert(2 * (2 * kStage) == kNs * kStage, "both kinds of operand fill the same region");
static_assert((kNs - 1) * kStage + 4 * 512 < 65536, "MN read offsets");

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

// Loads and fragment reads of one operand of extent 256 in its 64 KiB region at byte
// offset `roff`.
//  * MN (m/n-contiguous): a ring of kNs stages of one 32-wide k-step (16 KiB, rows of
//    512 bytes).  Wave w fills rows [8 w, +8), instruction i rows 8 w + 2 i + l/32, lane
//    slot l%32 taking chunk slot ^ 4 (row % 4) ^ 2 ((row / 8) % 2), where row % 4 =
//    l/32 + 2 (i % 2) and (row / 8) % 2 = w % 2.
//  * KM (k-contiguous): two slots of one 64-wide double step (32 KiB, 256 rows of 128
//    bytes), so that every load reads whole 128-byte lines; k-step t uses half t % 2 of
//    slot (t / 2) % 2.  Wave w fills rows [64 w, +64), instruction i rows 8 i + l/8,
//    lane slot l%8 taking chunk slot ^ ((row / 2) % 8), where (row / 2) % 8 =
//    4 (i % 2) + l/16.
template <bool MN>
struct DmaOp {
    static constexpr int kSlot = 2 * kStage;         // KM slot bytes
    static constexpr int kPieces = MN ? 2 : 1;       // LDS reads per fragment
    int4v rsrc;
    uint32_t voff[2];
    lds_char *rd[MN ? 8 : 2];
    H16Frag<MN, 8> fr;

    // X: the operand; mn0: the tile's first row (KM) or column (MN); wb: the wave's first
    // row or column within the tile.
    __device__ __forceinline__ void init(const uint16_t *X, int ld, int mn0, int wave, int lane,
                                         lds_char *L, int roff, int wb) {
        if constexpr (MN) {
            rsrc = rsrc_of(X + mn0);
            const int row = 2 * kI * wave + lane / 32, slot = lane & 31;
            const int kx = 2 * (wave & 1);
            voff[0] = (uint32_t)((row * ld + 8 * (slot ^ (4 * (lane >> 5)) ^ kx)) * 2);
            voff[1] = (uint32_t)((row * ld + 8 * (slot ^ (4 * ((lane >> 5) + 2)) ^ kx)) * 2);
            // block b, piece h: lane (g = l/16, e = (l%16)/4, q = l%4) reads row 8 g + 4 h +
            // e, chunk wb/8 + 2 b + q/2, byte 8 (q%2) of it; that row's swizzle key is
            // 4 e ^ 2 (g%2)
            const int g = lane >> 4, e = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
            for (int b = 0; b < 8; ++b)
                rd[b] = lds_reg(L + roff + (8 * g + e) * 512 +
                                16 * (wb / 8 + ((2 * b + (q >> 1)) ^ (4 * e) ^ (2 * (g & 1)))) +
                                8 * (q & 1));
        } else {
            rsrc = rsrc_of(X + (size_t)mn0 * ld);
            const int row = 64 * wave + lane / 8, slot = lane & 7;
            voff[0] = (uint32_t)((row * ld + 8 * (slot ^ ((0 + lane / 16) & 7))) * 2);
            voff[1] = (uint32_t)((row * ld + 8 * (slot ^ ((4 + lane / 16) & 7))) * 2);
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
            const uint32_t dst = lds0 + roff + place * kStage + (wave * kI + i) * 1024;
            load_lds16(dst, voff[i & 1], rsrc, (uint32_t)((k0 + 2 * i) * ld * 2));
        } else {
            const uint32_t dst = lds0 + roff + place * kSlot + (wave * 8 + i) * 1024;
            load_lds16(dst, voff[i & 1], rsrc, (uint32_t)((8 * i * ld + k0) * 2));
        }
    }
    // Piece h of block b of k-step u (u = t % kNs, so the MN stage is u, the KM slot
    // u / 2 and the KM half u % 2) into fragment slot `fslot`.
    __device__ __forceinline__ void read(int u, int fslot, int b, int h) {
        if constexpr (MN) {
            fr.f[fslot][b][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_shortx4 *)(rd[b] + u * kStage + 4 * h * 512));
        } else {
            fr.f[fslot][b] = *(const lds_u16x8 *)(rd[u % 2] + (u / 2) * kSlot + b * 2048);
        }
    }
};

// The order in which a k-step's fragment pieces are read: A block 0, then the B blocks,
// then the other A blocks, i.e. in the order the MFMAs (A block outer, B block inner,
// odd rows walking the B blocks backwards) first use them.
template <bool A_MN, bool B_MN>
struct PieceOrder {
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

// Empty volatile statements that take every accumulator quad in and out of an AGPR:
// code that defines the accumulators stays before them and code that reads them after,
// so they order the accumulators' writes and reads with respect to the explicit wait
// states around the inline-assembly MFMAs.
__device__ __forceinline__ void pin_acc(floatx4 (&acc)[kMB][kNB]) {
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// The FP32 accumulator quads of one wave, stored to C: quad (i, j) holds rows
// row0 + 16 i + 4 (l/16) + r, column col0 + 16 j + l%16.  For each row the eight quads of
// a block row go out back to back, so every 128-byte line of C is written whole by two
// consecutive stores.  The stores are ordinary (cached) ones: each instruction writes
// half lines, which the L2 merges; as non-temporal stores the same pattern took 40 %
// longer (64 MiB from 256 workgroups: 15.8 against 11.2 us).
template <int EPI, typename T>
__device__ __forceinline__ void store_tile(floatx4 (&acc)[kMB][kNB], float *__restrict__ C, int ldc,
                                           int row0, int col0, float sign, int flags) {
    const int lane = threadIdx.x & 63;
    const int rl = row0 + 4 * (lane >> 4);
    if constexpr (EPI == 0) {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    C[(size_t)(rl + 16 * i + r) * ldc + col0 + 16 * j + (lane & 15)] = acc[i][j][r];
    } else if constexpr (EPI == 1) {
        const bool use_old = flags & 1;
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                store_quad16_acc(acc[i][j], C, ldc, rl + 16 * i, col0 + 16 * j + (lane & 15), sign,
                                 use_old);
    } else {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kNB; j += 2)
                store_pair16_c16<T>(acc[i][j], acc[i][j + 1], (uint16_t *)C, ldc, rl + 16 * i,
                                    col0 + 16 * j, sign, flags);
    }
}

template <typename T, bool A_MN, bool B_MN, int EPI>
__device__ __forceinline__ void dma_tile(int K, const uint16_t *__restrict__ A, int lda,
                                         const uint16_t *__restrict__ B, int ldb,
                                         float *__restrict__ C, int ldc, float sign,
                                         int flags, int m0, int n0, char *lds_raw) {
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int wm = wave / kWN, wn = wave % kWN;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char *)lds_raw;
    lds_char *const L = (lds_char *)lds_raw;

    using OA = DmaOp<A_MN>;
    using OB = DmaOp<B_MN>;
    using PO = PieceOrder<A_MN, B_MN>;
    OA oa;
    OB ob;
    oa.init(A, lda, m0, wave, lane, L, 0, wm * kTM);
    ob.init(B, ldb, n0, wave, lane, L, kBOff, wn * kTN);
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

    // One k-step t = kt + u (u = t % 4 is a compile-time constant): kMf MFMAs on the
    // fragments in slot u % 2.  The step's loads (MN: k-step t+3 into stage (u+3) % 4; on
    // even steps KM: double step t/2 + 1 into slot (u/2 + 1) % 2) are spread over the
    // first kLoadHi MFMAs; after kBarrier MFMAs the wave waits until the loads step t+1
    // needs are done, then the barrier publishes them and the fragments of t+1 are read
    // into the other slot under the remaining MFMAs, in the order of their first use.
    // The wait counts: on an even step the 2 nMN + nKM youngest loads may stay in flight
    // (the MN loads of steps t+2 and t+3 and this step's KM loads; the KM loads of two
    // steps ago are older but already complete), on an odd step nMN (this step's MN
    // loads) when there are KM operands, else 2 nMN.  No branches: near the end the loads
    // repeat the last k-step or double step into free stages or slots.
    constexpr int kMf = kMB * kNB;
    constexpr int kBarrier = 40;
    constexpr int kLoadHi = 32;
    static_assert(kLoadHi <= kBarrier, "the step's loads precede its wait");
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
        constexpr int kWait = even ? 2 * nMN + nKM : (nKM ? nMN : 2 * nMN);
        const int t = kt + u;
        const int k_mn = min(t + kNs - 1, nk - 1) * kBK;
        const int k_km = min(t / 2 + 1, nk / 2 - 1) * 2 * kBK;
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
                    else issue_km((u / 2 + 1) % 2, k_km, w - nMN);
                }
            }
            if (qs == kBarrier - 1) {
                wait_vmcnt<kWait>();
                __syncthreads();
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // KM double step 0 into slot 0, MN k-steps 0 .. kNs-2 into stages 0 .. kNs-2; wait for
    // step 0's data (the MN loads of steps 1 and 2 may stay in flight), read its fragments
#pragma unroll
    for (int w = 0; w < nKM; ++w) issue_km(0, 0, w);
#pragma unroll
    for (int p = 0; p < kNs - 1; ++p)
#pragma unroll
        for (int w = 0; w < nMN; ++w) issue_mn(p, min(p, nk - 1) * kBK, w);
    wait_vmcnt<2 * nMN>();
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
    using U0 = std::integral_constant<int, 0>;
    using U1 = std::integral_constant<int, 1>;
    using U2 = std::integral_constant<int, 2>;
    using U3 = std::integral_constant<int, 3>;
    for (int kt = 0; kt < nk; kt += kNs) {
        kstep(kt, U0{});
        kstep(kt, U1{});
        kstep(kt, U2{});
        kstep(kt, U3{});
    }
    // nothing may still write this workgroup's LDS when it exits
    wait_vmcnt<0>();
    pin_acc(acc);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    pin_acc(acc);
    store_tile<EPI, T>(acc, C, ldc, m0 + wm * kTM, n0 + wn * kTN, sign, flags);
}

}  // namespace dma

template <typename T, bool A_MN, bool B_MN, int EPI>
__global__ __launch_bounds__(64 * dma::kWaves) __attribute__((amdgpu_waves_per_eu(1)))
void mfma_f16_dma_kernel(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                         const uint16_t *__restrict__ B, int ldb, float *__restrict__ C,
                         int ldc, float sign, int flags) {
    __shared__ __attribute__((aligned(1024))) char lds[dma::kLds];
    int tm, tn;
    grouped_tile(xcd_contiguous_id(blockIdx.x, gridDim.x), M / dma::kBM, N / dma::kBN, 4, tm, tn);
    dma::dma_tile<T, A_MN, B_MN, EPI>(K, A, lda, B, ldb, C, ldc, sign, flags, tm * dma::kBM,
                                      tn * dma::kBN, lds);
}
