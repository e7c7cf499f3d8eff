// 256 x 256 and 128 x 128 interior tiles of the FP16 / BF16 GEMM fed by direct global
// -> LDS loads and multiplied with v_mfma_f32_16x16x32_{f16,bf16}.  Included by
// h16_gemm.hpp.
//
// Data movement ("Kernel optimisation guide", Level 3 double buffering, extended to a
// ring; the overlap of loads and arithmetic in the scheduling section of "Advanced
// CUDA features - starting from GEMM"):
//  * K is walked in steps of 32.  An m/n-contiguous operand goes through a ring of kNs
//    stages (4 of 16 KiB for 256-wide tiles, 8 of 8 KiB for 128-wide ones, 8 of 4 KiB for
//    64-wide ones; 4 for 128- and 64-wide tiles two per CU or with K below 256), its loads of
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
//    c ^ 4 (k % 4) ^ 2 ((k / 8) % 2) (E = 192 or 64: the keys in DmaOp below).  With
//    these the fragment reads (ds_read_b128 for
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
//
// The tile routine is written over a general geometry (an EM x EN tile, WM x WN compute
// waves, NS ring stages, PW producer waves) so that other schedules of the same data
// movement can be built and measured against the dispatched one: the dispatched kernels
// are EM = EN = 256, 128 or 64 and EM x EN = 192 x 256 or 256 x 192, on 2 x 2 waves that
// all load; mfma_f16_dma_sched_kernel
// instantiates the others (wave specialisation with producer waves, eight waves, 256 x
// 128 tiles).
#pragma once

namespace dma {

constexpr int kBK = 32;

// Ring stages (32-wide k-steps) of a tile whose operands have extent E, one workgroup per
// CU: 4 of 16 KiB per operand for 256-wide tiles, 8 of 8 KiB for 128-wide ones (8 of 4 KiB
// for 64-wide ones).  A 128-wide tile's k-step is a quarter of a 256-wide one's arithmetic
// (16 MFMAs per wave, ~130 ns), so its ring is twice as deep to keep the loads as far ahead
// in time.  (With two 128-wide workgroups per CU each k-step takes twice as long, and 4
// stages, 64 KiB, do.)
constexpr int ring_stages(int E) { return E == 256 ? 4 : 8; }

// Geometry of an EM x EN tile: WM x WN compute waves, each owning (EM / WM) x (EN / WN) of
// C; NS ring stages; PW producer waves.  With PW = 0 every compute wave issues its share
// of the loads beside its MFMAs (the dispatched kernels); with PW > 0 only the PW
// producer waves load and the compute waves only read fragments and multiply.
template <int EM, int EN, int WM, int WN, int NS, int PW>
struct Geo {
    static constexpr int kCW = WM * WN;                   // compute waves
    static constexpr int kLW = PW > 0 ? PW : kCW;         // waves that issue the loads
    static constexpr int kWaves = kCW + PW;
    static constexpr int kNs = NS;
    static constexpr int kTM = EM / WM, kTN = EN / WN;    // wave tile
    static constexpr int kMB = kTM / 16, kNB = kTN / 16;  // accumulator quads per wave
    static constexpr int kStageA = EM * kBK * 2, kStageB = EN * kBK * 2;  // bytes per stage
    static constexpr int kBOff = NS * kStageA;            // the B ring follows the A ring
    static constexpr int kLds = NS * (kStageA + kStageB);
    // MFMAs per k-step, the step's wait and barrier after kBarrier of them, its loads
    // spread evenly over every MFMA before the wait (bunching them into fewer MFMAs
    // measured slower: 256 x 256, loads over 16 / 24 / 32 / 40 of 64 MFMAs at FP16 4096^3:
    // 104.3 / 102.3 / 101.5 / 100.7 us; over 40 instead of 32, BF16 8192^3 2.5 % faster)
    static constexpr int kMf = kMB * kNB;
    static constexpr int kBarrier = kMf * 5 / 8;
    static constexpr int kLoadHi = kBarrier;
    static_assert(kTM % 16 == 0 && kTN % 16 == 0, "wave tiles are whole 16 x 16 quads");
    static_assert(NS % 2 == 0 && NS >= 4, "a KM operand's double steps take two stages each");
    static_assert(kLds <= 160 * 1024, "LDS budget");
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

// The lane index from the exec mask, computed where it is used (volatile assembly, so no
// register holds it across the main loop: the 256-wide tile's loop uses all 256 VGPRs).
__device__ __forceinline__ int lane_here() {
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    return lane;
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
// `roff` (NS x E x 32 x 2 bytes: 64 KiB for E = 256 and 4 stages), LW waves sharing its
// loads, NB accumulator quads along it per compute wave.
//  * MN (m/n-contiguous): a ring of NS stages of one 32-wide k-step (E x 32 halves,
//    rows of 2 E bytes).  Loading wave w fills rows [R w, +R) with R = 32 / LW (8 or 4):
//    instruction i rows R w + P i + l / (64 / P) with P = 1024 / (2 E) rows per
//    instruction, lane slot l % (64 / P) taking chunk slot ^ 4 (row % 4) ^ 2 ((row / 8)
//    % 2), where (row / 8) % 2 = (R w / 8) % 2 and row % 4 = (P i + l / (64 / P)) % 4,
//    which depends on i only through its parity.
//  * KM (k-contiguous): NS / 2 slots of one 64-wide double step (E rows of 128 bytes),
//    so that every load reads whole 128-byte lines; k-step t uses half t % 2 of slot
//    (t / 2) % (NS / 2).  Loading wave w fills rows [R w, +R) with R = E / LW (a multiple
//    of 16), instruction i rows R w + 8 i + l/8, lane slot l%8 taking chunk slot ^ ((row
//    / 2) % 8), where (row / 2) % 8 = 4 (i % 2) + l/16.
//  * MN with E = 192 or 64 (kLin): rows of 384 or 128 bytes, 24 or 8 chunks, which the XOR
//    keys above (up to 14) would carry past the row's end.  Chunk c of row k is stored in
//    slot c ^ 4 ((k % 4) / 2) ^ 2 ((k / 8) % 2): keys below 8 keep every chunk within its
//    aligned group of 8, and since consecutive rows start 128 bytes apart modulo the 256
//    bytes of the 64 banks, the rows of odd k cover the bank half that the even ones
//    leave, so the eight rows a half-wave's b64 read touches (k % 4, (k / 8) % 2) still
//    land on distinct banks.  A stage (32 rows: 12 or 4 KiB) is filled as whole 1 KiB
//    instructions in order, wave w issuing instructions kI w .. kI w + kI - 1 (rows 8 w ..
//    8 w + 7; kI = 3 or 1): lane l of instruction j fills stage chunk 64 j + l, i.e. row
//    (64 j + l) / (E / 8), slot (64 j + l) % (E / 8), each instruction with its own
//    per-lane offset.
template <bool MN, int E, int LW, int NS, int NB>
struct DmaOp {
    static constexpr bool kLin = MN && (E == 64 || E == 192);
    static constexpr int kStage = E * kBK * 2;       // MN stage bytes
    static constexpr int kSlot = 2 * kStage;         // KM slot bytes
    static constexpr int kRowB = 2 * E;              // MN: bytes per LDS row (one k)
    static constexpr int kCpr = E / 8;               // MN: 16-byte chunks per row
    static constexpr int kRpi = 1024 / kRowB;        // MN: rows one load instruction fills
    static constexpr int kRows = MN ? kBK / LW : E / LW;  // rows a loading wave fills
    // load instructions per loading wave: per k-step (MN) or per double step (KM)
    static constexpr int kI = kLin ? kRows * kCpr / 64 : MN ? kRows / kRpi : kRows / 8;
    static_assert(kI >= 1, "every loading wave issues a whole instruction");
    // the MN swizzle XORs chunk slots with up to 14: a row needs at least 16 chunks
    static_assert(!MN || E == 64 || E == 128 || E == 192 || E == 256, "an MN operand's rows hold 8, 16, 24 or 32 chunks");
    static_assert(!MN || kLin || (kRows * LW == kBK && kI * kRpi == kRows && 8 % kRows == 0),
                  "an MN operand's loading wave fills rows of one (k / 8) parity");
    static_assert(!kLin || (kRows * LW == kBK && kI * 64 == kRows * kCpr),
                  "an 8- or 24-chunk operand's loading wave fills whole rows with whole instructions");
    static_assert(MN || (kRows * LW == E && kRows % 16 == 0), "KM rows per loading wave");
    // every ds_read immediate (slot / stage + block / row offsets) stays below 64 KiB
    static_assert(MN || (NS / 2 - 1) * kSlot + (NB - 1) * 2048 < 65536, "KM read offsets");
    static_assert(!MN || (NS - 1) * kStage + 4 * kRowB < 65536, "MN read offsets");
    int4v rsrc;
    // per lane: MN by instruction parity, KM and kLin by instruction
    uint32_t voff[MN && !kLin ? 2 : kI];
    // kLin: the swizzle key of row k
    __device__ __forceinline__ static int key24(int k) { return 4 * ((k & 3) >> 1) ^ 2 * ((k >> 3) & 1); }
    lds_char *rd[MN ? NB : 2];
    H16Frag<MN, NB> fr;

    // Loading side.  X: the operand, whose rows (KM) or columns (MN) number ext (a
    // multiple of 8 for MN); mn0: the tile's first row (KM) or column (MN); lw: the
    // loading wave's index.  In a ragged tile a lane whose source row (KM) or 16-byte
    // column chunk (MN) lies beyond ext loads the last one inside instead, so every load
    // stays within the operand; what it puts in LDS only reaches outputs beyond row M or
    // column N, which are never stored.
    __device__ __forceinline__ void init_load(const uint16_t *X, int ld, int ext, int mn0, int lw,
                                              int lane) {
        if constexpr (kLin) {
            rsrc = rsrc_of(X + mn0);
            const int last = (ext - mn0) / 8 - 1;
#pragma unroll
            for (int i = 0; i < kI; ++i) {
                const int p = 64 * (kI * lw + i) + lane, row = p / kCpr, slot = p % kCpr;
                voff[i] = (uint32_t)((row * ld + 8 * min(slot ^ key24(row), last)) * 2);
            }
        } else if constexpr (MN) {
            constexpr int lpr = 64 / kRpi;           // lanes per row of one load
            rsrc = rsrc_of(X + mn0);
            const int rl = lane / lpr, row = kRows * lw + rl, slot = lane % lpr;
            const int kx = 2 * ((kRows * lw / 8) & 1), last = (ext - mn0) / 8 - 1;
#pragma unroll
            for (int p = 0; p < 2; ++p)
                voff[p] = (uint32_t)((row * ld + 8 * min(slot ^ (4 * ((kRpi * p + rl) % 4)) ^ kx, last)) * 2);
        } else {
            rsrc = rsrc_of(X + (size_t)mn0 * ld);
            const int row = kRows * lw + lane / 8, slot = lane & 7, last = ext - mn0 - 1;
#pragma unroll
            for (int i = 0; i < kI; ++i)
                voff[i] = (uint32_t)((min(row + 8 * i, last) * ld +
                                      8 * (slot ^ ((4 * (i % 2) + lane / 16) & 7))) * 2);
        }
    }
    // Compute side: the fragment read addresses of the wave whose first row or column
    // within the tile is wb (a multiple of 16).
    __device__ __forceinline__ void init_read(int lane, lds_char *L, int roff, int wb) {
        if constexpr (MN) {
            // block b, piece h: lane (g = l/16, e = (l%16)/4, q = l%4) reads row 8 g + 4 h +
            // e, chunk wb/8 + 2 b + q/2, byte 8 (q%2) of it; that row's swizzle key is
            // 4 e ^ 2 (g%2) (kLin: 4 (e/2) ^ 2 (g%2)), the same for both pieces
            const int g = lane >> 4, e = (lane & 15) >> 2, q = lane & 3;
            const int key = kLin ? key24(8 * g + e) : (4 * e) ^ (2 * (g & 1));
#pragma unroll
            for (int b = 0; b < NB; ++b)
                rd[b] = lds_reg(L + roff + (8 * g + e) * kRowB +
                                16 * ((wb / 8 + 2 * b + (q >> 1)) ^ key) + 8 * (q & 1));
        } else {
            // block b, half h of the slot: row wb + 16 b + l%16, chunk 4 h + l/16, whose
            // swizzle key ((l%16) / 2) % 8 does not depend on b
            const int l16 = lane & 15, lq = lane >> 4;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                rd[h] = lds_reg(L + roff + (wb + l16) * 128 + 16 * ((4 * h + lq) ^ (l16 >> 1)));
        }
    }
    // Load instruction i of one issue: MN: k-step at k0 into stage `place`; KM: the
    // double step at k0 into slot `place`.  KR (K not a whole number of ring trips): a
    // lane whose chunk lies at k >= K (K a multiple of 8, so a chunk is wholly inside or
    // outside) takes an offset beyond the buffer's range instead, and the load writes
    // zeros to its 16 bytes of LDS, so the k-steps past K add nothing.
    // The k of lane `lane`'s 16-byte chunk in load i of loading wave lw, relative to the
    // issue's k0: MN its row, KM its chunk's first column (recomputed where needed rather
    // than held in registers across the loop).
    __device__ __forceinline__ static int kpos(int i, int lw, int lane) {
        if constexpr (kLin) return (64 * (kI * lw + i) + lane) / kCpr;
        else if constexpr (MN) return kRows * lw + kRpi * i + lane / (64 / kRpi);
        else return 8 * ((lane & 7) ^ ((4 * (i % 2) + lane / 16) & 7));
    }
    // One past the largest k that load i of loading wave lw reads, relative to k0.
    __device__ __forceinline__ static int kend(int i, int lw) {
        if constexpr (kLin) return (64 * (kI * lw + i) + 63) / kCpr + 1;
        else if constexpr (MN) return kRows * lw + kRpi * (i + 1);
        else return 2 * kBK;
    }
    // KR: the offset register of a chunk at k >= K is set past the buffer's range in place.
    // Every later load through that register reads a chunk at a larger or equal k (the
    // loads are issued in k order, and the clamped repeats at the end do not go back), so
    // it stays out of range, and no other register is needed.  Only a load that reaches K
    // selects per lane; the test is uniform over the wave (a scalar branch), so the loads
    // wholly inside K cost nothing more.
    template <bool KR>
    __device__ __forceinline__ uint32_t off(int k0, int i, int lw, int K) {
        constexpr uint32_t kOut = 0x80000000u;   // beyond num_records (2^31 - 1)
        uint32_t &v = voff[MN && !kLin ? (i & 1) : i];
        if constexpr (KR) {
            if (k0 + kend(i, lw) > K) v = k0 + kpos(i, lw, lane_here()) < K ? v : kOut;
        }
        return v;
    }
    __device__ __forceinline__ void issue_at(uint32_t lds0, int roff, int lw, int ld, int place,
                                             int k0, int i, uint32_t v) {
        if constexpr (MN) {
            const uint32_t dst = lds0 + roff + place * kStage + (lw * kI + i) * 1024;
            // kLin: the row within the stage is in the lane's offset
            load_lds16(dst, v, rsrc, (uint32_t)((k0 + (kLin ? 0 : kRpi * i)) * ld * 2));
        } else {
            const uint32_t dst = lds0 + roff + place * kSlot + (lw * kI + i) * 1024;
            load_lds16(dst, v, rsrc, (uint32_t)(k0 * 2));
        }
    }
    template <bool KR>
    __device__ __forceinline__ void issue(uint32_t lds0, int roff, int lw, int ld, int place,
                                          int k0, int i, int K) {
        issue_at(lds0, roff, lw, ld, place, k0, i, off<KR>(k0, i, lw, K));
    }
    // Piece h of block b of k-step u (u = t % NS, so the MN stage is u, the KM slot
    // u / 2 and the KM half u % 2) into fragment slot `fslot`.
    __device__ __forceinline__ void read(int u, int fslot, int b, int h) {
        if constexpr (MN) {
            fr.f[fslot][b][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_shortx4 *)(rd[b] + u * kStage + 4 * h * kRowB));
        } else {
            fr.f[fslot][b] = *(const lds_u16x8 *)(rd[u % 2] + (u / 2) * kSlot + b * 2048);
        }
    }
};

// The order in which a k-step's fragment pieces are read: A block 0, then the B blocks,
// then the other A blocks, i.e. in the order the MFMAs (A block outer, B block inner,
// odd rows walking the B blocks backwards) first use them.
template <bool A_MN, bool B_MN, int kMB, int kNB>
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

// kstep(kt, integral_constant<u>, b) for u = 0 .. kNs-1 in order.
template <typename F, typename B, int... U>
__device__ __forceinline__ void for_steps(F &kstep, int kt, std::integer_sequence<int, U...>, B b) {
    (kstep(kt, std::integral_constant<int, U>{}, b), ...);
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
// longer (64 MiB from 256 workgroups: 15.8 against 11.2 us).  Accumulating into C (FP32 in
// every tile; 16-bit in 4-byte words in interior tiles), the old values of a whole row of
// quads are loaded before any of them is used, and the next row's loads are issued before
// this row's stores, so the loads wait on memory kMB times rather than once per quad or pair
// (the loop's fragment registers are free by then).
template <int EPI, typename T, bool EDGE, int kMB, int kNB>
__device__ __forceinline__ void store_tile(floatx4 (&acc)[kMB][kNB], float *__restrict__ C, int ldc,
                                           int row0, int col0, int M, int N, float sign, int flags) {
    const int lane = lane_here();
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
        if (!use_old) {
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    store_quad16_acc<EDGE>(acc[i][j], C, ldc, rl + 16 * i, col0 + 16 * j + (lane & 15),
                                           M, N, sign, false);
            return;
        }
        // this lane's element of quad row i, quad j, row r: Cl[(16 i + r) ldc + 16 j]
        float *const Cl = C + (size_t)rl * ldc + col0 + (lane & 15);
        const int cl = col0 + (lane & 15);
        float old[2][kNB][4];
        const auto load_row = [&](int i, float (&o)[kNB][4]) {
            const float *Ci = Cl + (size_t)(16 * i) * ldc;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < kNB; ++j) {
                    const bool ok = !EDGE || (rl + 16 * i + r < M && cl + 16 * j < N);
                    // an element outside M x N reads C's first one instead, so the load is
                    // in bounds even where the compiler issues it anyway
                    const float *p = Ci + (size_t)r * ldc + 16 * j;
                    o[j][r] = ok ? *(ok ? p : C) : 0.f;
                }
        };
        __builtin_amdgcn_sched_barrier(0);
        load_row(0, old[0]);
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            if (i + 1 < kMB) load_row(i + 1, old[(i + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            float *Ci = Cl + (size_t)(16 * i) * ldc;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < kNB; ++j) {
                    float a;
                    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a) : "a"(acc[i][j][r]));
                    if (!EDGE || (rl + 16 * i + r < M && cl + 16 * j < N))
                        Ci[(size_t)r * ldc + 16 * j] = sign * a + old[i & 1][j][r];
                }
        }
        __builtin_amdgcn_sched_barrier(0);
    } else {
        if (EDGE || (flags & 3) != 3) {
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int j = 0; j < kNB; j += 2)
                    store_pair16_c16<EDGE, T>(acc[i][j], acc[i][j + 1], (uint16_t *)C, ldc, rl + 16 * i,
                                              col0 + 16 * j, M, N, sign, flags, lane);
            return;
        }
        // interior tiles accumulating with 4-byte words (store_pair16_c16's paired mode): the
        // old words of a row of quad pairs loaded a row ahead as above
        constexpr int kP = kNB / 2;
        const int odd = lane & 1;
        const int cw = col0 + (lane & 14) + 16 * odd;  // first column of this lane's word in pair 0
        uint16_t *const Cl = (uint16_t *)C + (size_t)rl * ldc + cw;
        uint32_t oldw[2][kP][4];
        const auto load_row = [&](int i, uint32_t (&o)[kP][4]) {
            const uint16_t *Ci = Cl + (size_t)(16 * i) * ldc;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int p = 0; p < kP; ++p) o[p][r] = *(const uint32_t *)(Ci + (size_t)r * ldc + 32 * p);
        };
        __builtin_amdgcn_sched_barrier(0);
        load_row(0, oldw[0]);
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            if (i + 1 < kMB) load_row(i + 1, oldw[(i + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            uint16_t *Ci = Cl + (size_t)(16 * i) * ldc;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int p = 0; p < kP; ++p) {
                    float a0, a1;
                    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a0) : "a"(acc[i][2 * p][r]));
                    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a1) : "a"(acc[i][2 * p + 1][r]));
                    *(uint32_t *)(Ci + (size_t)r * ldc + 32 * p) =
                        pair16_word<T>(a0, a1, odd, sign, oldw[i & 1][p][r], true);
                }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// WHOLE: the caller guarantees that the tile lies inside M x N (no guarded stores).
// KR: K is not a whole number of ring trips (K a multiple of 8): the loop runs to the next
// whole trip, every chunk at k >= K loads as zeros (DmaOp::issue), and the k-steps of the
// last trip that lie wholly at k >= K are skipped.
template <typename T, bool A_MN, bool B_MN, int EPI, int EM, int EN, int WM, int WN, int NS, int PW,
          bool WHOLE = false, bool KR = false>
__device__ __forceinline__ void dma_tile(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                                         const uint16_t *__restrict__ B, int ldb,
                                         float *__restrict__ C, int ldc, float sign,
                                         int flags, int m0, int n0, char *lds_raw) {
    // the producer waves run every k-step's barrier; they do not skip the tail's steps
    static_assert(!(KR && PW > 0), "K past whole ring trips needs the compute waves to load");
    using G = Geo<EM, EN, WM, WN, NS, PW>;
    constexpr int kMB = G::kMB, kNB = G::kNB, kBOff = G::kBOff, kNs = NS, kLW = G::kLW;
    using OA = DmaOp<A_MN, EM, kLW, NS, kMB>;
    using OB = DmaOp<B_MN, EN, kLW, NS, kNB>;
    using PO = PieceOrder<A_MN, B_MN, kMB, kNB>;
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char *)lds_raw;
    lds_char *const L = (lds_char *)lds_raw;
    OA oa;
    OB ob;
    // Loads per loading wave: nMN every k-step (the MN operands' next stage), nKM every
    // other k-step (the KM operands' next double step), MN loads first.
    constexpr int nMN = (A_MN ? OA::kI : 0) + (B_MN ? OB::kI : 0);
    constexpr int nKM = (A_MN ? 0 : OA::kI) + (B_MN ? 0 : OB::kI);
    // issue w of an MN batch (k-step at k0 into stage st) / of a KM batch (double step at
    // k0 into slot sl), by loading wave lw
    // (kr_c: whether this load may lie past K and selects its lanes' offsets)
    auto issue_mn = [&](int lw, int st, int k0, int w, auto kr_c) {
        constexpr bool kKR = decltype(kr_c)::value;
        if constexpr (A_MN) {
            if (w < OA::kI) { oa.template issue<kKR>(lds0, 0, lw, lda, st, k0, w, K); return; }
            w -= OA::kI;
        }
        if constexpr (B_MN) ob.template issue<kKR>(lds0, kBOff, lw, ldb, st, k0, w, K);
    };
    auto issue_km = [&](int lw, int sl, int k0, int w, auto kr_c) {
        constexpr bool kKR = decltype(kr_c)::value;
        if constexpr (!A_MN) {
            if (w < OA::kI) { oa.template issue<kKR>(lds0, 0, lw, lda, sl, k0, w, K); return; }
            w -= OA::kI;
        }
        if constexpr (!B_MN) ob.template issue<kKR>(lds0, kBOff, lw, ldb, sl, k0, w, K);
    };
    using KRc = std::integral_constant<bool, KR>;
    // k-steps: K / 32, or with KR the k-steps up to the next whole ring trip
    const int nk = KR ? cdiv(K, kBK * kNs) * kNs : K / kBK;
    // The wait before the barrier of k-step u (u = t % kNs): loads are issued in step
    // order (a step's MN loads, then its KM loads), the prologue's included, so the wait
    // counts are the loads of the steps after the one that issued what step t+1 needs: on
    // an even step t both of its operands' loads came from step t - kNs + 2, so the loads
    // of the kNs - 2 steps after it may stay in flight; on an odd step its KM loads came
    // from step t - kNs + 3 (those of kNs - 3 later steps may stay), its MN loads alone
    // from t - kNs + 2.
    auto wait_before_barrier = [](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr bool even = u % 2 == 0;
        constexpr int kWait = even ? (kNs - 2) * nMN + (kNs - 2) / 2 * nKM
                                   : (nKM ? (kNs - 3) * nMN + (kNs - 4) / 2 * nKM : (kNs - 2) * nMN);
        static_assert(kWait < 64, "vmcnt range");
        wait_vmcnt<kWait>();
    };
    // Prologue, in the order the steps before step 0 would have issued it: KM double step
    // 0, then MN k-steps 0 .. kNs-2 into stages 0 .. kNs-2, KM double step d after MN
    // k-step 2d + 1 (d = 1 .. kNs/2 - 2); then wait for step 0's data (everything after
    // MN k-step 0 may stay in flight).
    auto prologue_loads = [&](int lw) {
#pragma unroll
        for (int w = 0; w < nKM; ++w) issue_km(lw, 0, 0, w, KRc{});
#pragma unroll
        for (int p = 0; p < kNs - 1; ++p) {
#pragma unroll
            for (int w = 0; w < nMN; ++w) issue_mn(lw, p, min(p, nk - 1) * kBK, w, KRc{});
            if (p % 2 == 1 && p >= 3) {
#pragma unroll
                for (int w = 0; w < nKM; ++w)
                    issue_km(lw, (p - 1) / 2, min((p - 1) / 2, nk / 2 - 1) * 2 * kBK, w, KRc{});
            }
        }
        wait_vmcnt<(kNs - 2) * nMN + (kNs / 2 - 2) * nKM>();
    };
    // The loads of k-step t = kt + u: MN: k-step t + kNs - 1 into stage (u - 1) % kNs; on
    // even steps KM: double step t/2 + kNs/2 - 1 into the slot of double step t/2 - 1.  No
    // branches: near the end the loads repeat the last k-step or double step into free
    // stages or slots.
    auto k_mn_of = [&](int t) { return min(t + kNs - 1, nk - 1) * kBK; };
    auto k_km_of = [&](int t) { return min(t / 2 + kNs / 2 - 1, nk / 2 - 1) * 2 * kBK; };
    auto step_load = [&](int lw, int u, int w, int k_mn, int k_km, auto kr_c) {
        if (w < nMN) issue_mn(lw, (u + kNs - 1) % kNs, k_mn, w, kr_c);
        else issue_km(lw, (u / 2 + kNs / 2 - 1) % (kNs / 2), k_km, w - nMN, kr_c);
    };

    if constexpr (PW > 0) {
        // Producer waves: every load of the tile, one barrier per k-step (the compute
        // waves' barrier), nothing else.
        if (wave >= G::kCW) {
            const int lw = wave - G::kCW;
            oa.init_load(A, lda, M, m0, lw, lane);
            ob.init_load(B, ldb, N, n0, lw, lane);
            prologue_loads(lw);
            __syncthreads();
            auto pstep = [&](int kt, auto u_c, auto) {
                constexpr int u = decltype(u_c)::value;
                constexpr int nLd = nMN + (u % 2 == 0 ? nKM : 0);
                const int k_mn = k_mn_of(kt + u), k_km = k_km_of(kt + u);
#pragma unroll
                for (int w = 0; w < nLd; ++w) step_load(lw, u, w, k_mn, k_km, KRc{});
                wait_before_barrier(u_c);
                __syncthreads();
            };
            for (int kt = 0; kt < nk; kt += kNs)
                for_steps(pstep, kt, std::make_integer_sequence<int, kNs>{}, 0);
            // nothing may still write this workgroup's LDS when it exits
            wait_vmcnt<0>();
            return;
        }
    }
    const int wm = wave / WN, wn = wave % WN;
    if constexpr (PW == 0) {
        oa.init_load(A, lda, M, m0, wave, lane);
        ob.init_load(B, ldb, N, n0, wave, lane);
    }
    oa.init_read(lane, L, 0, wm * G::kTM);
    ob.init_read(lane, L, kBOff, wn * G::kTN);
    constexpr int kR = PO::kR;
    auto read_piece = [&](int u, int fslot, int p) {
        if (PO::op(p) == 0) oa.read(u, fslot, PO::blk(p), PO::half(p));
        else ob.read(u, fslot, PO::blk(p), PO::half(p));
    };

    floatx4 acc[kMB][kNB];

    // One k-step t = kt + u (u = t % kNs is a compile-time constant): kMf MFMAs on the
    // fragments in slot u % 2.  The step's loads (when the compute waves issue them) are
    // spread over the first kLoadHi MFMAs; after kBarrier MFMAs the wave waits until the
    // loads step t+1 needs are done, then the barrier publishes them and the fragments of
    // t+1 are read into the other slot under the remaining MFMAs, in the order of their
    // first use.
    constexpr int kMf = G::kMf;
    auto ev_begin = [](int qs, int n, int lo, int hi) {
        if (qs <= lo) return 0;
        if (qs >= hi) return n;
        return ((qs - lo) * n + (hi - lo) - 1) / (hi - lo);
    };
    auto kstep_impl = [&](int kt, auto u_c, auto b_c, auto kr_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int kBarrier = decltype(b_c)::value;
        constexpr int kLoadHi = kBarrier < G::kLoadHi ? kBarrier : G::kLoadHi;
        static_assert(kBarrier >= 1 && kBarrier < kMf, "barrier position");
        constexpr int u1 = (u + 1) % kNs;
        constexpr int f = u % 2;
        constexpr int nLd = PW > 0 ? 0 : nMN + (u % 2 == 0 ? nKM : 0);
        const int t = kt + u;
        const int k_mn = k_mn_of(t), k_km = k_km_of(t);
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
            if constexpr (nLd > 0) {
                const int lo = ev_begin(qs, nLd, 0, kLoadHi);
                const int hi = ev_begin(qs + 1, nLd, 0, kLoadHi);
#pragma unroll
                for (int w = lo; w < hi; ++w) step_load(wave, u, w, k_mn, k_km, kr_c);
            }
            if (qs == kBarrier - 1) {
                if constexpr (PW == 0) wait_before_barrier(u_c);
                __syncthreads();
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // the k-steps whose loads may lie past K (issued in the last two ring trips) take the
    // zero-filling offsets; the others the plain ones
    auto kstep = [&](int kt, auto u_c, auto b_c) { kstep_impl(kt, u_c, b_c, std::false_type{}); };
    auto kstep_kr = [&](int kt, auto u_c, auto b_c) { kstep_impl(kt, u_c, b_c, std::true_type{}); };
    // KR, last trip: a k-step that lies wholly at k >= K would multiply zeros, so it is
    // skipped whole, loads, wait and barrier included.  The test is uniform over the
    // workgroup, so every wave skips the same steps; the loads the skipped steps would
    // have waited for read nothing inside K, and the wait after the loop drains them.
    // The last trip's first step always holds some k < K (nk - kNs < cdiv(K, 32)).
    const int nk_live = cdiv(K, kBK);
    auto kstep_tail = [&](int kt, auto u_c, auto b_c) {
        constexpr int u = decltype(u_c)::value;
        if (u == 0 || __builtin_expect(kt + u < nk_live, 1)) kstep_impl(kt, u_c, b_c, std::true_type{});
    };

    if constexpr (PW == 0) prologue_loads(wave);
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
    if constexpr (KR) {
        // nk is at least two trips; the loads of every step before the last trip read
        // whole chunks inside K, so only the last two trips select offsets
        int kt = 0;
        for (; kt < nk - 2 * kNs; kt += kNs)
            for_steps(kstep, kt, std::make_integer_sequence<int, kNs>{},
                      std::integral_constant<int, G::kBarrier>{});
        for_steps(kstep_kr, kt, std::make_integer_sequence<int, kNs>{},
                  std::integral_constant<int, G::kBarrier>{});
        for_steps(kstep_tail, kt + kNs, std::make_integer_sequence<int, kNs>{},
                  std::integral_constant<int, G::kBarrier>{});
    } else {
        for (int kt = 0; kt < nk; kt += kNs)
            for_steps(kstep, kt, std::make_integer_sequence<int, kNs>{},
                      std::integral_constant<int, G::kBarrier>{});
    }
    // nothing may still write this workgroup's LDS when it exits
    if constexpr (PW == 0) wait_vmcnt<0>();
    pin_acc(acc);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    pin_acc(acc);
    if (WHOLE || (m0 + EM <= M && n0 + EN <= N))
        store_tile<EPI, T, false>(acc, C, ldc, m0 + wm * G::kTM, n0 + wn * G::kTN, M, N, sign, flags);
    else
        store_tile<EPI, T, true>(acc, C, ldc, m0 + wm * G::kTM, n0 + wn * G::kTN, M, N, sign, flags);
}

}  // namespace dma

// One workgroup per CU with the default ring (128 KiB of LDS for E = 256 and 128; E = 256
// also takes all 256 accumulator registers of a lane); E = 128 with NS = 4 (64 KiB, 144
// registers per lane) and E = 64 (64 KiB with 8 stages, 32 KiB with 4; 40-56 registers)
// run two workgroups per CU.
// KR: K not a whole number of ring trips (the last trip's chunks past K load as zeros).
template <typename T, bool A_MN, bool B_MN, int EPI, int E, bool KR = false, int NS = dma::ring_stages(E)>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void mfma_f16_dma_kernel(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                         const uint16_t *__restrict__ B, int ldb, float *__restrict__ C,
                         int ldc, float sign, int flags) {
    constexpr int kNs = NS;
    __shared__ __attribute__((aligned(1024))) char lds[dma::Geo<E, E, 2, 2, kNs, 0>::kLds];
    int tm, tn;
    grouped_tile(xcd_contiguous_id(blockIdx.x, gridDim.x), cdiv(M, E), cdiv(N, E), 4, tm, tn);
    dma::dma_tile<T, A_MN, B_MN, EPI, E, E, 2, 2, kNs, 0, false, KR>(M, N, K, A, lda, B, ldb, C, ldc, sign,
                                                                      flags, tm * E, tn * E, lds);
}

// 192 x 256 and 256 x 192 tiles, for products whose 256 x 256 grid leaves CUs idle where
// a grid with one extent of 192 fills them (3072^2: 192 tiles instead of 144; 4096 x 3072:
// 256 instead of 192).  The same tile routine on four waves of 96 x 128 or 128 x 96, one
// workgroup per CU; every epilogue kind is taken.  The operand on the 192 side takes 192
// rows (k-contiguous) or 192-element rows of 24 chunks (m/n-contiguous) per k-step, 112 KiB
// of LDS in all.
// KR: K not a whole number of ring trips (the last trip's chunks past K load as zeros).
template <typename T, bool A_MN, bool B_MN, int EPI, int EM, int EN, bool KR = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void mfma_f16_dma_rect_kernel(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                              const uint16_t *__restrict__ B, int ldb, float *__restrict__ C,
                              int ldc, float sign, int flags) {
    static_assert((EM == 192 && EN == 256) || (EM == 256 && EN == 192), "one extent of 192");
    constexpr int kNs = dma::ring_stages(256);
    __shared__ __attribute__((aligned(1024))) char lds[dma::Geo<EM, EN, 2, 2, kNs, 0>::kLds];
    int tm, tn;
    grouped_tile(xcd_contiguous_id(blockIdx.x, gridDim.x), cdiv(M, EM), cdiv(N, EN), 4, tm, tn);
    dma::dma_tile<T, A_MN, B_MN, EPI, EM, EN, 2, 2, kNs, 0, false, KR>(
        M, N, K, A, lda, B, ldb, C, ldc, sign, flags, tm * EM, tn * EN, lds);
}

// Schedules of the same data movement that are kept for measurement (gemm355_run_variant
// with the MFMA_* schedule variants; plain products of whole tiles only): an EM x EN tile
// on WM x WN compute waves and PW producer waves, NS ring stages, one workgroup per CU.
template <typename T, int EM, int EN, int WM, int WN, int NS, int PW>
__global__ __launch_bounds__(64 * (WM * WN + PW)) __attribute__((amdgpu_waves_per_eu((WM * WN + PW + 3) / 4)))
void mfma_f16_dma_sched_kernel(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                               const uint16_t *__restrict__ B, int ldb, float *__restrict__ C,
                               int ldc) {
    __shared__ __attribute__((aligned(1024))) char lds[dma::Geo<EM, EN, WM, WN, NS, PW>::kLds];
    int tm, tn;
    grouped_tile(xcd_contiguous_id(blockIdx.x, gridDim.x), cdiv(M, EM), cdiv(N, EN), 4, tm, tn);
    dma::dma_tile<T, false, true, 0, EM, EN, WM, WN, NS, PW, true>(M, N, K, A, lda, B, ldb, C, ldc, 1.0f,
                                                                    0, tm * EM, tn * EN, lds);
}
