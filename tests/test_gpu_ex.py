"""GPU parity of the general form C = s op(A) op(B) (+ C) (``gemm355_gemm_ex``: transposed
and negated operands, accumulation into C; the tensor-core instruction table of
"Advanced CUDA features - starting from GEMM") against the oracle, through the C ABI.

Bars as for the plain product (relative Frobenius error of the result against the
oracle's binary64 value: 1e-5 FP32, 1e-3 FP16/BF16, and for every operand type max-abs
1e-4 sqrt(K) (+ the old C's scale when accumulating); with 16-bit C each element within
that bound plus its own rounding to the 16-bit format; small integers bit-exact).  Stored operands sit in
NaN-padded buffers with guard rows; C sits between sentinel guard words, and its M x N
region starts as NaN when it is overwritten (so every element must be written) or as
the values to accumulate into.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle
from gpu_util import NP_STORAGE, errors, nan_fill, place, to_device
from roofline_optimisation_amd import binding as gb
from roofline_optimisation_amd import inputs

pytestmark = pytest.mark.gpu

SENT = np.float32(7777.0)
GUARD = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def flags_of(ta, tb, na, nb, acc):
    return ((gb.TRANS_A if ta else 0) | (gb.TRANS_B if tb else 0) | (gb.NEG_A if na else 0)
            | (gb.NEG_B if nb else 0) | (gb.ACCUMULATE if acc else 0))


def run_ex(opA, opB, dtype, ta, tb, na, nb, acc, Cin=None, variant=gb.VARIANT_AUTO,
           pad=(0, 0, 0)):
    """Run the GPU form on op(A) (M x K) and op(B) (K x N) stored as the flags say.
    Returns (C, intact, stored A, stored B)."""
    import torch
    M, K = opA.shape
    N = opB.shape[1]
    SA = np.ascontiguousarray(opA.T) if ta else opA
    SB = np.ascontiguousarray(opB.T) if tb else opB
    lda, ldb, ldc = SA.shape[1] + pad[0], SB.shape[1] + pad[1], N + pad[2]
    dA = to_device(place(SA, max(lda, 1), 0, 1, nan_fill(dtype)))
    dB = to_device(place(SB, max(ldb, 1), 0, 1, nan_fill(dtype)))
    cbuf = np.full(2 * GUARD + M * ldc, SENT, np.float32)
    region = cbuf[GUARD:GUARD + M * ldc].reshape(M, ldc)
    region[:, :N] = Cin if acc else np.float32(np.nan)
    dC = to_device(cbuf)
    st = gb.gemm355_gemm_ex(variant, gb.DTYPE_CODES[dtype], flags_of(ta, tb, na, nb, acc), M, N, K,
                            dA.data_ptr(), max(lda, 1), dB.data_ptr(), max(ldb, 1),
                            dC.data_ptr() + 4 * GUARD, max(ldc, 1),
                            torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK, st
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    C = out[GUARD:GUARD + M * ldc].reshape(M, ldc)[:, :N].copy()
    mask = np.ones(out.shape, bool)
    mask[GUARD:GUARD + M * ldc].reshape(M, ldc)[:, :N] = False
    return C, bool(np.all(out[mask] == SENT)), SA, SB


def check(C, C64, dtype, K, Cin, intact, what):
    assert intact, f"{what}: wrote outside C"
    assert not np.isnan(C).any(), f"{what}: NaN (an element not written, or a read outside)"
    rel, mx = errors(C, C64)
    trel = 1e-5 if dtype == "f32" else 1e-3
    # Element bound for every operand type (16-bit products are exact in binary32, so
    # only the FP32 accumulation rounds): 1e-4 sqrt(K) for the sum, plus one rounding of
    # the old C
    tabs = 1e-4 * np.sqrt(max(K, 1)) + (np.abs(Cin).max() * 2 ** -23 if Cin is not None else 0)
    print(f"{what}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= trel and mx <= tabs, f"{what}: rel {rel:.3e} (<= {trel}), max {mx:.3e} (<= {tabs})"


def operands(M, N, K, dtype, seed, dist="uniform"):
    A, B = inputs.make_operands(M, N, K, seed, dist, dtype)
    Cin = np.random.default_rng(seed + 1000).uniform(-1, 1, (M, N)).astype(np.float32)
    return A, B, Cin


def compare(M, N, K, dtype, ta, tb, na, nb, acc, seed, variant=gb.VARIANT_AUTO, pad=(0, 0, 0)):
    A, B, Cin = operands(M, N, K, dtype, seed)
    C, ok, SA, SB = run_ex(A, B, dtype, ta, tb, na, nb, acc, Cin, variant, pad)
    C64, _ = oracle.gemm_ex(SA, SB, dtype, ta, tb, na, nb, Cin if acc else None)
    check(C, C64, dtype, K, Cin if acc else None, ok,
          f"ex {dtype} {M}x{N}x{K} ta={ta} tb={tb} na={na} nb={nb} acc={acc} v={variant} pad={pad}")


FLAGS = list(itertools.product([False, True], repeat=5))


@pytest.mark.parametrize("variant", [gb.VARIANT_MFMA, gb.VARIANT_NAIVE], ids=["mfma", "naive"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("fl", FLAGS, ids=lambda f: "".join(n for n, b in zip(("ta", "tb", "na", "nb", "acc"), f) if b) or "plain")
def test_flag_matrix_ragged(fl, dtype, variant):
    compare(129, 97, 75, dtype, *fl, seed=50, variant=variant)


# Interior tiles of every layout: FP32 192 x 192 (3072), 128 x 128 (2048), 96 x 96 (1536; ragged
# M, N and K), 64 x 64; FP16/BF16 256 x 256 direct-to-LDS (3072^2, K % 128 == 0, and K = 192
# with the chunks past K zero-filled), 256 x 256 register-staged (K = 64, below one ring
# trip) and 128 x 128; each plain, negated and accumulating.  16-bit C adds K = 196 (not a
# multiple of 8: the clamped register-staged kernel).
LAYOUTS = list(itertools.product([False, True], repeat=2))
MODES = [(False, False, False), (True, False, False), (False, True, True)]  # na, nb, acc
SHAPES = {"f32": [(3072, 3072, 64), (1024, 768, 96), (2048, 2048, 64), (1536, 1536, 96), (1351, 1537, 100),
                  (2000, 1996, 256), (2000, 1996, 260)],
          "f16": [(3072, 3072, 128), (3072, 2816, 192), (1024, 1024, 128), (4000, 3992, 128),
                  (3072, 3072, 64), (2048, 2048, 264), (2560, 2048, 192)],
          "bf16": [(3072, 3072, 256), (1024, 512, 64), (2000, 2040, 256)]}
# FP32 (2000, 1996, 256) and (2000, 1996, 260): ragged tiles in the unpredicated kernel
# with the full ones, the latter with a zero-filled last k-step.
# (3072, 2816, 192) and (2048, 2048, 264): K not a whole number of ring trips on the
# direct-to-LDS kernel (256 x 256 and 128 x 128 tiles; the last trip's steps past K are
# skipped: 2 of 4 and 7 of 8).
# (2560, 2048, 192): 320 tiles of 128 x 128 on the direct-to-LDS kernel's 4-stage ring, two
# workgroups per CU, K not a whole number of its trips (192 = 128 + 64).
# (3072, 3072, 128), (3072, 2816, 192) and BF16 (3072, 3072, 256), every layout and mode:
# the 192 x 256 direct-to-LDS tile (with A transposed its A in LDS rows of 24 chunks), the second
# with K not a whole number of ring trips; with both transposed the 256 x 192 tile (B
# k-contiguous on the 192 side).
# (4000, 3992, 128) and (2000, 2040, 256): every tile, ragged ones included, on the
# direct-to-LDS kernel (256 x 256 and 128 x 128 tiles); the padding around the operands
# holds NaN, so a ragged tile's loads past the matrix would show in its stored outputs.


@pytest.mark.parametrize("mode", MODES, ids=["plain", "neg_a", "neg_b_acc"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"ta{int(l[0])}tb{int(l[1])}")
@pytest.mark.parametrize("dtype,shape", [(d, s) for d in SHAPES for s in SHAPES[d]],
                         ids=lambda x: x if isinstance(x, str) else "x".join(map(str, x)))
def test_tiles_every_layout(dtype, shape, layout, mode):
    compare(*shape, dtype, *layout, *mode, seed=51)


@pytest.mark.parametrize("mode", MODES, ids=["plain", "neg_a", "neg_b_acc"])
@pytest.mark.parametrize("pad", [(0, 0, 0), (1, 3, 2)], ids=["packed", "unaligned"])
def test_f32_both_mn_whole_192_tiles(pad, mode):
    """A transposed, B not (both operands m/n-contiguous) with M, N multiples of 192: the
    192 x 192 tile's unpaired interior kernels, an odd number of k-steps, 16-byte loads
    at 16-byte and at element alignment."""
    compare(1152, 1536, 96, "f32", True, False, *mode, seed=66, pad=pad)


@pytest.mark.parametrize("mode", MODES, ids=["plain", "neg_a", "neg_b_acc"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"ta{int(l[0])}tb{int(l[1])}")
def test_f32_unaligned_rows_every_tile(layout, mode):
    """FP32 rows that are not 16-byte aligned, K a multiple of 4 and m/n-contiguous extents
    multiples of 4: every tile, ragged ones included, in one unpredicated launch with dword
    loads at clamped coordinates (K = 500: the last k-step zero-filled)."""
    compare(996, 1000, 512, "f32", *layout, *mode, seed=68, pad=(1, 3, 2))
    compare(996, 1000, 500, "f32", *layout, *mode, seed=69, pad=(1, 3, 2))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"ta{int(l[0])}tb{int(l[1])}")
def test_unaligned_strides(dtype, layout):
    """Row strides that are not multiples of 16 bytes take 16-byte loads at element alignment."""
    compare(300, 260, 130, dtype, *layout, False, False, True, seed=52, pad=(1, 3, 2))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("fl", [(True, False, True, False, True), (False, True, False, False, False),
                                (True, True, True, True, True)],
                         ids=["ta_na_acc", "tb", "all"])
def test_integers_bit_exact(dtype, fl):
    for (M, N, K) in [(257, 130, 77), (512, 512, 256)]:
        A, B = inputs.make_operands(M, N, K, 53, "int", dtype)
        Cin = np.random.default_rng(54).integers(-50, 51, (M, N)).astype(np.float32)
        C, ok, SA, SB = run_ex(A, B, dtype, *fl, Cin)
        _, C32 = oracle.gemm_ex(SA, SB, dtype, *fl[:4], Cin if fl[4] else None)
        assert ok and np.array_equal(C, C32), (dtype, fl, M, N, K)


# Transposed layouts on the register-staged kernel's clamped ragged tiles with the
# two-set pipeline (K = 1004: 16 64-wide k-steps, every tile ragged in K, K not a multiple
# of 8 so the direct-to-LDS kernel does not take it): every element within the float bar,
# and integer operands bit for bit.
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("layout", [(True, False), (False, True), (True, True)],
                         ids=["ta", "tb", "tatb"])
def test_clamped_paired_transposed(dtype, layout):
    ta, tb = layout
    M, N, K = 1000, 1000, 1004
    P = 1 << 20
    flags = flags_of(ta, tb, False, False, False)
    lda, ldb = (M if ta else K), (K if tb else N)
    desc = gb.gemm355_kernel_desc_ex(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], flags, M, N, K,
                                     P, lda, P, ldb, P, N)
    assert desc.endswith("| edges=clamped,paired"), desc
    compare(M, N, K, dtype, ta, tb, False, False, False, seed=61)
    A, B = inputs.make_operands(M, N, K, 62, "int", dtype)
    C, ok, SA, SB = run_ex(A, B, dtype, ta, tb, False, False, False)
    _, C32 = oracle.gemm_ex(SA, SB, dtype, ta, tb, False, False, None)
    assert ok and np.array_equal(C, C32)


def test_k_zero():
    import torch
    # K = 0: C = +0 (negated: -0, equal in value), or C unchanged when accumulating
    for acc in (False, True):
        A = np.zeros((5, 0), np.float32)
        B = np.zeros((0, 7), np.float32)
        Cin = np.arange(35, dtype=np.float32).reshape(5, 7)
        C, ok, _, _ = run_ex(A, B, "f32", False, False, True, False, acc, Cin)
        assert ok and np.array_equal(C, Cin if acc else np.zeros((5, 7), np.float32))


def test_matmul_wrapper_options():
    import torch
    A, B, Cin = operands(70, 50, 40, "f32", 55)
    dA = torch.from_numpy(np.ascontiguousarray(A.T)).cuda()
    dB = torch.from_numpy(np.ascontiguousarray(B.T)).cuda()
    out = torch.from_numpy(Cin.copy()).cuda()
    gb.matmul(dA, dB, out=out, trans_a=True, trans_b=True, neg_a=True, accumulate=True)
    C64, _ = oracle.gemm_ex(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), "f32", True, True,
                            True, False, Cin)
    check(out.cpu().numpy(), C64, "f32", 40, Cin, True, "matmul wrapper ex")


# ---------------------------------------------------------------- C in the 16-bit type

SENT16 = np.uint16(0x7777)
NAN16 = {"f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}
P16 = {"f16": 11, "bf16": 8}


def decode16(bits: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_ex16(opA, opB, dtype, ta, tb, na, nb, acc, Cin16=None, variant=gb.VARIANT_AUTO,
             pad=(0, 0, 0), coff=0):
    """Like run_ex with GEMM355_C_16: C (and Cin16) are 16-bit patterns of `dtype`; C
    starts `coff` elements after a 4-byte aligned guard (coff = 1: only 2-byte aligned)."""
    import torch
    M, K = opA.shape
    N = opB.shape[1]
    SA = np.ascontiguousarray(opA.T) if ta else opA
    SB = np.ascontiguousarray(opB.T) if tb else opB
    lda, ldb, ldc = SA.shape[1] + pad[0], SB.shape[1] + pad[1], N + pad[2]
    dA = to_device(place(SA, max(lda, 1), 0, 1, nan_fill(dtype)))
    dB = to_device(place(SB, max(ldb, 1), 0, 1, nan_fill(dtype)))
    g0 = GUARD + coff
    cbuf = np.full(2 * GUARD + coff + M * ldc, SENT16, np.uint16)
    region = cbuf[g0:g0 + M * ldc].reshape(M, ldc)
    region[:, :N] = Cin16 if acc else NAN16[dtype]
    dC = to_device(cbuf)
    flags = flags_of(ta, tb, na, nb, acc) | gb.C_16
    st = gb.gemm355_gemm_ex(variant, gb.DTYPE_CODES[dtype], flags, M, N, K, dA.data_ptr(), max(lda, 1),
                            dB.data_ptr(), max(ldb, 1), dC.data_ptr() + 2 * g0, max(ldc, 1),
                            torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK, st
    torch.cuda.synchronize()
    out = dC.cpu().numpy().view(np.uint16)
    C = out[g0:g0 + M * ldc].reshape(M, ldc)[:, :N].copy()
    mask = np.ones(out.shape, bool)
    mask[g0:g0 + M * ldc].reshape(M, ldc)[:, :N] = False
    return C, bool(np.all(out[mask] == SENT16)), SA, SB


def compare16(M, N, K, dtype, ta, tb, na, nb, acc, seed, variant=gb.VARIANT_AUTO, pad=(0, 0, 0),
              coff=0):
    A, B = inputs.make_operands(M, N, K, seed, "uniform", dtype)
    Cin16 = inputs.to_storage(np.random.default_rng(seed + 1000).uniform(-1, 1, (M, N)).astype(np.float32), dtype)
    C, ok, SA, SB = run_ex16(A, B, dtype, ta, tb, na, nb, acc, Cin16, variant, pad, coff)
    C64, _ = oracle.gemm_ex16(SA, SB, dtype, ta, tb, na, nb, Cin16 if acc else None)
    what = (f"ex16 {dtype} {M}x{N}x{K} ta={ta} tb={tb} na={na} nb={nb} acc={acc} v={variant} "
            f"pad={pad} coff={coff}")
    assert ok, f"{what}: wrote outside C"
    got = decode16(C, dtype)
    assert not np.isnan(got).any(), f"{what}: NaN (an element not written, or a read outside)"
    rel, mx = errors(got, C64)
    bar = 2.0 ** -P16[dtype] + 1e-5
    # Element bound: the binary32 value s.sum (+ old C) is within 1e-4 sqrt(K) of the
    # exact one (the FP32 bar; the old C is exact in binary32), and rounding it to the
    # 16-bit format moves it by at most 2^-p of its magnitude, or by half the binary16
    # subnormal spacing (2^-25) below the normal range.
    tabs = 1e-4 * np.sqrt(max(K, 1))
    sub = 2.0 ** -25 if dtype == "f16" else 0.0
    elem = tabs * (1 + 2.0 ** -P16[dtype]) + 2.0 ** -P16[dtype] * np.abs(C64) + sub
    worst = float((np.abs(got - C64) / elem).max()) if got.size else 0.0
    print(f"{what}: rel_frob={rel:.3e} (bar {bar:.3e}) worst element/bound={worst:.3f}", flush=True)
    assert rel <= bar, f"{what}: rel {rel:.3e} > {bar:.3e}"
    assert worst <= 1.0, f"{what}: an element is {worst:.3f} x its bound"


FLAGS16 = list(itertools.product([False, True], repeat=5))


@pytest.mark.parametrize("variant", [gb.VARIANT_MFMA, gb.VARIANT_NAIVE], ids=["mfma", "naive"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("fl", FLAGS16, ids=lambda f: "".join(n for n, b in zip(("ta", "tb", "na", "nb", "acc"), f) if b) or "plain")
def test_c16_flag_matrix_ragged(fl, dtype, variant):
    compare16(129, 97, 75, dtype, *fl, seed=56, variant=variant)


SHAPES16 = [(3072, 3072, 128), (3072, 2816, 192), (1024, 1024, 128), (1024, 512, 64), (3072, 3072, 196),
            (2560, 2048, 192)]


@pytest.mark.parametrize("mode", MODES, ids=["plain", "neg_a", "neg_b_acc"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"ta{int(l[0])}tb{int(l[1])}")
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES16, ids=lambda s: "x".join(map(str, s)))
def test_c16_tiles_every_layout(shape, dtype, layout, mode):
    compare16(*shape, dtype, *layout, *mode, seed=57)


@pytest.mark.parametrize("mode", [MODES[0], MODES[2]], ids=["plain", "neg_b_acc"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"ta{int(l[0])}tb{int(l[1])}")
def test_c16_ragged_direct_to_lds(layout, mode):
    """2824^2 x 128 on the direct-to-LDS kernel, with C in FP16 (guarded 2- and 4-byte
    stores): A k-contiguous on 15 x 12 tiles of 192 x 256, the last row of tiles 136 high;
    A transposed on 12 x 12 tiles of 256, the last row 8 high; the last column of tiles 8
    wide in both."""
    compare16(2824, 2824, 128, "f16", *layout, *mode, seed=58)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"ta{int(l[0])}tb{int(l[1])}")
def test_c16_unaligned_strides(dtype, layout):
    compare16(300, 260, 130, dtype, *layout, False, False, True, seed=58, pad=(1, 3, 2))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("fl", [(False, False, False, False, False), (True, False, True, False, True),
                                (False, True, False, False, True), (True, True, True, True, True)],
                         ids=["plain", "ta_na_acc", "tb_acc", "all"])
def test_c16_integers_bit_exact(dtype, fl):
    """Integer sums are exact in FP32, so both sides round the same exact value once."""
    for (M, N, K) in [(257, 130, 77), (512, 512, 256), (3072, 3072, 128)]:
        A, B = inputs.make_operands(M, N, K, 59, "int", dtype)
        Cin16 = inputs.to_storage(np.random.default_rng(60).integers(-50, 51, (M, N)).astype(np.float32), dtype)
        C, ok, SA, SB = run_ex16(A, B, dtype, *fl, Cin16)
        _, C16 = oracle.gemm_ex16(SA, SB, dtype, *fl[:4], Cin16 if fl[4] else None)
        # values, not zero signs (a negated product summing to 0 is -0.0)
        assert ok and np.array_equal(decode16(C, dtype), decode16(C16, dtype)), (dtype, fl, M, N, K)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("fl", [(False, False, False, False, False), (False, False, True, False, True),
                                (True, True, False, True, True)], ids=["plain", "na_acc", "ta_tb_nb_acc"])
@pytest.mark.parametrize("case", ["odd_n_even_ldc", "c_2byte_aligned", "big_odd_n"])
def test_c16_column_pairs(case, fl, dtype):
    """The column-pair epilogue (even ldc, 4-byte aligned C) with an odd N (its last pair
    is half inside), and the per-element epilogue when C is only 2-byte aligned."""
    if case == "odd_n_even_ldc":
        compare16(129, 97, 75, dtype, *fl, seed=61, pad=(0, 0, 1))
    elif case == "c_2byte_aligned":
        compare16(520, 300, 96, dtype, *fl, seed=62, coff=1)
    else:
        compare16(1300, 1025, 256, dtype, *fl, seed=63, pad=(0, 0, 3))


def test_c16_k_zero():
    for dtype in ("f16", "bf16"):
        A = np.zeros((5, 0), np.uint16)
        B = np.zeros((0, 7), np.uint16)
        Cin16 = inputs.to_storage(np.arange(35, dtype=np.float32).reshape(5, 7), dtype)
        for acc in (False, True):
            C, ok, _, _ = run_ex16(A, B, dtype, False, False, False, False, acc, Cin16)
            want = decode16(Cin16, dtype) if acc else np.zeros((5, 7))
            assert ok and np.array_equal(decode16(C, dtype), want), (dtype, acc)


def test_matmul_wrapper_c16():
    import torch
    A, B = inputs.make_operands(70, 50, 40, 64, "uniform", "bf16")
    Cin16 = inputs.to_storage(np.random.default_rng(65).uniform(-1, 1, (70, 50)).astype(np.float32), "bf16")
    dA = torch.from_numpy(A.view(np.int16)).cuda().view(torch.bfloat16)
    dB = torch.from_numpy(B.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.from_numpy(Cin16.view(np.int16)).cuda().view(torch.bfloat16)
    gb.matmul(dA, dB, out=out, neg_b=True, accumulate=True)
    C64, _ = oracle.gemm_ex16(A, B, "bf16", False, False, False, True, Cin16)
    got = decode16(out.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    rel, _ = errors(got, C64)
    assert rel <= 2.0 ** -8 + 1e-5, rel


# The 192 x 256 and 256 x 192 direct-to-LDS tiles in the general form: 192 x 256 with B
# transposed, negated and accumulating (K not a whole number of ring trips) and with B not
# transposed; 256 x 192 (B transposed, so k-contiguous) with A transposed, ragged M and N,
# K not a whole number of ring trips, negated and accumulating, and plain on 4096 x 3072
# (256 tiles against 192 of 256 x 256); and with the 192 side m/n-contiguous, in LDS rows
# of 24 chunks: 192 x 256 with A transposed (ragged N, K past whole trips, negated B, accumulating)
# and 256 x 192 with B n-contiguous (negated A, padded B rows, 520 = 4 x 128 + 8); each with
# FP32 and with 16-bit C, against the oracle and bit for bit against the same call on
# 256 x 256 tiles (VARIANT_MFMA_T256X256).
RECT_EX = [("f16", (3072, 3072, 264), (False, True, True, False, True), (8, 8, 8), "192x256x32"),
           ("bf16", (3000, 3072, 256), (False, False, False, True, True), (0, 0, 0), "192x256x32"),
           ("bf16", (3000, 3000, 1000), (True, True, True, False, True), (8, 8, 8), "256x192x32"),
           ("f16", (4096, 3072, 512), (False, True, False, False, False), (0, 0, 0), "256x192x32"),
           ("f16", (3072, 3000, 264), (True, False, False, True, True), (8, 8, 8), "192x256x32"),
           ("bf16", (4096, 3072, 520), (False, False, True, False, False), (0, 8, 0), "256x192x32"),
           # one ring trip exactly, and one trip plus one 8-wide chunk of K
           ("f16", (3072, 3072, 128), (False, False, False, False, False), (0, 0, 0), "192x256x32"),
           ("bf16", (3000, 3000, 136), (True, False, False, False, True), (8, 8, 8), "192x256x32")]


@pytest.mark.parametrize("case", RECT_EX, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])) + "_" + c[4][:7])
def test_rect_tile_general_form(case):
    dtype, (M, N, K), fl, pad, tile = case
    ta, tb = fl[0], fl[1]
    lda = (M if ta else K) + pad[0]
    ldb = (K if tb else N) + pad[1]
    P = 1 << 20
    flags = flags_of(*fl)
    code = gb.DTYPE_CODES[dtype]
    assert gb.gemm355_kernel_desc_ex(gb.VARIANT_AUTO, code, flags, M, N, K, P, lda, P, ldb, P,
                                     N + pad[2]).startswith(f"mfma_{dtype} {tile}")
    assert gb.gemm355_kernel_desc_ex(gb.VARIANT_MFMA_T256X256, code, flags, M, N, K, P, lda, P, ldb, P,
                                     N + pad[2]).startswith(f"mfma_{dtype} 256x256x32")
    A, B, Cin = operands(M, N, K, dtype, 67)
    Cr, ok_r, SA, SB = run_ex(A, B, dtype, *fl, Cin, gb.VARIANT_AUTO, pad)
    Cs, ok_s, _, _ = run_ex(A, B, dtype, *fl, Cin, gb.VARIANT_MFMA_T256X256, pad)
    assert np.array_equal(Cr.view(np.uint32), Cs.view(np.uint32)), "192 x 256 and 256 x 256 tiles differ"
    C64, _ = oracle.gemm_ex(SA, SB, dtype, *fl[:4], Cin if fl[4] else None)
    check(Cr, C64, dtype, K, Cin if fl[4] else None, ok_r and ok_s, f"ex rect {dtype} {M}x{N}x{K} {fl}")
    Cin16 = inputs.to_storage(Cin, dtype)
    C16r, ok_r, SA, SB = run_ex16(A, B, dtype, *fl, Cin16, gb.VARIANT_AUTO, pad)
    C16s, ok_s, _, _ = run_ex16(A, B, dtype, *fl, Cin16, gb.VARIANT_MFMA_T256X256, pad)
    assert ok_r and ok_s and np.array_equal(C16r, C16s), "16-bit C: 192 x 256 and 256 x 256 tiles differ"


# The 64 x 64 direct-to-LDS tile in the general form (the 128 x 128 grid would leave CUs
# idle, the 64 x 64 one holds at most 512 tiles): every transpose, negation and
# accumulation, ragged M and N (1000 = 15 x 64 + 40, 904 = 14 x 64 + 8), K not a whole
# number of 256-deep ring trips (1000, 264) with NaN-padded strides, 1400 x 1400 (484
# tiles); each with FP32 and with 16-bit C, against the oracle.
DMA64_EX = [("f16", (1024, 1024, 1024), (True, False, False, False, False), (0, 0, 0)),
            ("bf16", (1024, 1024, 1024), (False, True, True, False, True), (0, 0, 0)),
            ("f16", (1000, 904, 1000), (True, True, False, True, True), (8, 8, 8)),
            ("bf16", (512, 512, 264), (True, False, True, True, False), (8, 0, 8)),
            ("f16", (768, 768, 1024), (False, False, True, True, True), (0, 8, 0)),
            ("bf16", (1400, 1400, 1000), (False, False, False, False, False), (8, 8, 8)),
            # K from 128 to 255: the 4-stage ring (192 = 128 + 64)
            ("f16", (1024, 1024, 192), (True, True, True, False, True), (8, 8, 8)),
            # thin M or N of 72 (a last tile 8 wide): A m-contiguous, B n-contiguous
            ("bf16", (72, 4096, 512), (True, False, False, False, False), (8, 8, 8)),
            ("f16", (4096, 72, 1024), (False, False, False, True, True), (0, 8, 0))]


@pytest.mark.parametrize("case", DMA64_EX, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])) + "_" +
                         "".join("1" if f else "0" for f in c[2]))
def test_dma64_general_form(case):
    dtype, (M, N, K), fl, pad = case
    ta, tb = fl[0], fl[1]
    lda = (M if ta else K) + pad[0]
    ldb = (K if tb else N) + pad[1]
    P = 1 << 20
    flags = flags_of(*fl)
    code = gb.DTYPE_CODES[dtype]
    desc = gb.gemm355_kernel_desc_ex(gb.VARIANT_AUTO, code, flags, M, N, K, P, lda, P, ldb, P, N + pad[2])
    assert desc.startswith(f"mfma_{dtype} 64x64x32 w2x2 lds-dma"), desc
    A, B, Cin = operands(M, N, K, dtype, 71)
    C, ok, SA, SB = run_ex(A, B, dtype, *fl, Cin, gb.VARIANT_AUTO, pad)
    C64, _ = oracle.gemm_ex(SA, SB, dtype, *fl[:4], Cin if fl[4] else None)
    check(C, C64, dtype, K, Cin if fl[4] else None, ok, f"ex dma64 {dtype} {M}x{N}x{K} {fl}")
    assert gb.gemm355_kernel_desc_ex(gb.VARIANT_AUTO, code, flags | gb.C_16, M, N, K, P, lda, P, ldb, P,
                                     N + pad[2]).startswith(f"mfma_{dtype} 64x64x32 w2x2 lds-dma")
    compare16(M, N, K, dtype, *fl, 72, gb.VARIANT_AUTO, pad)
