"""GPU parity of the measurement-only schedules of the FP16/BF16 direct-to-LDS kernel
(``gemm355_run_variant`` with VARIANT_MFMA_SPLIT: four producer waves load while four
compute waves multiply; VARIANT_MFMA_W8: eight waves, two per SIMD; VARIANT_MFMA_T256X128:
256 x 128 tiles), through the C ABI, against the oracle.

Bars as for the dispatched kernel: relative Frobenius error <= 1e-3 and every element
within 1e-4 sqrt(K) of the oracle's binary64 value (16-bit products are exact in binary32),
small-integer operands bit-exact.  Operands sit in NaN-padded buffers with guard rows and
C between sentinels (gpu_util.gpu_gemm)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import errors, gpu_gemm, sample_rows, tolerance
from roofline_optimisation_amd import binding as gb
from roofline_optimisation_amd import inputs

pytestmark = pytest.mark.gpu

SCHED = [gb.VARIANT_MFMA_SPLIT, gb.VARIANT_MFMA_W8, gb.VARIANT_MFMA_T256X128]
SNAME = {gb.VARIANT_MFMA_SPLIT: "split", gb.VARIANT_MFMA_W8: "w8",
         gb.VARIANT_MFMA_T256X128: "t256x128"}
P = 1 << 20  # a 16-byte-aligned non-null address for host-only queries


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def check(C, C64, dtype, K, intact, what):
    assert intact, f"{what}: wrote outside C"
    assert not np.isnan(C).any(), f"{what}: NaN in result (read outside the operands?)"
    rel, mx = errors(C, C64)
    trel, tabs = tolerance(dtype, "uniform", K)
    print(f"{what}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= trel and mx <= tabs, f"{what}: rel {rel:.3e} (<= {trel}), max {mx:.3e} (<= {tabs})"


# The shortest K (one trip of the 4-stage ring), several trips on a non-square grid of
# tiles, padded 16-byte-aligned strides, and the 4096^3 workload in full.
CASES = [((512, 512, 128), (0, 0, 0)), ((1024, 768, 512), (0, 0, 0)),
         ((768, 1024, 384), (8, 16, 8)), ((4096, 4096, 4096), (0, 0, 0))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}")
@pytest.mark.parametrize("variant", SCHED, ids=lambda v: SNAME[v])
def test_sched_parity(variant, case, dtype):
    (M, N, K), pad = case
    code = gb.DTYPE_CODES[dtype]
    desc = gb.gemm355_kernel_desc(variant, code, M, N, K, P, K + pad[0], P, N + pad[1], P, N + pad[2])
    assert "lds-dma" in desc, desc
    A, B = inputs.make_operands(M, N, K, 71, "uniform", dtype)
    C64, _ = oracle.gemm(A, B, dtype)
    C, ok = gpu_gemm(A, B, dtype, variant, pad=pad, guard_rows=1)
    check(C, C64, dtype, K, ok, f"{SNAME[variant]} {dtype} {M}x{N}x{K} pad={pad}")
    if M * N * K <= 1 << 30:
        Ai, Bi = inputs.make_operands(M, N, K, 72, "int", dtype)
        _, C32 = oracle.gemm(Ai, Bi, dtype)
        Ci, ok = gpu_gemm(Ai, Bi, dtype, variant, pad=pad)
        assert ok and np.array_equal(Ci, C32), f"{SNAME[variant]} {dtype} integers not bit-exact"


@pytest.mark.parametrize("variant", SCHED, ids=lambda v: SNAME[v])
def test_sched_8192_sampled(variant):
    """8192^3 BF16 (four tiles per CU at 256 x 256): sampled rows, the first and last of
    each 256-row tile band included."""
    M = N = K = 8192
    A, B = inputs.make_operands(M, N, K, 73, "uniform", "bf16")
    C, ok = gpu_gemm(A, B, "bf16", variant)
    rows = np.array(sorted(set(sample_rows(M, 24).tolist()) | {255, 256, 4095, 4096, M - 1}))
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, "bf16")
    check(C[rows], C64, "bf16", K, ok, f"{SNAME[variant]} bf16 8192^3 sampled")


@pytest.mark.parametrize("variant", SCHED, ids=lambda v: SNAME[v])
def test_sched_run_twice_bitwise(variant):
    M, N, K = 1024, 1024, 1024
    A, B = inputs.make_operands(M, N, K, 74, "uniform", "f16")
    C1, _ = gpu_gemm(A, B, "f16", variant)
    C2, _ = gpu_gemm(A, B, "f16", variant)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


# VARIANT_MFMA_T256X256 (the dispatcher without the 192-wide tiles) at shapes where the
# dispatcher takes 192 x 256: the same result bit for bit as the dispatched call (both
# tiles add each element's products in the same order), and within the bars of the
# oracle on sampled rows; ragged M and N, K not a whole number of ring trips, padded
# strides.
SQUARE_CASES = [("f16", (3072, 3072, 3072), (0, 0, 0)), ("bf16", (3000, 3072, 1000), (8, 8, 8)),
                ("f16", (4096, 4104, 512), (0, 8, 0))]


@pytest.mark.parametrize("case", SQUARE_CASES, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])))
def test_square_tile_variant_matches_dispatched(case):
    dtype, (M, N, K), pad = case
    code = gb.DTYPE_CODES[dtype]
    v = gb.VARIANT_MFMA_T256X256
    args = (M, N, K, P, K + pad[0], P, N + pad[1], P, N + pad[2])
    assert gb.gemm355_kernel_desc(gb.VARIANT_AUTO, code, *args).startswith(f"mfma_{dtype} 192x256x32")
    assert gb.gemm355_kernel_desc(v, code, *args).startswith(f"mfma_{dtype} 256x256x32")
    A, B = inputs.make_operands(M, N, K, 75, "uniform", dtype)
    Cs, ok_s = gpu_gemm(A, B, dtype, v, pad=pad, guard_rows=1)
    Cd, ok_d = gpu_gemm(A, B, dtype, gb.VARIANT_AUTO, pad=pad, guard_rows=1)
    assert ok_s and ok_d, "wrote outside C"
    assert np.array_equal(Cs.view(np.uint32), Cd.view(np.uint32)), "256 x 256 and 192 x 256 tiles differ"
    rows = np.array(sorted(set(sample_rows(M, 24).tolist()) | {191, 192, 255, 256, M - 1}))
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype)
    check(Cs[rows], C64, dtype, K, ok_s, f"t256x256 {dtype} {M}x{N}x{K} pad={pad}")


# VARIANT_MFMA_STAGED128 (the dispatcher without the two-per-CU 128 x 128 direct-to-LDS
# tile) where the dispatcher takes that tile: the register-staged kernel, within the bars
# of the oracle (the two kernels may round differently: one or two MFMAs per 32-wide
# k-step).
STAGED_CASES = [("f16", (2304, 2304, 512), (0, 0, 0)), ("bf16", (2500, 2600, 1000), (8, 8, 8))]


@pytest.mark.parametrize("case", STAGED_CASES, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])))
def test_staged128_variant(case):
    dtype, (M, N, K), pad = case
    code = gb.DTYPE_CODES[dtype]
    v = gb.VARIANT_MFMA_STAGED128
    args = (M, N, K, P, K + pad[0], P, N + pad[1], P, N + pad[2])
    assert "lds-dma ring4" in gb.gemm355_kernel_desc(gb.VARIANT_AUTO, code, *args)
    assert "128x128x64 w2x2 dwordx4" in gb.gemm355_kernel_desc(v, code, *args)
    A, B = inputs.make_operands(M, N, K, 76, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, v, pad=pad, guard_rows=1)
    C64, _ = oracle.gemm(A, B, dtype)
    check(C, C64, dtype, K, ok, f"staged128 {dtype} {M}x{N}x{K} pad={pad}")


# VARIANT_MFMA_STAGED_SMALL (the dispatcher without the direct-to-LDS tiles of small grids)
# where the dispatcher takes one of them: the register-staged 64 x 64 and 128 x 64 tiles of
# plain products, and register staging for K from 128 to 255 (136, predicated tiles); within
# the bars of the oracle.
STAGED_SMALL_CASES = [("bf16", (1024, 1024, 1024), (0, 0, 0), "64x64x64 w1x2 dwordx4"),
                      ("f16", (1536, 1536, 1536), (8, 8, 8), "128x64x64 w2x2 dwordx4"),
                      ("f16", (2048, 2048, 136), (8, 8, 8), "128x128x64 w2x2 dwordx4")]


@pytest.mark.parametrize("case", STAGED_SMALL_CASES, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])))
def test_staged_small_variant(case):
    dtype, (M, N, K), pad, kernel = case
    code = gb.DTYPE_CODES[dtype]
    v = gb.VARIANT_MFMA_STAGED_SMALL
    args = (M, N, K, P, K + pad[0], P, N + pad[1], P, N + pad[2])
    assert "lds-dma" in gb.gemm355_kernel_desc(gb.VARIANT_AUTO, code, *args)
    desc = gb.gemm355_kernel_desc(v, code, *args)
    assert kernel in desc, desc
    A, B = inputs.make_operands(M, N, K, 77, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, v, pad=pad, guard_rows=1)
    C64, _ = oracle.gemm(A, B, dtype)
    check(C, C64, dtype, K, ok, f"staged_small {dtype} {M}x{N}x{K} pad={pad}")
