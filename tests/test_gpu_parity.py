"""GPU parity: every kernel family, through the C ABI, against the CPU oracle.

Bars: bit-exact on small-integer inputs (every partial sum is an exact integer below
2^24); FP32 with U[-1,1] inputs: relative Frobenius error <= 1e-5 and max-abs error
<= 1e-4 sqrt(K); FP32 with N(0,1) inputs: 1e-5 and 3e-4 sqrt(K); FP16/BF16 inputs,
against the oracle on the same rounded inputs: relative Frobenius error <= 1e-3 and the
same element bound as FP32 (16-bit products are exact in binary32; only the FP32
accumulation rounds).
Out-of-range reads are caught by NaN-poisoned padding and guard rows, out-of-range
writes by a sentinel-filled C buffer.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import errors, gpu_gemm, sample_rows, tolerance
from roofline_optimisation_amd import binding as gb
from roofline_optimisation_amd import inputs

pytestmark = pytest.mark.gpu

F32_VARIANTS = [gb.VARIANT_NAIVE, gb.VARIANT_LDS_TILED, gb.VARIANT_REGBLOCK, gb.VARIANT_MFMA]
H_VARIANTS = [gb.VARIANT_NAIVE, gb.VARIANT_MFMA]
VNAME = {v: k for k, v in gb.VARIANTS.items()}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def check(C, C64, dtype, dist, K, intact, what):
    assert intact, f"{what}: wrote outside C"
    assert not np.isnan(C).any(), f"{what}: NaN in result (read outside the operands?)"
    rel, mx = errors(C, C64)
    trel, tabs = tolerance(dtype, dist, K)
    print(f"{what}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= trel and mx <= tabs, f"{what}: rel {rel:.3e} (<= {trel}), max {mx:.3e} (<= {tabs})"


def case_params():
    out = []
    for v in F32_VARIANTS:
        out.append(("f32", v))
    for v in H_VARIANTS:
        out += [("f16", v), ("bf16", v)]
    return out


# ------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("variant", F32_VARIANTS, ids=lambda v: VNAME[v])
def test_f32_256(variant):
    c = inputs.CASES["f32_256"]
    A, B = inputs.operands_for(c)
    C64, _ = oracle.gemm(A, B)
    C, ok = gpu_gemm(A, B, "f32", variant, pad=(3, 5, 7), guard_rows=2)
    check(C, C64, "f32", c.dist, c.K, ok, f"f32_256 {VNAME[variant]}")


@pytest.mark.parametrize("dtype,variant", case_params(), ids=lambda x: str(x))
def test_small_integers_bit_exact(dtype, variant):
    c = inputs.CASES["f32_256_int"]
    A, B = inputs.make_operands(c.M, c.N, c.K, c.seed, "int", dtype)
    _, C32 = oracle.gemm(A, B, dtype)
    C, ok = gpu_gemm(A, B, dtype, variant)
    assert ok and np.array_equal(C, C32), f"{dtype} {VNAME[variant]} not bit-exact"
    # ragged integer case crossing every tile edge and the K tail
    A, B = inputs.make_operands(211, 173, 333, 5, "int", dtype)
    _, C32 = oracle.gemm(A, B, dtype)
    C, ok = gpu_gemm(A, B, dtype, variant, pad=(1, 3, 2), offset=1, guard_rows=1)
    assert ok and np.array_equal(C, C32), f"{dtype} {VNAME[variant]} ragged not bit-exact"


@pytest.mark.parametrize("name", ["f32_1000", "f32_1023x997x515"])
@pytest.mark.parametrize("variant", F32_VARIANTS, ids=lambda v: VNAME[v])
def test_f32_ragged(name, variant):
    c = inputs.CASES[name]
    A, B = inputs.operands_for(c)
    C64, _ = oracle.gemm(A, B)
    C, ok = gpu_gemm(A, B, "f32", variant, guard_rows=1)
    check(C, C64, "f32", c.dist, c.K, ok, f"{name} {VNAME[variant]}")


def test_f32_3072_full():
    """The bench's workload, in the bench's launch configuration (typed entry point,
    packed strides), against the oracle on every element."""
    c = inputs.CASES["f32_3072"]
    A, B = inputs.operands_for(c)
    C, ok = gpu_gemm(A, B, "f32", entry="typed")
    C64, _ = oracle.gemm(A, B)
    check(C, C64, "f32", c.dist, c.K, ok, "f32_3072 auto")


@pytest.mark.parametrize("variant", [gb.VARIANT_LDS_TILED, gb.VARIANT_REGBLOCK],
                         ids=lambda v: VNAME[v])
def test_f32_3072_sampled(variant):
    c = inputs.CASES["f32_3072"]
    A, B = inputs.operands_for(c)
    C, ok = gpu_gemm(A, B, "f32", variant)
    rows = sample_rows(c.M, 96)
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B)
    check(C[rows], C64, "f32", c.dist, c.K, ok, f"f32_3072 {VNAME[variant]} sampled")


def test_f16_4096_full():
    """The bench's FP16 workload, in the bench's launch configuration (typed entry point,
    packed strides, the direct-to-LDS kernel), against the oracle on every element."""
    c = inputs.CASES["f16_4096"]
    A, B = inputs.operands_for(c)
    C, ok = gpu_gemm(A, B, "f16", entry="typed")
    C64, _ = oracle.gemm(A, B, "f16")
    check(C, C64, "f16", c.dist, c.K, ok, "f16_4096 auto")


SWEEP_FULL = (128, 256, 512, 1024)
SWEEP_SAMPLED = (2048, 4096, 8192)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", SWEEP_FULL + SWEEP_SAMPLED)
def test_sweep(dtype, n):
    A, B = inputs.make_operands(n, n, n, inputs.SWEEP_SEED, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype)
    if n in SWEEP_FULL:
        C64, _ = oracle.gemm(A, B, dtype)
        check(C, C64, dtype, "uniform", n, ok, f"sweep {dtype} n={n}")
    else:
        rows = sample_rows(n, 64 if n < 8192 else 24)
        C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype)
        check(C[rows], C64, dtype, "uniform", n, ok, f"sweep {dtype} n={n} sampled")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tall_skinny(dtype):
    A, B = inputs.make_operands(16384, 4096, 4096, inputs.SWEEP_SEED, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype)
    rows = sample_rows(16384, 32)
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype)
    check(C[rows], C64, dtype, "uniform", 4096, ok, f"tall-skinny {dtype} sampled")


# ------------------------------------------------------------ edges and contract

EDGE_SHAPES = [(1, 1, 1), (1, 77, 5), (77, 1, 5), (3, 5, 1), (33, 65, 17), (64, 64, 32),
               (65, 63, 33), (191, 193, 37), (129, 257, 200), (200, 130, 1), (17, 300, 999)]


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype,variant", case_params(), ids=lambda x: str(x))
def test_edge_shapes(shape, dtype, variant):
    M, N, K = shape
    A, B = inputs.make_operands(M, N, K, 21, "uniform", dtype)
    C64, _ = oracle.gemm(A, B, dtype)
    for pad, off in (((0, 0, 0), 0), ((5, 3, 1), 1), ((8, 8, 4), 0)):
        C, ok = gpu_gemm(A, B, dtype, variant, pad=pad, offset=off, guard_rows=2)
        check(C, C64, dtype, "uniform", K, ok, f"{shape} {dtype} {VNAME[variant]} pad={pad} off={off}")


@pytest.mark.parametrize("dtype,variant", case_params(), ids=lambda x: str(x))
def test_k_zero_writes_zero(dtype, variant):
    A = np.zeros((37, 0), inputs.to_storage(np.zeros(1, np.float32), dtype).dtype)
    B = np.zeros((0, 45), A.dtype)
    C, ok = gpu_gemm(A, B, dtype, variant, pad=(1, 0, 3))
    assert ok and np.all(C == 0) and not np.signbit(C).any()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_empty_m_or_n_is_noop(dtype):
    A, B = inputs.make_operands(0, 8, 8, 1, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, pad=(0, 0, 2))
    assert ok and C.shape == (0, 8)
    A, B = inputs.make_operands(8, 0, 8, 1, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, pad=(0, 0, 2))
    assert ok and C.shape == (8, 0)


@pytest.mark.parametrize("dtype,variant", case_params(), ids=lambda x: str(x))
def test_run_twice_bitwise(dtype, variant):
    A, B = inputs.make_operands(515, 389, 777, 31, "normal", dtype)
    C1, _ = gpu_gemm(A, B, dtype, variant)
    C2, _ = gpu_gemm(A, B, dtype, variant)
    assert np.array_equal(C1, C2)


@pytest.mark.parametrize("name", ["f32_1000", "f32_1023x997x515"])
def test_valu_families_agree_bitwise(name):
    """naive, LDS-tiled and register-blocked kernels each sum an element by fmaf in
    increasing k from +0.0, so they round identically."""
    A, B = inputs.operands_for(inputs.CASES[name])
    outs = [gpu_gemm(A, B, "f32", v)[0] for v in
            (gb.VARIANT_NAIVE, gb.VARIANT_LDS_TILED, gb.VARIANT_REGBLOCK)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_typed_entry_matches_auto_variant(dtype):
    A, B = inputs.make_operands(300, 260, 140, 8, "uniform", dtype)
    C1, _ = gpu_gemm(A, B, dtype, gb.VARIANT_AUTO)
    C2, _ = gpu_gemm(A, B, dtype, entry="typed")
    assert np.array_equal(C1, C2)


def test_non_default_stream():
    import torch
    s = torch.cuda.Stream()
    A, B = inputs.make_operands(700, 600, 500, 9, "uniform", "f32")
    C64, _ = oracle.gemm(A, B)
    with torch.cuda.stream(s):
        C, ok = gpu_gemm(A, B, "f32", stream=s)
    check(C, C64, "f32", "uniform", 500, ok, "side stream")


def test_invalid_args_with_device():
    import torch
    buf = torch.zeros(64, device="cuda")
    p = buf.data_ptr()
    assert gb.gemm_f32(4, 4, 8, p, 7, p, 4, p, 4, 0) == gb.ERR_INVALID_ARG
    assert gb.gemm_f32(4, 4, 4, 0, 4, p, 4, p, 4, 0) == gb.ERR_INVALID_ARG
    assert gb.gemm355_run_variant(gb.VARIANT_REGBLOCK, gb.F16, 4, 4, 4, p, 4, p, 4, p, 4, 0) \
        == gb.ERR_UNSUPPORTED


def test_torch_matmul_wrapper():
    import torch
    A, B = inputs.make_operands(129, 65, 33, 3, "uniform", "f32")
    out = gb.matmul(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda())
    C64, _ = oracle.gemm(A, B)
    check(out.cpu().numpy(), C64, "f32", "uniform", 33, True, "matmul wrapper")


# Whole-tile products of the 16-bit kernel at small sizes: K of 256 and 320 (the 64 x 64
# direct-to-LDS tile, the second past whole ring trips), 192 (three 64-wide k-steps on the
# register-staged tile) and a single k-step, rows that are not 16-byte aligned (register
# staging, 16-byte loads at element alignment), and a misaligned base; each with M, N
# multiples of the tile.
INTERIOR_CASES = [((512, 512, 256), (0, 0, 0), 0), ((512, 512, 320), (0, 0, 0), 0),
                  ((256, 256, 64), (0, 0, 0), 0), ((512, 256, 256), (1, 3, 0), 0),
                  ((256, 512, 128), (0, 0, 0), 1), ((1024, 768, 192), (8, 8, 8), 0)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", INTERIOR_CASES, ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}_off{c[2]}")
def test_h16_interior_instances(dtype, case):
    (M, N, K), pad, off = case
    A, B = inputs.make_operands(M, N, K, 41, "uniform", dtype)
    C64, _ = oracle.gemm(A, B, dtype)
    C, ok = gpu_gemm(A, B, dtype, gb.VARIANT_MFMA, pad=pad, offset=off, guard_rows=1)
    check(C, C64, dtype, "uniform", K, ok, f"interior {dtype} {M}x{N}x{K} pad={pad} off={off}")
    Ai, Bi = inputs.make_operands(M, N, K, 42, "int", dtype)
    _, C32 = oracle.gemm(Ai, Bi, dtype)
    Ci, ok = gpu_gemm(Ai, Bi, dtype, gb.VARIANT_MFMA, pad=pad, offset=off)
    assert ok and np.array_equal(Ci, C32)


# Interior 256 x 256 tiles with K a multiple of 128 run the direct-to-LDS kernel (the
# cost model picks 256 x 256 tiles from about 2800^2 outputs): the shortest K (4
# k-steps, one trip of the ring), 12 k-steps on a non-square grid, padded
# 16-byte-aligned strides, and a long K.
DMA_CASES = [((3072, 3072, 128), (0, 0, 0)), ((2816, 3072, 384), (0, 0, 0)),
             ((3072, 2816, 256), (8, 16, 8)), ((3072, 3072, 2048), (0, 0, 0))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", DMA_CASES, ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}")
def test_h16_dma_instances(dtype, case):
    (M, N, K), pad = case
    A, B = inputs.make_operands(M, N, K, 44, "uniform", dtype)
    code = gb.DTYPE_CODES[dtype]
    lda, ldb, ldc = K + pad[0], N + pad[1], N + pad[2]
    P = 1 << 20  # any 16-byte-aligned non-null address: the query only inspects it
    assert "lds-dma" in gb.gemm355_kernel_desc(gb.VARIANT_MFMA, code, M, N, K, P, lda, P, ldb, P, ldc)
    C64, _ = oracle.gemm(A, B, dtype)
    C, ok = gpu_gemm(A, B, dtype, gb.VARIANT_MFMA, pad=pad, guard_rows=1)
    check(C, C64, dtype, "uniform", K, ok, f"dma {dtype} {M}x{N}x{K} pad={pad}")
    Ai, Bi = inputs.make_operands(M, N, K, 45, "int", dtype)
    _, C32 = oracle.gemm(Ai, Bi, dtype)
    Ci, ok = gpu_gemm(Ai, Bi, dtype, gb.VARIANT_MFMA, pad=pad)
    assert ok and np.array_equal(Ci, C32)


# 128 x 128 tiles on the direct-to-LDS kernel (one round of at most 256 interior tiles,
# when the cost model prefers 128-wide tiles and plain products have 256 tiles or more;
# K a multiple of 256, one trip of its 8-stage ring): the shortest K, padded
# 16-byte-aligned strides on a non-square grid, and a long K.
DMA128_CASES = [((2048, 2048, 256), (0, 0, 0)), ((4096, 1024, 512), (8, 16, 8)),
                ((1024, 4096, 2048), (0, 0, 0))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", DMA128_CASES, ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}")
def test_h16_dma128_instances(dtype, case):
    (M, N, K), pad = case
    A, B = inputs.make_operands(M, N, K, 47, "uniform", dtype)
    code = gb.DTYPE_CODES[dtype]
    lda, ldb, ldc = K + pad[0], N + pad[1], N + pad[2]
    P = 1 << 20
    assert "128x128x32 w2x2 lds-dma" in gb.gemm355_kernel_desc(gb.VARIANT_MFMA, code, M, N, K, P, lda, P, ldb, P, ldc)
    rows = np.array(sorted(set(sample_rows(M, 192).tolist()) | {127, 128, M - 1}))
    C, ok = gpu_gemm(A, B, dtype, gb.VARIANT_MFMA, pad=pad, guard_rows=1)
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype)
    check(C[rows], C64, dtype, "uniform", K, ok, f"dma128 {dtype} {M}x{N}x{K} pad={pad} sampled")
    Ai, Bi = inputs.make_operands(M, N, K, 48, "int", dtype)
    _, C32 = oracle.gemm(np.ascontiguousarray(Ai[rows]), Bi, dtype)
    Ci, ok = gpu_gemm(Ai, Bi, dtype, gb.VARIANT_MFMA, pad=pad)
    assert ok and np.array_equal(Ci[rows], C32)


def test_h16_dma128_ragged():
    """2040 x 2000: 16 x 16 tiles of 128, the last row of tiles 120 high and the last
    column 80 wide, every tile on the direct-to-LDS kernel; rows sampled from both
    regions."""
    M, N, K = 2040, 2000, 256
    A, B = inputs.make_operands(M, N, K, 49, "uniform", "f16")
    P = 1 << 20
    assert "128x128x32 w2x2 lds-dma" in gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.F16, M, N, K, P, K, P, N, P, N)
    C, ok = gpu_gemm(A, B, "f16", entry="typed", guard_rows=1)
    rows = np.array(sorted(set(sample_rows(M, 64).tolist()) | {1919, 1920, 2039}))
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, "f16")
    check(C[rows], C64, "f16", "uniform", K, ok, "dma128 ragged f16 2040x2000x256 sampled")


def test_h16_dma_interior_with_edges():
    """4000^2: 16 x 16 tiles of 256 on the direct-to-LDS kernel, the last row and column
    of tiles 160 wide (their loads clamped to the matrix, their stores guarded); rows
    sampled from both regions."""
    M = N = 4000
    K = 256
    A, B = inputs.make_operands(M, N, K, 46, "uniform", "bf16")
    P = 1 << 20
    assert "lds-dma" in gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.BF16, M, N, K, P, K, P, N, P, N)
    C, ok = gpu_gemm(A, B, "bf16", entry="typed", guard_rows=1)
    rows = np.array(sorted(set(sample_rows(M, 48).tolist()) | {3839, 3840, 3999}))
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, "bf16")
    check(C[rows], C64, "bf16", "uniform", K, ok, "dma+edge bf16 4000x4000x256 sampled")


# Ragged tiles of the register-staged 16-bit kernel with clamped loads (each chunk read
# from inside the matrix and shifted / zeroed when staged to LDS): an n-contiguous extent
# that is not a multiple of 8 (one launch over every tile), rows that are not 16-byte
# aligned with K ragged by a non-multiple of 8, odd strides, and more tiles than CUs
# (interior launch, then the ragged strips).  512 x 768 x 200 (whole tiles, K ragged by
# a multiple of 8, aligned rows) keeps the predicated loads.
# Each case states the launches it must get (the kernel description names them): one
# clamped launch over every tile with the two-set pipeline (an even number of 64-wide
# k-steps: 4, 16) or with one set (5), an interior launch followed by the clamped strips
# (a single k-step: one set; two k-steps with 16-byte-aligned padded rows: buffer loads and
# the two-set pipeline in both launches), and the predicated strips.
CLAMP_CASES = [((4000, 4004, 256), (0, 0, 0), "all", "all=clamped,paired"),
               ((1000, 1000, 1000), (1, 0, 0), "all", "edges=clamped,paired"),
               ((777, 1030, 301), (3, 5, 0), "all", "edges=clamped"),
               ((8000, 8004, 64), (0, 0, 0), "rows", "interior=pointer edges=clamped"),
               ((8000, 8004, 128), (0, 4, 4), "rows", "interior=buffer,paired edges=clamped,paired"),
               ((512, 768, 120), (0, 0, 0), "all", "edges=predicated")]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", CLAMP_CASES, ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}{c[1][1]}")
def test_h16_clamped_ragged(dtype, case):
    (M, N, K), pad, cmp, launches = case
    P = 1 << 20  # a 16-byte-aligned address: the query only inspects it
    desc = gb.gemm355_kernel_desc(gb.VARIANT_MFMA, gb.DTYPE_CODES[dtype], M, N, K, P, K + pad[0],
                                  P, N + pad[1], P, N + pad[2])
    assert desc.endswith("| " + launches), desc
    A, B = inputs.make_operands(M, N, K, 47, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, gb.VARIANT_MFMA, pad=pad, guard_rows=1)
    rows = np.arange(M) if cmp == "all" else np.array(sorted(
        set(sample_rows(M, 48).tolist()) | {M - 65, M - 64, M - 1}))
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype)
    check(C[rows], C64, dtype, "uniform", K, ok, f"clamped {dtype} {M}x{N}x{K} pad={pad}")
    if cmp == "all":
        Ai, Bi = inputs.make_operands(M, N, K, 48, "int", dtype)
        _, C32 = oracle.gemm(Ai, Bi, dtype)
        Ci, ok = gpu_gemm(Ai, Bi, dtype, gb.VARIANT_MFMA, pad=pad)
        assert ok and np.array_equal(Ci, C32)


# FP32 with rows that are not 16-byte aligned and ragged M and N, in one launch: with K a
# multiple of 4 and N of 4 the unpredicated kernel takes every tile with dword loads at
# clamped coordinates (1000 x 1000 x 1024, 4000^3 and 3000 x 3000 x 3008 sampled; K not a
# multiple of 32, the last k-step zero-filled: 1000^3, 3000 x 2996 x 2996 sampled); with N
# not a multiple of 4, when every tile fits in two rounds, the predicated kernel takes the
# interior tiles too (700 x 650 x 96).
@pytest.mark.parametrize("case", [((1000, 1000, 1024), (1, 0, 0)), ((700, 650, 96), (1, 3, 0)),
                                  ((4000, 4000, 4000), (1, 1, 0)), ((3000, 3000, 3008), (1, 1, 1)),
                                  ((1000, 1000, 1000), (1, 1, 0)), ((3000, 2996, 2996), (3, 1, 2))],
                         ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}{c[1][1]}")
def test_f32_ragged_one_launch(case):
    (M, N, K), pad = case
    A, B = inputs.make_operands(M, N, K, 49, "uniform", "f32")
    C, ok = gpu_gemm(A, B, "f32", gb.VARIANT_MFMA, pad=pad, guard_rows=1)
    rows = np.arange(M) if M * N * K <= 1 << 30 else np.array(
        sorted(set(sample_rows(M, 48).tolist()) | {M - 1, M - 2, (M // 128) * 128 - 1, (M // 192) * 192}))
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, "f32")
    check(C[rows], C64, "f32", "uniform", K, ok, f"one-launch f32 {M}x{N}x{K} pad={pad}")
    Ai, Bi = inputs.make_operands(M, N, K, 50, "int", "f32")
    _, C32 = oracle.gemm(np.ascontiguousarray(Ai[rows]), Bi, "f32")
    Ci, ok = gpu_gemm(Ai, Bi, "f32", gb.VARIANT_MFMA, pad=pad)
    assert ok and np.array_equal(Ci[rows], C32)


@pytest.mark.parametrize("case", [(384, 384, 64), (768, 384, 96), (384, 576, 3072)],
                         ids=lambda c: "x".join(map(str, c)))
def test_f32_interior_instances(case):
    M, N, K = case
    A, B = inputs.make_operands(M, N, K, 43, "uniform", "f32")
    C64, _ = oracle.gemm(A, B)
    C, ok = gpu_gemm(A, B, "f32", gb.VARIANT_MFMA, guard_rows=1)
    check(C, C64, "f32", "uniform", K, ok, f"interior f32 {M}x{N}x{K}")


# Every FP32 tile class the picker chooses, interior and predicated: 192 (3072^2), 128 with
# 2 x 4 waves (2048^2), 96 with 1 x 3 waves (1536^2; K tail; ragged M, N and K), 64.
F32_TILE_CASES = [((1536, 1536, 128), "96x96"), ((1536, 1536, 100), "96x96"),
                  ((1351, 1537, 100), "96x96"), ((2048, 2048, 96), "128x128"),
                  ((2000, 2048, 64), "128x128"), ((1024, 1024, 64), "64x64")]


# FP32 shapes whose ragged tiles run in the unpredicated kernel with the full tiles
# (aligned rows, N a multiple of 4, K a multiple of 32 or, with a zero-filled last
# k-step, of 4): loads clamped to the matrix, stores guarded; NaN padding around the
# operands would show in a stored output.
F32_RAGGED_CASES = [((4000, 4000, 512), (4, 8, 4), "128x128"), ((2000, 1996, 256), (0, 0, 0), "128x128"),
                    ((3000, 3000, 320), (0, 4, 0), "192x192"),
                    # K not a multiple of 32 (but of 4): the last k-step zero-filled
                    ((3000, 3000, 3000), (0, 0, 0), "192x192"), ((1000, 1000, 1000), (4, 4, 0), "64x64"),
                    ((2048, 2048, 1028), (8, 0, 4), "128x128")]


@pytest.mark.parametrize("case", F32_RAGGED_CASES, ids=lambda c: "x".join(map(str, c[0])))
def test_f32_ragged_all_tiles(case):
    (M, N, K), pad, tile = case
    lda, ldb, ldc = K + pad[0], N + pad[1], N + pad[2]
    P = 1 << 20
    desc = gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.F32, M, N, K, P, lda, P, ldb, P, ldc)
    assert tile in desc and desc.endswith("dwordx4"), desc
    A, B = inputs.make_operands(M, N, K, 61, "uniform", "f32")
    C, ok = gpu_gemm(A, B, "f32", entry="typed", pad=pad, guard_rows=1)
    rows = np.array(sorted(set(sample_rows(M, 96).tolist()) | {M - 1, M - 2, (M // 128) * 128 - 1}))
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B)
    check(C[rows], C64, "f32", "uniform", K, ok, f"f32 ragged all tiles {M}x{N}x{K} sampled")
    Ai, Bi = inputs.make_operands(M, N, K, 62, "int", "f32")
    _, C32 = oracle.gemm(np.ascontiguousarray(Ai[rows]), Bi)
    Ci, ok = gpu_gemm(Ai, Bi, "f32", entry="typed", pad=pad)
    assert ok and np.array_equal(Ci[rows], C32)


@pytest.mark.parametrize("case", F32_TILE_CASES, ids=lambda c: "x".join(map(str, c[0])))
def test_f32_tile_classes(case):
    (M, N, K), tile = case
    P = 1 << 20  # any 16-byte-aligned non-null address: the query only inspects it
    if tile is not None:
        assert tile in gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.F32, M, N, K, P, K, P, N, P, N)
    A, B = inputs.make_operands(M, N, K, 44, "uniform", "f32")
    C, ok = gpu_gemm(A, B, "f32", entry="typed", guard_rows=1)
    rows = sample_rows(M, 96)
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B)
    check(C[rows], C64, "f32", "uniform", K, ok, f"f32 tile class {tile} {M}x{N}x{K}")


# FP16/BF16 tile classes of plain products: 64 x 64 (the 128 x 64 tiling would still leave
# CUs idle) register-staged (K below 128, not a multiple of 8, rows not 16-byte aligned, or
# a plain product with K of 128 or 192; interior, ragged, K tail) and direct-to-LDS
# (8-stage ring, and the 4-stage one for other K from 128 to 255), 128 x 64 register-staged
# (the 128 x 128 tiling would leave CUs idle; interior and ragged), 128 x 128 direct-to-LDS
# on the 4-stage ring, 256 x 256 direct-to-LDS.
H16_TILE_CASES = [("f16", (1024, 1024, 120), "64x64x64 w1x2"), ("f16", (1024, 1024, 256), "64x64x32 w2x2 lds-dma"),
                  ("f16", (1024, 1024, 128), "64x64x64 w1x2"), ("f16", (1024, 1024, 136), "64x64x32 w2x2 lds-dma ring4"),
                  ("bf16", (1000, 900, 200), "64x64x64 w1x2"),
                  ("f16", (512, 512, 100), "64x64x64 w1x2"), ("bf16", (1536, 1536, 120), "128x64x64"),
                  ("bf16", (1536, 1536, 128), "128x64x64"), ("bf16", (1536, 1536, 200), "128x128x32 w2x2 lds-dma ring4"),
                  ("f16", (1500, 1450, 200), "128x64x64"), ("bf16", (2048, 2048, 128), "128x128"),
                  ("f16", (3072, 3072, 128), "lds-dma")]


@pytest.mark.parametrize("case", H16_TILE_CASES, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])))
def test_h16_tile_classes(case):
    dtype, (M, N, K), tile = case
    P = 1 << 20  # any 16-byte-aligned non-null address: the query only inspects it
    assert tile in gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], M, N, K, P, K, P, N, P, N)
    A, B = inputs.make_operands(M, N, K, 45, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, entry="typed", guard_rows=1)
    rows = sample_rows(M, 96)
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype)
    check(C[rows], C64, dtype, "uniform", K, ok, f"{dtype} tile class {tile} {M}x{N}x{K}")

# The 192 x 256 direct-to-LDS tile (plain products whose 256 x 256 grid would leave CUs
# idle: 3072^2 takes 192 tiles instead of 144): whole tiles, ragged M (3000 = 15 x 192 +
# 120) and ragged N (3000 = 11 x 256 + 184) with NaN-padded strides, K not a whole number
# of ring trips, and three rounds of tiles.
RECT_CASES = [("f16", (3072, 3072, 3072), (0, 0, 0), "full", "192x256x32 w2x2 lds-dma"),
              ("bf16", (3000, 3072, 1024), (8, 8, 8), "full", "192x256x32 w2x2 lds-dma"),
              ("f16", (3072, 3000, 512), (8, 8, 0), "full", "192x256x32 w2x2 lds-dma"),
              ("f16", (3072, 3072, 1000), (8, 0, 0), "rows", "192x256x32 w2x2 lds-dma k-zero-fill"),
              ("bf16", (6144, 6144, 512), (0, 0, 0), "rows", "192x256x32 w2x2 lds-dma")]


@pytest.mark.parametrize("case", RECT_CASES, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])) + f"_pad{c[2][0]}")
def test_dma_rect_tile(case):
    dtype, (M, N, K), pad, cmp, kernel = case
    P = 1 << 20  # a 16-byte-aligned address: the query only inspects it
    desc = gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], M, N, K, P, K + pad[0],
                                  P, N + pad[1], P, N + pad[2])
    assert desc.endswith(kernel), desc
    A, B = inputs.make_operands(M, N, K, 83, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, entry="typed", pad=pad, guard_rows=1)
    rows = np.arange(M) if cmp == "full" else np.array(sorted(
        set(sample_rows(M, 48).tolist()) | {191, 192, M - 1}))
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype)
    check(C[rows], C64, dtype, "uniform", K, ok, f"192x256 dma {dtype} {M}x{N}x{K} pad={pad}")
    Ai, Bi = inputs.make_operands(M, N, K, 84, "int", dtype)
    _, C32 = oracle.gemm(np.ascontiguousarray(Ai[rows]), Bi, dtype)
    Ci, ok = gpu_gemm(Ai, Bi, dtype, entry="typed", pad=pad)
    assert ok and np.array_equal(Ci[rows], C32), f"192x256 dma {dtype} {M}x{N}x{K} integers not bit-exact"


# The 128 x 128 direct-to-LDS tile with a 4-stage ring, two workgroups per CU (grids of
# more than 256 128-wide tiles): whole tiles with K a whole number of trips, exactly two
# tiles per CU, and ragged M and N (2500 = 19 x 128 + 68, 2600 = 20 x 128 + 40) with
# NaN-padded strides and K not a whole number of trips (1000 = 7 x 128 + 104).
RING4_CASES = [("f16", (2304, 2304, 512), (0, 0, 0), "mfma_f16 128x128x32 w2x2 lds-dma ring4"),
               ("bf16", (2048, 4096, 256), (0, 0, 0), "mfma_bf16 128x128x32 w2x2 lds-dma ring4"),
               ("bf16", (2500, 2600, 1000), (8, 8, 8), "mfma_bf16 128x128x32 w2x2 lds-dma ring4 k-zero-fill"),
               # one workgroup per CU with K from 128 to 255 (136 = 128 + 8)
               ("f16", (2048, 2048, 136), (8, 8, 8), "mfma_f16 128x128x32 w2x2 lds-dma ring4 k-zero-fill")]


@pytest.mark.parametrize("case", RING4_CASES, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])) + f"_pad{c[2][0]}")
def test_dma_128_two_per_cu(case):
    dtype, (M, N, K), pad, kernel = case
    P = 1 << 20  # a 16-byte-aligned address: the query only inspects it
    desc = gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], M, N, K, P, K + pad[0],
                                  P, N + pad[1], P, N + pad[2])
    assert desc == kernel, desc
    A, B = inputs.make_operands(M, N, K, 85, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, entry="typed", pad=pad, guard_rows=1)
    C64, _ = oracle.gemm(A, B, dtype)
    check(C, C64, dtype, "uniform", K, ok, f"128 ring4 dma {dtype} {M}x{N}x{K} pad={pad}")
    Ai, Bi = inputs.make_operands(M, N, K, 86, "int", dtype)
    _, C32 = oracle.gemm(Ai, Bi, dtype)
    Ci, ok = gpu_gemm(Ai, Bi, dtype, entry="typed", pad=pad)
    assert ok and np.array_equal(Ci, C32), f"128 ring4 dma {dtype} {M}x{N}x{K} integers not bit-exact"


# The 64 x 64 direct-to-LDS tile (plain products whose 128 x 64 grid would leave CUs idle,
# K a multiple of 8 and at least one 256-deep ring trip): a single tile, whole tiles, ragged
# M (1000 = 15 x 64 + 40) and N (904 = 14 x 64 + 8: a last tile one 16-byte chunk wide)
# with NaN-padded strides and K not a whole number of trips (1000 = 3 x 256 + 232, 264 =
# 256 + 8), a deep K (4096), and K from 128 to 255 on the 4-stage ring (136 = 128 + 8,
# and 200 = 128 + 72 on ragged tiles).
DMA64_CASES = [("f16", (64, 64, 256), (0, 0, 0), "mfma_f16 64x64x32 w2x2 lds-dma"),
               ("f16", (1024, 1024, 1024), (0, 0, 0), "mfma_f16 64x64x32 w2x2 lds-dma"),
               ("bf16", (1000, 904, 1000), (8, 8, 8), "mfma_bf16 64x64x32 w2x2 lds-dma k-zero-fill"),
               ("bf16", (512, 512, 264), (8, 0, 8), "mfma_bf16 64x64x32 w2x2 lds-dma k-zero-fill"),
               ("f16", (520, 1000, 4096), (0, 8, 0), "mfma_f16 64x64x32 w2x2 lds-dma"),
               ("f16", (512, 512, 136), (0, 0, 0), "mfma_f16 64x64x32 w2x2 lds-dma ring4 k-zero-fill"),
               ("bf16", (1000, 904, 200), (8, 8, 8), "mfma_bf16 64x64x32 w2x2 lds-dma ring4 k-zero-fill")]


@pytest.mark.parametrize("case", DMA64_CASES, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])) + f"_pad{c[2][0]}")
def test_dma_64_tile(case):
    dtype, (M, N, K), pad, kernel = case
    P = 1 << 20  # a 16-byte-aligned address: the query only inspects it
    desc = gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], M, N, K, P, K + pad[0],
                                  P, N + pad[1], P, N + pad[2])
    assert desc == kernel, desc
    A, B = inputs.make_operands(M, N, K, 87, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, entry="typed", pad=pad, guard_rows=1)
    C64, _ = oracle.gemm(A, B, dtype)
    check(C, C64, dtype, "uniform", K, ok, f"64 dma {dtype} {M}x{N}x{K} pad={pad}")
    Ai, Bi = inputs.make_operands(M, N, K, 88, "int", dtype)
    _, C32 = oracle.gemm(Ai, Bi, dtype)
    Ci, ok = gpu_gemm(Ai, Bi, dtype, entry="typed", pad=pad)
    assert ok and np.array_equal(Ci, C32), f"64 dma {dtype} {M}x{N}x{K} integers not bit-exact"


# The direct-to-LDS kernel with K not a whole number of its ring trips (128 for 256-wide
# tiles, 256 for 128-wide ones): the loop runs to the next trip and every 16-byte chunk at
# k >= K loads as zeros.  K = 4000, 4064 (ragged by whole 32-wide k-steps), 4072 (a
# partial last k-step), K just over one trip (136), the 128-wide tile (2000), and ragged
# tiles with ragged K (4000 x 4000 x 1000).  Padded strides hold NaN past K in every row,
# so any chunk past K that is read instead of zero-filled poisons the result.
RAGGED_K_CASES = [("bf16", (4096, 4096, 4000), (0, 0, 0), "full"),
                  ("f16", (4096, 4096, 4064), (8, 8, 8), "rows"),
                  ("bf16", (4096, 4096, 4072), (8, 16, 8), "rows"),
                  ("f16", (3072, 2816, 136), (8, 8, 8), "full"),
                  ("bf16", (2048, 2048, 2000), (8, 8, 0), "full"),
                  ("f16", (4000, 4000, 1000), (8, 0, 0), "rows"),
                  ("bf16", (4096, 4096, 4104), (0, 0, 0), "rows"),
                  ("f16", (2048, 2048, 1800), (8, 8, 8), "full"),
                  ("f16", (2048, 2048, 264), (0, 0, 0), "full")]
# The ring runs whole trips of 4 (256 x 256 tile) or 8 (128 x 128) 32-wide k-steps, and
# the k-steps of the last trip that lie wholly past K are skipped: K = 4000 skips 3 of its
# last trip's 4, 4064 one, 4072 none (its last step is part zeros), 4104 three; 2000, 1800
# and 264 skip 1, 7 and 7 of 8 (264: one plain trip, then a trip with a single live step).


@pytest.mark.parametrize("case", RAGGED_K_CASES, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])) + f"_pad{c[2][0]}")
def test_dma_ragged_k(case):
    dtype, (M, N, K), pad, cmp = case
    P = 1 << 20  # a 16-byte-aligned address: the query only inspects it
    desc = gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], M, N, K, P, K + pad[0],
                                  P, N + pad[1], P, N + pad[2])
    assert "lds-dma k-zero-fill" in desc, desc
    A, B = inputs.make_operands(M, N, K, 81, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, entry="typed", pad=pad, guard_rows=1)
    rows = np.arange(M) if cmp == "full" else np.array(sorted(
        set(sample_rows(M, 48).tolist()) | {255, 256, M - 1}))
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype)
    check(C[rows], C64, dtype, "uniform", K, ok, f"ragged-K dma {dtype} {M}x{N}x{K} pad={pad}")
    Ai, Bi = inputs.make_operands(M, N, K, 82, "int", dtype)
    _, C32 = oracle.gemm(np.ascontiguousarray(Ai[rows]), Bi, dtype)
    Ci, ok = gpu_gemm(Ai, Bi, dtype, entry="typed", pad=pad)
    assert ok and np.array_equal(Ci[rows], C32), f"ragged-K dma {dtype} {M}x{N}x{K} integers not bit-exact"

