"""GPU parity on operands larger than 2 GiB (the largest inputs the entry points take
with int32 sizes): the kernels address each tile of a k-contiguous operand from its own
64-bit base and keep every buffer offset within 31 bits, so

* an A of more than 2^31 bytes puts the bases of its later tiles past 2^31 bytes while
  each tile's offsets stay small (the direct-to-LDS and buffer-load kernels), and
* a B whose byte offsets from its first row reach past 2^31 (K x N x element size above
  2 GiB) makes the host fall back to pointer loads.

Checked on sampled rows (those whose first byte lies on either side of 2^31 included)
and, where B is the large operand, sampled columns, against the oracle on the same
rows and columns; same bars as the other parity tests.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import SENTINEL, errors, gpu_gemm, nan_fill, place, sample_rows, to_device, tolerance
from roofline_optimisation_amd import binding as gb
from roofline_optimisation_amd import inputs

pytestmark = pytest.mark.gpu

ESIZE = {"f32": 4, "f16": 2, "bf16": 2}

# dtype, (M, N, K), the operand above 2 GiB, a part of the kernel description it must get
LARGE_CASES = [
    ("f16", (131328, 512, 8192), "A", "256x256x32 w2x2 lds-dma"),      # A 2.15 GB
    ("f32", (140032, 256, 4096), "A", "mfma_f32 128x128x32"),          # A 2.29 GB
    ("f16", (256, 26624, 40960), "B", "| interior=pointer"),           # B 2.18 GB
    ("f32", (256, 33024, 16384), "B", "mfma_f32 64x64x32"),            # B 2.16 GB
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("case", LARGE_CASES,
                         ids=lambda c: f"{c[0]}_" + "x".join(map(str, c[1])) + f"_big{c[2]}")
def test_operand_over_2gib(case):
    dtype, (M, N, K), big, part = case
    es = ESIZE[dtype]
    assert (M * K if big == "A" else K * N) * es > 2 ** 31
    P = 1 << 20  # a 16-byte-aligned address: the query only inspects it
    desc = gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], M, N, K, P, K, P, N, P, N)
    assert part in desc, desc
    print(f"large {dtype} {M}x{N}x{K} ({big} above 2 GiB): {desc}", flush=True)
    A, B = inputs.make_operands(M, N, K, 61, "uniform", dtype)
    C, ok = gpu_gemm(A, B, dtype, entry="typed", guard_rows=1)
    assert ok, "wrote outside C"
    if big == "A":
        r0 = 2 ** 31 // (K * es)  # first row that starts at or past byte 2^31
        rows = np.array(sorted(set(sample_rows(M, 40, seed=1).tolist()) |
                               {r0 - 1, r0, r0 + 1, M - 1}))
        cols = np.arange(N)
    else:
        rows = sample_rows(M, 16, seed=2)
        cols = sample_rows(N, 64, seed=3)
    Ab = np.ascontiguousarray(A[rows])
    Bb = np.ascontiguousarray(B[:, cols])
    del A, B
    C64, _ = oracle.gemm(Ab, Bb, dtype)
    Cs = C[np.ix_(rows, cols)]
    assert not np.isnan(Cs).any(), "NaN in result (read outside the operands?)"
    rel, mx = errors(Cs, C64)
    trel, tabs = tolerance(dtype, "uniform", K)
    print(f"large {dtype} {M}x{N}x{K}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= trel and mx <= tabs, f"rel {rel:.3e} (<= {trel}), max {mx:.3e} (<= {tabs})"


# The general form (gemm355_gemm_ex) with the large operand transposed: A stored K x M
# (m-contiguous: its offsets pass 2^31, pointer loads) or B stored N x K (k-contiguous:
# its later tiles start past 2^31, on the buffer-load and direct-to-LDS kernels; the BF16
# case takes 256 x 192 tiles, 684 of them against 513 of 256 x 256, three rounds either
# way).  The
# stored matrices are drawn in their stored shape: A from default_rng(seed), B from
# default_rng(seed + 1).
EX_CASES = [
    ("f16", (26624, 256, 40960), "ta", "| interior=pointer"),          # stored A 2.18 GB
    ("f32", (256, 140032, 4096), "tb", "mfma_f32 128x128x32"),         # stored B 2.29 GB
    ("bf16", (256, 131328, 8192), "tb", "256x192x32 w2x2 lds-dma"),    # stored B 2.15 GB
]


@pytest.mark.parametrize("case", EX_CASES,
                         ids=lambda c: f"{c[0]}_" + "x".join(map(str, c[1])) + f"_{c[2]}")
def test_general_form_operand_over_2gib(case):
    import torch
    dtype, (M, N, K), t, part = case
    ta = t == "ta"
    flags = gb.TRANS_A if ta else gb.TRANS_B
    es = ESIZE[dtype]
    sa_shape = (K, M) if ta else (M, K)
    sb_shape = (K, N) if ta else (N, K)
    assert (M * K if ta else N * K) * es > 2 ** 31
    P = 1 << 20  # a 16-byte-aligned address: the query only inspects it
    desc = gb.gemm355_kernel_desc_ex(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], flags, M, N, K,
                                     P, sa_shape[1], P, sb_shape[1], P, N)
    assert part in desc, desc
    print(f"large general form {dtype} {M}x{N}x{K} {t}: {desc}", flush=True)
    SA = inputs.draw_rows(*sa_shape, 63, "uniform", dtype)
    SB = inputs.draw_rows(*sb_shape, 64, "uniform", dtype)
    dA = to_device(place(SA, sa_shape[1], 0, 1, nan_fill(dtype)))
    dB = to_device(place(SB, sb_shape[1], 0, 1, nan_fill(dtype)))
    dC = torch.full((M + 1, N), float(SENTINEL), dtype=torch.float32, device="cuda")
    st = gb.gemm355_gemm_ex(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], flags, M, N, K,
                            dA.data_ptr(), sa_shape[1], dB.data_ptr(), sb_shape[1],
                            dC.data_ptr(), N, torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK, st
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    del dA, dB, dC
    assert np.all(out[M] == SENTINEL), "wrote past C"
    C = out[:M]
    if ta:
        rows = sample_rows(M, 24, seed=4)
        cols = np.arange(N)
        C64, _ = oracle.gemm_ex(np.ascontiguousarray(SA[:, rows]), SB, dtype, True, False)
    else:
        n0 = 2 ** 31 // (K * es)  # first stored row of B that starts at or past byte 2^31
        rows = np.arange(M)
        cols = np.array(sorted(set(sample_rows(N, 40, seed=5).tolist()) | {n0 - 1, n0, n0 + 1}))
        C64, _ = oracle.gemm_ex(SA, np.ascontiguousarray(SB[cols]), dtype, False, True)
    Cs = C[np.ix_(rows, cols)]
    assert not np.isnan(Cs).any(), "NaN in result (read outside the operands?)"
    rel, mx = errors(Cs, C64)
    trel, tabs = tolerance(dtype, "uniform", K)
    print(f"large general form {dtype} {M}x{N}x{K} {t}: rel_frob={rel:.3e} max_abs={mx:.3e}",
          flush=True)
    assert rel <= trel and mx <= tabs, f"rel {rel:.3e} (<= {trel}), max {mx:.3e} (<= {tabs})"


# A C of more than 2^31 elements (8.6 GB of FP32): the epilogues index C in 64 bits.  C
# starts as NaN (an element left unwritten would show) with one guard row of the
# sentinel after it; sampled rows (the first row past element 2^31 included) are read
# back and compared with the oracle on the same rows.
C_CASES = [("f16", (65792, 32768, 128), "256x256x32 w2x2 lds-dma"),
           ("f32", (65792, 32768, 100), "mfma_f32 128x128x32")]   # K tail: 100 = 3 x 32 + 4


@pytest.mark.parametrize("case", C_CASES, ids=lambda c: f"{c[0]}_" + "x".join(map(str, c[1])))
def test_c_over_2g_elements(case):
    import torch
    dtype, (M, N, K), part = case
    assert M * N > 2 ** 31
    P = 1 << 20  # a 16-byte-aligned address: the query only inspects it
    desc = gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.DTYPE_CODES[dtype], M, N, K, P, K, P, N, P, N)
    assert part in desc, desc
    print(f"large C {dtype} {M}x{N}x{K}: {desc}", flush=True)
    A, B = inputs.make_operands(M, N, K, 65, "uniform", dtype)
    dA, dB = to_device(A), to_device(B)
    dC = torch.full((M + 1, N), float("nan"), dtype=torch.float32, device="cuda")
    dC[M] = float(SENTINEL)
    f = {"f32": gb.gemm_f32, "f16": gb.gemm_f16f32acc, "bf16": gb.gemm_bf16f32acc}[dtype]
    st = f(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
           torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK, st
    torch.cuda.synchronize()
    r0 = -(-2 ** 31 // N)  # first row whose elements all lie past element 2^31
    rows = np.array(sorted(set(sample_rows(M, 24, seed=6).tolist()) | {r0 - 1, r0, M - 1}))
    C = dC[torch.from_numpy(rows).cuda()].cpu().numpy()
    guard = dC[M].cpu().numpy()
    del dA, dB, dC
    assert np.all(guard == SENTINEL), "wrote past C"
    assert not np.isnan(C).any(), "an element of C was not written"
    C64, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype)
    rel, mx = errors(C, C64)
    trel, tabs = tolerance(dtype, "uniform", K)
    print(f"large C {dtype} {M}x{N}x{K}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= trel and mx <= tabs, f"rel {rel:.3e} (<= {trel}), max {mx:.3e} (<= {tabs})"
