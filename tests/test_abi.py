"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects invalid arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from roofline_optimisation_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h)
           for h in ("gemm355.h", "gemm355_probe.h", "gemm355_stream.h", "gemm355_softmax.h")]


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.append(m.group(1))
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gb.LIB_PATH):
        pytest.fail("libgemm355.so is not built (run __graft_entry__.build())")
    return gb.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    raw = ctypes.CDLL(gb.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"{n} declared but not exported"
    assert set(names) == set(gb.EXPORTS)


def test_version_and_strings(lib):
    assert gb.gemm355_version() == 100
    assert gb.gemm355_status_string(0) == "ok"
    assert gb.gemm355_status_string(1) == "invalid argument"
    assert gb.gemm355_status_string(99) == "unknown"
    assert [gb.gemm355_variant_name(v) for v in (-1, 0, 1, 2, 3, 10)] == \
        ["auto", "naive", "lds_tiled", "regblock", "mfma", "unknown"]


P = 1 << 20  # a fake, 16-byte aligned "device" address; never dereferenced


@pytest.mark.parametrize("args", [
    (-1, 4, 4, P, 4, P, 4, P, 4),        # negative M
    (4, -1, 4, P, 4, P, 4, P, 4),        # negative N
    (4, 4, -1, P, 4, P, 4, P, 4),        # negative K
    (4, 4, 8, P, 7, P, 4, P, 4),         # lda < K
    (4, 8, 4, P, 4, P, 7, P, 8),         # ldb < N
    (4, 8, 4, P, 4, P, 8, P, 7),         # ldc < N
    (4, 4, 4, 0, 4, P, 4, P, 4),         # null A
    (4, 4, 4, P, 4, 0, 4, P, 4),         # null B
    (4, 4, 4, P, 4, P, 4, 0, 4),         # null C
    (4, 4, 0, P, 0, P, 4, P, 4),         # lda must be >= 1 even when K = 0
])
def test_invalid_arguments_rejected_on_host(lib, args):
    for f in (gb.gemm_f32, gb.gemm_f16f32acc, gb.gemm_bf16f32acc):
        assert f(*args, 0) == gb.ERR_INVALID_ARG
    for v in (-1, 0, 3):
        assert gb.gemm355_run_variant(v, 0, *args, 0) == gb.ERR_INVALID_ARG
    assert gb.gemm355_select_variant(0, *args) == -1
    assert gb.gemm355_kernel_desc(-1, 0, *args) == "invalid"


def test_unknown_variant_and_dtype(lib):
    args = (4, 4, 4, P, 4, P, 4, P, 4, 0)
    assert gb.gemm355_run_variant(10, 0, *args) == gb.ERR_INVALID_ARG
    assert gb.gemm355_run_variant(-2, 0, *args) == gb.ERR_INVALID_ARG
    assert gb.gemm355_run_variant(0, 3, *args) == gb.ERR_INVALID_ARG
    # FP32-only families reject 16-bit operands before touching the device
    assert gb.gemm355_run_variant(gb.VARIANT_LDS_TILED, gb.F16, *args) == gb.ERR_UNSUPPORTED
    assert gb.gemm355_run_variant(gb.VARIANT_REGBLOCK, gb.BF16, *args) == gb.ERR_UNSUPPORTED


def test_degenerate_shapes_are_noops_without_device(lib):
    # M = 0 or N = 0: nothing to do, OK even with null pointers and no GPU
    assert gb.gemm_f32(0, 5, 5, 0, 5, P, 5, 0, 5, 0) == gb.OK
    assert gb.gemm_f32(5, 0, 5, P, 5, 0, 1, 0, 1, 0) == gb.OK
    assert gb.gemm_f16f32acc(0, 0, 0, 0, 1, 0, 1, 0, 1, 0) == gb.OK


def test_dispatch_choices(lib):
    d = lambda *a: gb.gemm355_kernel_desc(*a)
    assert gb.gemm355_select_variant(0, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == gb.VARIANT_MFMA
    assert d(-1, 0, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072).startswith("mfma_f32 192x192")
    assert d(-1, 0, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096).startswith("mfma_f32 128x128")
    assert d(-1, 1, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096).startswith("mfma_f16")
    assert d(-1, 2, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096).startswith("mfma_bf16")
    # 256 x 256 tiles with K a multiple of 8 and at least 128, and one round of 128 x 128
    # tiles with K a multiple of 8 and at least 256, load straight into LDS, ragged tiles
    # included; a K that is not a whole number of ring trips (128, 256) zero-fills the
    # chunks past K; other K, unaligned rows and more 128-wide tiles keep register staging
    assert d(-1, 1, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == "mfma_f16 256x256x32 w2x2 lds-dma"
    assert d(-1, 2, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == "mfma_bf16 256x256x32 w2x2 lds-dma"
    assert d(-1, 1, 4096, 4096, 4160, P, 4160, P, 4096, P, 4096) == "mfma_f16 256x256x32 w2x2 lds-dma k-zero-fill"
    assert d(-1, 1, 4096, 4096, 4096, P + 2, 4096, P, 4096, P, 4096) == "mfma_f16 256x256x64 w2x2 dwordx4 unaligned | interior=pointer"
    assert d(-1, 1, 2048, 2048, 2048, P, 2048, P, 2048, P, 2048) == "mfma_f16 128x128x32 w2x2 lds-dma"
    assert d(-1, 1, 2048, 2048, 2176, P, 2176, P, 2048, P, 2048) == "mfma_f16 128x128x32 w2x2 lds-dma k-zero-fill"
    # more than 256 128-wide tiles: the 4-stage ring, two workgroups per CU; K below its
    # trip (128) stays staged
    assert d(-1, 2, 2560, 2560, 2560, P, 2560, P, 2560, P, 2560) == "mfma_bf16 128x128x32 w2x2 lds-dma ring4"
    assert d(-1, 1, 2560, 2560, 1000, P, 1000, P, 2560, P, 2560) == \
        "mfma_f16 128x128x32 w2x2 lds-dma ring4 k-zero-fill"
    assert d(-1, 1, 2560, 2560, 120, P, 120, P, 2560, P, 2560).startswith("mfma_f16 128x128x64 w2x2 dwordx4")
    assert d(-1, 1, 4000, 4000, 4096, P, 4096, P, 4000, P, 4000) == "mfma_f16 256x256x32 w2x2 lds-dma"
    # 192 x 256 tiles where the 256 x 256 grid would take more 256-CU rounds of work per
    # CU: 3072^2 (144 tiles against 192), 4096 x 4104 (272 tiles, two rounds, against 374),
    # 4608^2; not at 4096^2 or 8192^2, whose 256 x 256 tiles fill whole rounds, nor for the
    # transposed A or the other epilogues
    assert d(-1, 1, 4096, 4104, 4096, P, 4096, P, 4104, P, 4104) == "mfma_f16 192x256x32 w2x2 lds-dma"
    assert d(-1, 1, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == "mfma_f16 192x256x32 w2x2 lds-dma"
    assert d(-1, 2, 3072, 3072, 1000, P, 1000, P, 3072, P, 3072) == "mfma_bf16 192x256x32 w2x2 lds-dma k-zero-fill"
    assert d(-1, 1, 4608, 4608, 4608, P, 4608, P, 4608, P, 4608) == "mfma_f16 192x256x32 w2x2 lds-dma"
    assert d(-1, 2, 8192, 8192, 8192, P, 8192, P, 8192, P, 8192) == "mfma_bf16 256x256x32 w2x2 lds-dma"
    assert d(-1, 1, 5120, 5120, 5120, P, 5120, P, 5120, P, 5120) == "mfma_f16 256x256x32 w2x2 lds-dma"
    assert d(-1, 2, 4096, 4096, 4000, P, 4000, P, 4096, P, 4096) == "mfma_bf16 256x256x32 w2x2 lds-dma k-zero-fill"
    assert d(-1, 2, 4096, 4096, 4001, P, 4008, P, 4096, P, 4096) == "mfma_bf16 256x256x64 w2x2 dwordx4 | edges=clamped"
    assert d(-1, 1, 4096, 4096, 120, P, 120, P, 4096, P, 4096).startswith("mfma_f16 256x256x64 w2x2 dwordx4")
    # an m/n-contiguous extent that is not a whole number of 16-byte chunks stays staged
    assert d(-1, 1, 4000, 4004, 4096, P, 4096, P, 4008, P, 4004) == "mfma_f16 256x256x64 w2x2 dwordx4 | all=clamped,paired"
    # rows not 16-byte aligned (lda = 515 floats) take the dword load path
    assert d(-1, 0, 1023, 997, 515, P, 515, P, 997, P, 997).endswith("dword")
    assert d(-1, 0, 1000, 1000, 1000, P, 1000, P, 1000, P, 1000).endswith("dwordx4")
    assert d(-1, 0, 1000, 1000, 1000, P + 4, 1000, P, 1000, P, 1000).endswith("dword")
    assert d(0, 1, 8, 8, 8, P, 8, P, 8, P, 8).startswith("naive")
    assert d(1, 0, 8, 8, 8, P, 8, P, 8, P, 8).startswith("lds_tiled")
    assert d(2, 0, 8, 8, 8, P, 8, P, 8, P, 8).startswith("regblock")
    assert d(1, 1, 8, 8, 8, P, 8, P, 8, P, 8) == "invalid"
    # the register-staged 16-bit kernel's launches: the interior launch with an odd number
    # of 64-wide k-steps (4160 / 64 = 65) runs one staging set, with an even number the
    # two-set pipeline; ragged strips with clamped loads
    assert d(-1, 1, 8000, 8004, 128, P, 128, P, 8008, P, 8004) == \
        "mfma_f16 256x256x64 w2x2 dwordx4 | interior=buffer,paired edges=clamped,paired"
    assert d(-1, 1, 8000, 8004, 192, P, 192, P, 8008, P, 8004) == \
        "mfma_f16 256x256x64 w2x2 dwordx4 | interior=buffer edges=clamped"


def test_dispatch_choices_general_form(lib):
    dx = lambda *a: gb.gemm355_kernel_desc_ex(*a)
    # flag-free equals the plain query
    assert dx(-1, 1, 0, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == \
        gb.gemm355_kernel_desc(-1, 1, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096)
    # transposed operands with K ragged and not a multiple of 8 (1004 = 15 64-wide k-steps
    # + 44): every tile takes the clamped kernel; 16 k-steps (even) run the two-set
    # pipeline
    assert dx(-1, 1, gb.TRANS_A, 1000, 1000, 1004, P, 1000, P, 1000, P, 1000) == \
        "mfma_f16 128x128x64 w2x2 dwordx4 | edges=clamped,paired"
    assert dx(-1, 2, gb.TRANS_B, 1000, 1000, 1004, P, 1004, P, 1004, P, 1000) == \
        "mfma_bf16 64x64x64 w1x2 dwordx4 unaligned | edges=clamped,paired"
    # signed and accumulating epilogues keep to one staging set
    assert dx(-1, 1, gb.TRANS_A | gb.NEG_A, 1000, 1000, 1004, P, 1000, P, 1000, P, 1000) == \
        "mfma_f16 128x128x64 w2x2 dwordx4 | edges=clamped"
    # with K a multiple of 8 the direct-to-LDS kernel zero-fills past K in every layout
    assert dx(-1, 1, gb.TRANS_A | gb.TRANS_B, 1000, 1000, 1000, P, 1000, P, 1000, P, 1000) == \
        "mfma_f16 64x64x32 w2x2 lds-dma k-zero-fill"
    # the 64 x 64 direct-to-LDS tile: any layout and epilogue where the 128 x 128 grid leaves
    # CUs idle and the 64 x 64 one holds at most 512 tiles (beyond, the 128 x 128
    # direct-to-LDS tile, plain products included); register staging below K = 256
    assert dx(-1, 2, gb.TRANS_A | gb.ACCUMULATE, 1024, 1024, 1024, P, 1024, P, 1024, P, 1024) == \
        "mfma_bf16 64x64x32 w2x2 lds-dma"
    assert dx(-1, 1, gb.C_16 | gb.NEG_B, 768, 768, 1024, P, 1024, P, 768, P, 768) == \
        "mfma_f16 64x64x32 w2x2 lds-dma"
    assert dx(-1, 2, 0, 1400, 1400, 1000, P, 1000, P, 1400, P, 1400) == \
        "mfma_bf16 64x64x32 w2x2 lds-dma k-zero-fill"
    assert dx(-1, 2, 0, 1500, 1456, 1000, P, 1000, P, 1456, P, 1456) == \
        "mfma_bf16 128x128x32 w2x2 lds-dma k-zero-fill"
    assert dx(-1, 1, gb.TRANS_A, 1536, 1536, 1536, P, 1536, P, 1536, P, 1536) == \
        "mfma_f16 128x128x32 w2x2 lds-dma"
    assert dx(-1, 1, gb.TRANS_A, 1792, 1792, 1792, P, 1792, P, 1792, P, 1792) == \
        "mfma_f16 128x128x32 w2x2 lds-dma"
    assert dx(-1, 1, 0, 1792, 1792, 1792, P, 1792, P, 1792, P, 1792) == "mfma_f16 128x128x32 w2x2 lds-dma"
    # K from 128 to 255 on the 4-stage ring, but for plain products with K of 128 or 192; the
    # register-staged 128 x 64 and 64 x 64 tiles where the direct-to-LDS one does not run
    assert dx(-1, 1, 0, 1792, 1792, 200, P, 200, P, 1792, P, 1792) == \
        "mfma_f16 128x128x32 w2x2 lds-dma ring4 k-zero-fill"
    assert dx(-1, 2, gb.TRANS_A, 1024, 1024, 128, P, 1024, P, 1024, P, 1024) == "mfma_bf16 64x64x32 w2x2 lds-dma ring4"
    assert dx(-1, 1, 0, 1792, 1792, 100, P, 100, P, 1792, P, 1792).startswith("mfma_f16 128x64x64")
    assert dx(-1, 1, gb.TRANS_B, 1024, 1024, 120, P, 120, P, 120, P, 1024).startswith("mfma_f16 64x64x64 w1x2")
    assert dx(-1, 2, 0, 2048, 2048, 128, P, 128, P, 2048, P, 2048).startswith("mfma_bf16 128x128x64 w2x2 dwordx4")
    assert dx(-1, 2, 0, 2048, 4096, 128, P, 128, P, 4096, P, 4096) == "mfma_bf16 128x128x32 w2x2 lds-dma ring4"
    assert dx(-1, 2, gb.ACCUMULATE, 2048, 2048, 192, P, 192, P, 2048, P, 2048) == \
        "mfma_bf16 128x128x32 w2x2 lds-dma ring4 k-zero-fill"
    assert dx(-1, 1, gb.TRANS_A, 1024, 1024, 120, P, 1024, P, 1024, P, 1024).startswith("mfma_f16 128x128x64")
    # the 192 x 256 and 256 x 192 tiles take every layout (an m/n-contiguous operand of
    # extent 192 in LDS rows of 24 chunks) and every epilogue (signed, accumulating, 16-bit
    # C); between equal grids the one whose 192 side is k-contiguous wins, then 192 x 256
    assert dx(-1, 1, gb.TRANS_B, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == \
        "mfma_f16 192x256x32 w2x2 lds-dma"
    assert dx(-1, 1, gb.TRANS_A, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == \
        "mfma_f16 192x256x32 w2x2 lds-dma"
    assert dx(-1, 2, gb.NEG_A, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == \
        "mfma_bf16 192x256x32 w2x2 lds-dma"
    assert dx(-1, 1, gb.TRANS_B | gb.ACCUMULATE, 3072, 3072, 1000, P, 1000, P, 1000, P, 3072) == \
        "mfma_f16 192x256x32 w2x2 lds-dma k-zero-fill"
    assert dx(-1, 2, gb.C_16 | gb.NEG_B, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == \
        "mfma_bf16 192x256x32 w2x2 lds-dma"
    assert dx(-1, 1, gb.TRANS_A | gb.TRANS_B, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == \
        "mfma_f16 256x192x32 w2x2 lds-dma"
    # 4096 x 3072: 192 tiles of 256 x 256, 264 of 192 x 256 (two rounds), 256 of 256 x 192
    assert dx(-1, 1, gb.TRANS_B, 4096, 3072, 4096, P, 4096, P, 4096, P, 3072) == \
        "mfma_f16 256x192x32 w2x2 lds-dma"
    assert dx(-1, 1, 0, 4096, 3072, 4096, P, 4096, P, 3072, P, 3072) == "mfma_f16 256x192x32 w2x2 lds-dma"
    assert dx(-1, 2, gb.TRANS_A, 4096, 3072, 4096, P, 4096, P, 3072, P, 3072) == "mfma_bf16 256x192x32 w2x2 lds-dma"
    assert dx(-1, 2, gb.TRANS_A | gb.TRANS_B | gb.ACCUMULATE, 3000, 3000, 1000, P, 3000, P, 1000, P, 3000) == \
        "mfma_bf16 256x192x32 w2x2 lds-dma k-zero-fill"
    # what gemm355_gemm_ex rejects
    assert dx(-1, 0, gb.C_16, 8, 8, 8, P, 8, P, 8, P, 8) == "invalid"
    assert dx(-1, 1, 64, 8, 8, 8, P, 8, P, 8, P, 8) == "invalid"
    assert dx(gb.VARIANT_LDS_TILED, 0, gb.TRANS_A, 8, 8, 8, P, 8, P, 8, P, 8) == "invalid"
    assert dx(-1, 1, gb.TRANS_A, 8, 8, 8, P, 4, P, 8, P, 8) == "invalid"


def test_no_device_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert gb.gemm_f32(4, 4, 4, P, 4, P, 4, P, 4, 0) == gb.ERR_DEVICE


def test_probe_argument_checks(lib):
    assert gb.gemm355_probe_mfma_shape(0) == (1, 16)
    assert gb.gemm355_probe_mfma_shape(3) == (8, 4)
    with pytest.raises(ValueError):
        gb.gemm355_probe_mfma_shape(6)
    assert gb.gemm355_probe_mfma(6, 1, P, P, P) == gb.ERR_INVALID_ARG
    assert gb.gemm355_probe_mfma(0, 0, P, P, P) == gb.ERR_INVALID_ARG
    assert gb.gemm355_probe_ds_read_tr16([8 * i for i in range(63)] + [4], P) == gb.ERR_INVALID_ARG
    assert gb.gemm355_probe_ds_read_tr16([8 * i for i in range(63)] + [4096], P) == gb.ERR_INVALID_ARG


def test_gemm_ex_argument_checks(lib):
    E = gb.gemm355_gemm_ex
    # M=8, N=6, K=4: stored A is 8 x 4 (or 4 x 8 transposed), B 4 x 6 (or 6 x 4)
    assert E(0, 0, 64, 8, 6, 4, P, 4, P, 6, P, 6) == gb.ERR_INVALID_ARG          # unknown flag
    assert E(0, 0, gb.C_16, 8, 6, 4, P, 4, P, 6, P, 6) == gb.ERR_INVALID_ARG     # 16-bit C, FP32 in
    for dt in (gb.F16, gb.BF16):                                                  # 16-bit C, 16-bit in
        assert E(-1, dt, gb.C_16 | gb.ACCUMULATE, 8, 6, 4, P, 4, P, 6, P, 6) in (gb.OK, gb.ERR_DEVICE)
    assert E(0, 0, gb.TRANS_A, 8, 6, 4, P, 4, P, 6, P, 6) == gb.ERR_INVALID_ARG  # lda < M
    assert E(0, 0, gb.TRANS_B, 8, 6, 4, P, 4, P, 2, P, 6) == gb.ERR_INVALID_ARG  # ldb < K
    assert E(0, 0, 0, 8, 6, 4, P, 3, P, 6, P, 6) == gb.ERR_INVALID_ARG           # lda < K
    assert E(0, 0, 0, 8, 6, 4, P, 4, P, 6, P, 5) == gb.ERR_INVALID_ARG           # ldc < N
    assert E(0, 3, 0, 8, 6, 4, P, 4, P, 6, P, 6) == gb.ERR_INVALID_ARG           # dtype
    assert E(10, 0, 0, 8, 6, 4, P, 4, P, 6, P, 6) == gb.ERR_INVALID_ARG          # variant
    assert E(0, 0, 0, 8, 6, 4, 0, 4, P, 6, P, 6) == gb.ERR_INVALID_ARG           # null A
    # with a flag only the naive and MFMA families exist
    for v in (gb.VARIANT_LDS_TILED, gb.VARIANT_REGBLOCK):
        assert E(v, 0, gb.NEG_A, 8, 6, 4, P, 4, P, 6, P, 6) == gb.ERR_UNSUPPORTED
    # valid arguments reach the device check (no GPU here) or run
    for f in (0, gb.TRANS_A, gb.TRANS_B, gb.TRANS_A | gb.TRANS_B | gb.NEG_A | gb.ACCUMULATE):
        lda = 8 if f & gb.TRANS_A else 4
        ldb = 4 if f & gb.TRANS_B else 6
        assert E(-1, 0, f, 8, 6, 4, P, lda, P, ldb, P, 6) in (gb.OK, gb.ERR_DEVICE)
    assert E(-1, 0, gb.ACCUMULATE, 0, 6, 4, P, 4, P, 6, P, 6) == gb.OK            # M = 0


def test_stream_and_chase_argument_checks(lib):
    ok = dict(mode=gb.STREAM_COPY, src=P, dst=P + (1 << 20), n_bytes=4096, vec_bytes=16, unroll=4,
              threads=256, lds_bytes=0, grid=256)
    def st(**kw):
        a = dict(ok, **kw)
        return gb.gemm355_stream(a["mode"], a["src"], a["dst"], a["n_bytes"], a["vec_bytes"],
                                 a["unroll"], a["threads"], a["lds_bytes"], a["grid"])
    bad = [dict(mode=3), dict(mode=-1), dict(n_bytes=-4), dict(n_bytes=6), dict(vec_bytes=12), dict(unroll=3),
           dict(threads=32), dict(threads=96), dict(threads=2048), dict(lds_bytes=-1),
           dict(lds_bytes=163841), dict(grid=0), dict(grid=(1 << 20) + 1), dict(src=0),
           dict(dst=0), dict(src=P + 4), dict(dst=P + 8 + (1 << 20)),
           dict(dst=P + 1024),                      # overlaps the source
           dict(mode=gb.STREAM_READ_XOR, dst=0), dict(mode=gb.STREAM_READ_XOR, dst=P + 2),
           dict(mode=gb.STREAM_COPY_NT, dst=P + 1024), dict(mode=gb.STREAM_COPY_NT, src=0)]
    for b in bad:
        assert st(**b) == gb.ERR_INVALID_ARG, b
    # an empty copy needs no buffers; a READ_XOR always writes its grid entries
    assert st(n_bytes=0, src=0, dst=0) in (gb.OK, gb.ERR_DEVICE)
    C = gb.gemm355_chase
    assert C(0, 16, 0, 1, P) == gb.ERR_INVALID_ARG
    assert C(P, 16, 0, 1, 0) == gb.ERR_INVALID_ARG
    assert C(P, 0, 0, 1, P) == gb.ERR_INVALID_ARG
    assert C(P, (1 << 32) + 1, 0, 1, P) == gb.ERR_INVALID_ARG
    assert C(P, 16, 16, 1, P) == gb.ERR_INVALID_ARG
    assert C(P, 16, 0, 0, P) == gb.ERR_INVALID_ARG
    assert C(P, 16, 0, (1 << 30) + 1, P) == gb.ERR_INVALID_ARG


def test_softmax_and_row_sum_argument_checks(lib):
    S, R = gb.gemm355_softmax_f32, gb.gemm355_row_sum_f32
    Q = P + (1 << 24)
    bad = [(-1, 4, P, 4, Q, 4), (2, -1, P, 4, Q, 4), (2, 4, P, 3, Q, 4), (2, 4, P, 4, Q, 3),
           (2, (1 << 30) + 1, P, (1 << 30) + 1, Q, (1 << 30) + 1), ((1 << 30) + 1, 4, P, 4, Q, 4),
           (2, 4, 0, 4, Q, 4),
           (2, 4, P, 4, 0, 4),
           (2, 4, P, 8, P, 4),            # in place with different strides
           (4, 64, P, 64, P + 256, 64)]   # partial overlap
    for b in bad:
        assert S(*b) == gb.ERR_INVALID_ARG, b
    assert S(0, 4, 0, 4, 0, 4) == gb.OK and S(3, 0, 0, 1, 0, 1) == gb.OK   # no-ops
    assert S(2, 4, P, 4, P, 4) in (gb.OK, gb.ERR_DEVICE)                   # in place
    assert S(2, 4, P, 4, P + 32, 4) in (gb.OK, gb.ERR_DEVICE)              # adjacent spans
    bad = [(-1, 4, P, 4, Q), (2, -1, P, 4, Q), (2, 4, P, 3, Q), (2, 4, 0, 4, Q), (2, 4, P, 4, 0),
           ((1 << 30) + 1, 4, P, 4, Q),
           (2, 4, P, 4, P + 16)]          # out overlaps X
    for b in bad:
        assert R(*b) == gb.ERR_INVALID_ARG, b
    assert R(0, 4, 0, 4, 0) == gb.OK
    assert R(3, 0, 0, 1, Q) in (gb.OK, gb.ERR_DEVICE)                      # writes zeros


def test_matmul_refuses_cpu_tensors(lib):
    import torch
    a = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        gb.matmul(a, a)


def test_schedule_variants_contract(lib):
    """The measurement-only schedules take plain F16/BF16 products of whole tiles with
    16-byte-aligned rows and K a multiple of 128; anything else is UNSUPPORTED (checked on
    the host, before any HIP call)."""
    d = gb.gemm355_kernel_desc
    for v in (gb.VARIANT_MFMA_SPLIT, gb.VARIANT_MFMA_W8, gb.VARIANT_MFMA_T256X128):
        assert "lds-dma" in d(v, gb.F16, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096)
        assert "mfma_bf16" in d(v, gb.BF16, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096)
        assert d(v, gb.F32, 4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == "invalid"
        assert d(v, gb.F16, 4096, 4096, 4000, P, 4000, P, 4096, P, 4096) == "invalid"  # K % 128
        assert d(v, gb.F16, 4000, 4096, 4096, P, 4096, P, 4096, P, 4096) == "invalid"  # M % 256
        assert d(v, gb.F16, 4096, 4096, 4096, P + 2, 4096, P, 4096, P, 4096) == "invalid"
        assert gb.gemm355_run_variant(v, gb.F32, 256, 256, 128, P, 128, P, 256, P, 256, 0) == gb.ERR_UNSUPPORTED
        assert gb.gemm355_run_variant(v, gb.F16, 256, 256, 100, P, 100, P, 256, P, 256, 0) == gb.ERR_UNSUPPORTED
        assert gb.gemm355_gemm_ex(v, gb.F16, gb.TRANS_A, 256, 256, 128, P, 256, P, 256, P, 256, 0) == gb.ERR_UNSUPPORTED
        assert gb.gemm355_variant_name(v).startswith("mfma_")
    assert d(gb.VARIANT_MFMA_W8, gb.F16, 512, 512, 128, P, 128, P, 512, P, 512) == "mfma_f16 256x256x32 w2x4 lds-dma"
    assert d(gb.VARIANT_MFMA_T256X128, gb.F16, 512, 384, 128, P, 128, P, 384, P, 384) == "mfma_f16 256x128x32 w2x2 lds-dma"
    assert d(gb.VARIANT_MFMA_SPLIT, gb.F16, 512, 384, 128, P, 128, P, 384, P, 384) == \
        "mfma_f16 256x128x32 w2x2 + 4 producer waves lds-dma"
    assert d(gb.VARIANT_MFMA_W8, gb.F16, 512, 384, 128, P, 128, P, 384, P, 384) == "invalid"  # N % 256
    assert gb.gemm355_run_variant(10, gb.F16, 8, 8, 8, P, 8, P, 8, P, 8, 0) == gb.ERR_INVALID_ARG


def test_square_tile_variant_contract(lib):
    """MFMA_T256X256 is the dispatcher with the 192 x 256 and 256 x 192 tiles turned off:
    every F16 / BF16 product (general form included), as dispatched except that 256 x 256
    replaces them."""
    d = gb.gemm355_kernel_desc
    v = gb.VARIANT_MFMA_T256X256
    assert gb.gemm355_variant_name(v) == "mfma_t256x256"
    assert d(-1, gb.F16, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == "mfma_f16 192x256x32 w2x2 lds-dma"
    assert d(v, gb.F16, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == "mfma_f16 256x256x32 w2x2 lds-dma"
    assert d(v, gb.BF16, 3072, 3072, 1000, P, 1000, P, 3072, P, 3072) == \
        "mfma_bf16 256x256x32 w2x2 lds-dma k-zero-fill"
    for shape in ((4096, 4096, 4096), (2048, 2048, 2048), (1000, 1000, 1004), (300, 260, 130)):
        M, N, K = shape
        for dt in (gb.F16, gb.BF16):
            assert d(v, dt, M, N, K, P, K, P, N, P, N) == d(-1, dt, M, N, K, P, K, P, N, P, N)
    assert d(v, gb.F32, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == "invalid"
    assert gb.gemm355_run_variant(v, gb.F32, 256, 256, 128, P, 128, P, 256, P, 256, 0) == gb.ERR_UNSUPPORTED
    # the general form too: 256 x 256 where the dispatcher takes 192 x 256
    dx = gb.gemm355_kernel_desc_ex
    for fl in (gb.TRANS_B, gb.NEG_A | gb.ACCUMULATE, gb.C_16):
        assert dx(-1, gb.F16, fl, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072).startswith("mfma_f16 192x256x32")
        assert dx(v, gb.F16, fl, 3072, 3072, 3072, P, 3072, P, 3072, P, 3072) == "mfma_f16 256x256x32 w2x2 lds-dma"
    assert dx(v, gb.BF16, gb.TRANS_A, 1000, 1000, 1004, P, 1000, P, 1000, P, 1000) == \
        dx(-1, gb.BF16, gb.TRANS_A, 1000, 1000, 1004, P, 1000, P, 1000, P, 1000)
    assert dx(v, gb.F32, gb.TRANS_B, 256, 256, 128, P, 128, P, 128, P, 256) == "invalid"


def test_staged128_variant_contract(lib):
    """MFMA_STAGED128 is the dispatcher with the two-per-CU 128 x 128 direct-to-LDS tile
    turned off: grids of more than 256 128-wide tiles go to the register-staged kernel,
    every other F16 / BF16 call (general form included) as dispatched."""
    d = gb.gemm355_kernel_desc
    dx = gb.gemm355_kernel_desc_ex
    v = gb.VARIANT_MFMA_STAGED128
    assert gb.gemm355_variant_name(v) == "mfma_staged128"
    assert d(v, gb.BF16, 2560, 2560, 2560, P, 2560, P, 2560, P, 2560) == \
        "mfma_bf16 128x128x64 w2x2 dwordx4 | interior=buffer,paired"
    assert dx(v, gb.F16, gb.TRANS_A, 2560, 2048, 192, P, 2560, P, 2048, P, 2048) == \
        "mfma_f16 128x128x64 w2x2 dwordx4 | interior=buffer"
    assert dx(-1, gb.F16, gb.TRANS_A, 2560, 2048, 192, P, 2560, P, 2048, P, 2048) == \
        "mfma_f16 128x128x32 w2x2 lds-dma ring4 k-zero-fill"
    for shape in ((4096, 4096, 4096), (3072, 3072, 3072), (2048, 2048, 2048), (1000, 1000, 1004), (300, 260, 130)):
        M, N, K = shape
        for dt in (gb.F16, gb.BF16):
            assert d(v, dt, M, N, K, P, K, P, N, P, N) == d(-1, dt, M, N, K, P, K, P, N, P, N)
    assert d(v, gb.F32, 2560, 2560, 2560, P, 2560, P, 2560, P, 2560) == "invalid"
    assert gb.gemm355_run_variant(v, gb.F32, 256, 256, 128, P, 128, P, 256, P, 256, 0) == gb.ERR_UNSUPPORTED


def test_staged_small_variant_contract(lib):
    """MFMA_STAGED_SMALL is the dispatcher with the direct-to-LDS tiles of small grids turned
    off: no 64 x 64 direct-to-LDS tile, no 4-stage ring for K from 128 to 255 where the
    8-stage one would run, plain products on the register-staged 128 x 64 / 64 x 64 tiles
    where the 128 x 128 grid leaves CUs idle; every other F16 / BF16 call as dispatched."""
    d = gb.gemm355_kernel_desc
    dx = gb.gemm355_kernel_desc_ex
    v = gb.VARIANT_MFMA_STAGED_SMALL
    assert gb.gemm355_variant_name(v) == "mfma_staged_small"
    assert d(-1, gb.BF16, 1024, 1024, 1024, P, 1024, P, 1024, P, 1024) == "mfma_bf16 64x64x32 w2x2 lds-dma"
    assert d(v, gb.BF16, 1024, 1024, 1024, P, 1024, P, 1024, P, 1024) == \
        "mfma_bf16 64x64x64 w1x2 dwordx4 | interior=buffer,paired"
    assert d(v, gb.F16, 1536, 1536, 1536, P, 1536, P, 1536, P, 1536).startswith("mfma_f16 128x64x64 w2x2 dwordx4")
    assert dx(v, gb.F16, gb.TRANS_A, 1024, 1024, 1024, P, 1024, P, 1024, P, 1024) == \
        "mfma_f16 128x128x32 w2x2 lds-dma"
    assert dx(v, gb.F16, gb.TRANS_A, 1024, 1024, 200, P, 1024, P, 1024, P, 1024).startswith(
        "mfma_f16 128x128x64 w2x2 dwordx4")
    # two per CU on the 4-stage ring, and the larger tiles, as dispatched
    for shape in ((4096, 4096, 4096), (3072, 3072, 3072), (2048, 4096, 128), (2560, 2560, 2560), (1000, 1000, 1004)):
        M, N, K = shape
        for dt in (gb.F16, gb.BF16):
            assert d(v, dt, M, N, K, P, K, P, N, P, N) == d(-1, dt, M, N, K, P, K, P, N, P, N)
    assert d(v, gb.F32, 1024, 1024, 1024, P, 1024, P, 1024, P, 1024) == "invalid"
    assert gb.gemm355_run_variant(v, gb.F32, 256, 256, 128, P, 128, P, 256, P, 256, 0) == gb.ERR_UNSUPPORTED
