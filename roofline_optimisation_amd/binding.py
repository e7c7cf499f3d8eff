"""ctypes binding of libgemm355 (argument marshalling only).

The functions named like the C entry points take plain integers (device pointers as
ints, a stream handle as an int) and return the C status code.  ``matmul``, ``softmax``
and ``row_sum`` are convenience wrappers for torch tensors that derive sizes, strides,
pointers and the current stream, call the C entry point and raise on a non-OK status.
Nothing here computes any part of the results: every step runs in the HIP kernels of
``libgemm355.so``.  If the library is missing or cannot be loaded, every call raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgemm355.so")

OK, ERR_INVALID_ARG, ERR_DEVICE, ERR_LAUNCH, ERR_UNSUPPORTED = 0, 1, 2, 3, 4
F32, F16, BF16 = 0, 1, 2
VARIANT_AUTO, VARIANT_NAIVE, VARIANT_LDS_TILED, VARIANT_REGBLOCK, VARIANT_MFMA = -1, 0, 1, 2, 3
# measurement-only schedules of the FP16/BF16 direct-to-LDS kernel (plain products)
VARIANT_MFMA_SPLIT, VARIANT_MFMA_W8, VARIANT_MFMA_T256X128 = 4, 5, 6
# measurement only: the dispatched kernels without the 192 x 256 and 256 x 192 tiles,
# without the two-per-CU 128 x 128 direct-to-LDS tile, or without the direct-to-LDS tiles
# of small grids
VARIANT_MFMA_T256X256, VARIANT_MFMA_STAGED128, VARIANT_MFMA_STAGED_SMALL = 7, 8, 9
VARIANTS = {"naive": VARIANT_NAIVE, "lds_tiled": VARIANT_LDS_TILED,
            "regblock": VARIANT_REGBLOCK, "mfma": VARIANT_MFMA, "auto": VARIANT_AUTO,
            "mfma_split": VARIANT_MFMA_SPLIT, "mfma_w8": VARIANT_MFMA_W8,
            "mfma_t256x128": VARIANT_MFMA_T256X128, "mfma_t256x256": VARIANT_MFMA_T256X256,
            "mfma_staged128": VARIANT_MFMA_STAGED128, "mfma_staged_small": VARIANT_MFMA_STAGED_SMALL}
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16}
TRANS_A, TRANS_B, NEG_A, NEG_B, ACCUMULATE, C_16 = 1, 2, 4, 8, 16, 32

# Every symbol the public headers declare.
EXPORTS = (
    "gemm_f32", "gemm_f16f32acc", "gemm_bf16f32acc", "gemm355_run_variant",
    "gemm355_select_variant", "gemm355_kernel_desc", "gemm355_kernel_desc_ex",
    "gemm355_status_string",
    "gemm355_variant_name", "gemm355_version", "gemm355_gemm_ex",
    "gemm355_probe_mfma_shape", "gemm355_probe_mfma", "gemm355_probe_ds_read_tr16",
    "gemm355_probe_global_load_lds", "gemm355_stream", "gemm355_chase",
    "gemm355_softmax_f32", "gemm355_row_sum_f32",
)

STREAM_COPY, STREAM_READ_XOR, STREAM_COPY_NT = 0, 1, 2


class Gemm355Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def _configure(lib):
    i, p, s = ctypes.c_int, ctypes.c_void_p, ctypes.c_char_p
    gemm_args = [i, i, i, p, i, p, i, p, i, p]
    for name in ("gemm_f32", "gemm_f16f32acc", "gemm_bf16f32acc"):
        f = getattr(lib, name)
        f.argtypes = gemm_args
        f.restype = i
    lib.gemm355_run_variant.argtypes = [i, i] + gemm_args
    lib.gemm355_run_variant.restype = i
    lib.gemm355_gemm_ex.argtypes = [i, i, ctypes.c_uint] + gemm_args
    lib.gemm355_gemm_ex.restype = i
    lib.gemm355_select_variant.argtypes = [i, i, i, i, p, i, p, i, p, i]
    lib.gemm355_select_variant.restype = i
    lib.gemm355_kernel_desc.argtypes = [i, i, i, i, i, p, i, p, i, p, i]
    lib.gemm355_kernel_desc.restype = s
    lib.gemm355_kernel_desc_ex.argtypes = [i, i, ctypes.c_uint, i, i, i, p, i, p, i, p, i]
    lib.gemm355_kernel_desc_ex.restype = s
    lib.gemm355_status_string.argtypes = [i]
    lib.gemm355_status_string.restype = s
    lib.gemm355_variant_name.argtypes = [i]
    lib.gemm355_variant_name.restype = s
    lib.gemm355_version.argtypes = []
    lib.gemm355_version.restype = i
    lib.gemm355_probe_mfma_shape.argtypes = [i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.gemm355_probe_mfma_shape.restype = i
    lib.gemm355_probe_mfma.argtypes = [i, i, p, p, p, p]
    lib.gemm355_probe_mfma.restype = i
    lib.gemm355_probe_ds_read_tr16.argtypes = [ctypes.POINTER(ctypes.c_uint32), p, p]
    lib.gemm355_probe_ds_read_tr16.restype = i
    lib.gemm355_probe_global_load_lds.argtypes = [p, ctypes.POINTER(ctypes.c_uint32),
                                                  ctypes.c_uint32, p, p]
    lib.gemm355_probe_global_load_lds.restype = i
    i64 = ctypes.c_int64
    lib.gemm355_stream.argtypes = [i, p, p, i64, i, i, i, i, i, p]
    lib.gemm355_stream.restype = i
    lib.gemm355_chase.argtypes = [p, i64, ctypes.c_uint32, i, p, p]
    lib.gemm355_chase.restype = i
    lib.gemm355_softmax_f32.argtypes = [i, i, p, i, p, i, p]
    lib.gemm355_softmax_f32.restype = i
    lib.gemm355_row_sum_f32.argtypes = [i, i, p, i, p, p]
    lib.gemm355_row_sum_f32.restype = i
    return lib


def lib():
    """The loaded ``libgemm355.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        _lib = _configure(ctypes.CDLL(LIB_PATH))
    return _lib


# ----------------------------------------------------------- C entry points

def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    return lib().gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f16f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    return lib().gemm_f16f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    return lib().gemm_bf16f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm355_run_variant(variant, dtype, M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    return lib().gemm355_run_variant(variant, dtype, M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm355_gemm_ex(variant, dtype, flags, M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    return lib().gemm355_gemm_ex(variant, dtype, flags, M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm355_select_variant(dtype, M, N, K, A, lda, B, ldb, C, ldc) -> int:
    return lib().gemm355_select_variant(dtype, M, N, K, A, lda, B, ldb, C, ldc)


def gemm355_kernel_desc(variant, dtype, M, N, K, A, lda, B, ldb, C, ldc) -> str:
    return lib().gemm355_kernel_desc(variant, dtype, M, N, K, A, lda, B, ldb, C, ldc).decode()


def gemm355_kernel_desc_ex(variant, dtype, flags, M, N, K, A, lda, B, ldb, C, ldc) -> str:
    return lib().gemm355_kernel_desc_ex(variant, dtype, flags, M, N, K, A, lda, B, ldb, C,
                                        ldc).decode()


def gemm355_status_string(status: int) -> str:
    return lib().gemm355_status_string(status).decode()


def gemm355_variant_name(variant: int) -> str:
    return lib().gemm355_variant_name(variant).decode()


def gemm355_version() -> int:
    return lib().gemm355_version()


def gemm355_probe_mfma_shape(kind: int) -> tuple[int, int]:
    e, r = ctypes.c_int(), ctypes.c_int()
    if lib().gemm355_probe_mfma_shape(kind, ctypes.byref(e), ctypes.byref(r)) != 0:
        raise ValueError(f"unknown probe kind {kind}")
    return e.value, r.value


def gemm355_probe_mfma(kind, nruns, dev_a, dev_b, dev_d, stream=0) -> int:
    return lib().gemm355_probe_mfma(kind, nruns, dev_a, dev_b, dev_d, stream)


def gemm355_probe_ds_read_tr16(host_addrs, dev_out, stream=0) -> int:
    arr = (ctypes.c_uint32 * 64)(*[int(a) for a in host_addrs])
    return lib().gemm355_probe_ds_read_tr16(arr, dev_out, stream)


def gemm355_probe_global_load_lds(dev_src, host_chunks, lds_base, dev_out, stream=0) -> int:
    arr = (ctypes.c_uint32 * 64)(*[int(c) for c in host_chunks])
    return lib().gemm355_probe_global_load_lds(dev_src, arr, int(lds_base), dev_out, stream)


def gemm355_stream(mode, src, dst, n_bytes, vec_bytes, unroll, threads, lds_bytes, grid,
                   stream=0) -> int:
    return lib().gemm355_stream(mode, src, dst, n_bytes, vec_bytes, unroll, threads, lds_bytes,
                                grid, stream)


def gemm355_chase(next_words, n_words, start, hops, dev_out, stream=0) -> int:
    return lib().gemm355_chase(next_words, n_words, start, hops, dev_out, stream)


def gemm355_softmax_f32(rows, cols, X, ldx, Y, ldy, stream=0) -> int:
    return lib().gemm355_softmax_f32(rows, cols, X, ldx, Y, ldy, stream)


def gemm355_row_sum_f32(rows, cols, X, ldx, out, stream=0) -> int:
    return lib().gemm355_row_sum_f32(rows, cols, X, ldx, out, stream)


def status_string(status: int) -> str:
    try:
        return gemm355_status_string(status)
    except Exception:  # library not loadable: still describe the code
        return {0: "ok", 1: "invalid argument", 2: "no gfx950 device", 3: "kernel launch failed",
                4: "variant not available for this dtype"}.get(status, "unknown")


# ----------------------------------------------------------- torch marshalling

def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride(1) == 1)")
    return max(int(t.stride(0)) if t.shape[0] > 1 else int(t.shape[1]), int(t.shape[1]), 1)


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported operand dtype {t.dtype}")
    return codes[t.dtype]


def matmul(A, B, out=None, variant: int | str = VARIANT_AUTO, stream=None, *,
           trans_a: bool = False, trans_b: bool = False, neg_a: bool = False,
           neg_b: bool = False, accumulate: bool = False):
    """C = (+-op(A)) (+-op(B)) [+ out] on the GPU through libgemm355.  A and B are the
    stored 2-D CUDA tensors (float32, float16 or bfloat16, rows contiguous): A is M x K,
    or K x M with trans_a; B is K x N, or N x K with trans_b.  The result is float32,
    or A's 16-bit type when `out` is given in that type (GEMM355_C_16); with accumulate,
    `out` (M x N) is added to and required.  Raises Gemm355Error on a non-OK status;
    never falls back to another implementation."""
    import torch
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("operands must be CUDA tensors")
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    M, K = (A.shape[1], A.shape[0]) if trans_a else tuple(A.shape)
    K2, N = (B.shape[1], B.shape[0]) if trans_b else tuple(B.shape)
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs `out`")
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    c16 = out.dtype != torch.float32
    if (c16 and (out.dtype != A.dtype or A.dtype == torch.float32)) or tuple(out.shape) != (M, N):
        raise ValueError("out must be an M x N tensor in float32 or in A's 16-bit type")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    handle = s.cuda_stream if hasattr(s, "cuda_stream") else int(s)
    flags = ((TRANS_A if trans_a else 0) | (TRANS_B if trans_b else 0) | (NEG_A if neg_a else 0)
             | (NEG_B if neg_b else 0) | (ACCUMULATE if accumulate else 0) | (C_16 if c16 else 0))
    if flags:
        st = gemm355_gemm_ex(variant, _dtype_code(A), flags, M, N, K, A.data_ptr(), _ld(A),
                             B.data_ptr(), _ld(B), out.data_ptr(), _ld(out), handle)
        where = "gemm355_gemm_ex"
    else:
        st = gemm355_run_variant(variant, _dtype_code(A), M, N, K, A.data_ptr(), _ld(A),
                                 B.data_ptr(), _ld(B), out.data_ptr(), _ld(out), handle)
        where = "gemm355_run_variant"
    if st != OK:
        raise Gemm355Error(st, where)
    return out


def _stream_handle(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def _f32_matrix(t, what):
    import torch
    if not t.is_cuda or t.dtype != torch.float32 or t.dim() != 2:
        raise ValueError(f"{what} must be a 2-D float32 CUDA tensor")


def softmax(X, out=None, stream=None):
    """Row-wise softmax of a 2-D float32 CUDA tensor through gemm355_softmax_f32 (`out`
    may be X itself for an in-place call).  Raises Gemm355Error on a non-OK status."""
    import torch
    _f32_matrix(X, "X")
    if out is None:
        out = torch.empty_like(X, memory_format=torch.contiguous_format)
    _f32_matrix(out, "out")
    if tuple(out.shape) != tuple(X.shape):
        raise ValueError("out must have X's shape")
    rows, cols = X.shape
    st = gemm355_softmax_f32(rows, cols, X.data_ptr(), _ld(X), out.data_ptr(), _ld(out),
                             _stream_handle(stream, X.device))
    if st != OK:
        raise Gemm355Error(st, "gemm355_softmax_f32")
    return out


def row_sum(X, out=None, stream=None):
    """Sums of the rows of a 2-D float32 CUDA tensor through gemm355_row_sum_f32."""
    import torch
    _f32_matrix(X, "X")
    rows, cols = X.shape
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=X.device)
    if not out.is_cuda or out.dtype != torch.float32 or out.numel() != rows or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 CUDA tensor of `rows` elements")
    st = gemm355_row_sum_f32(rows, cols, X.data_ptr(), _ld(X), out.data_ptr(),
                             _stream_handle(stream, X.device))
    if st != OK:
        raise Gemm355Error(st, "gemm355_row_sum_f32")
    return out
