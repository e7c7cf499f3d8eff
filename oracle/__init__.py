"""CPU oracle for the dense GEMM C = A.B (plain C, fp64 accumulation, i-k-j loop), and
for the memory-slope probes (XOR of a word stream, a dependent-index walk).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg may import this package.  It never imports the GPU
library and the GPU library never imports it.

The computation is the definition of the product on the pages ("Advanced CUDA
features - starting from GEMM", roofline section case (4); "Kernel optimisation
guide", Level 1; "GEMM kernels" memo, first kernel): C_ij = sum_k A_ik * B_kj.  All
arithmetic happens in ``oracle.c``; this module only marshals numpy arrays.

Pins (in ``tests/test_oracle.py``): a hand-worked product, identity and permutation
matrices, small-integer inputs against exact integer products, exact rational brute
force for every M, N, K in 1..8, the transpose identity, stride handling with
NaN-filled padding, the error bound against an independent binary64 matrix product,
exhaustive fp16/bf16 decoding against numpy, and planted mistakes that the pins catch.
``gemm_ex`` (transposed / negated operands, accumulation into C) is pinned in
``tests/test_oracle_ex.py``.  The probe functions (``stream_xor``, ``chase``; "Advanced CUDA features - starting from
GEMM", section on Little's law and occupancy) are pinned in ``tests/test_oracle_stream.py``:
the closed form of the XOR of 0..n-1, per-bit parity counts, successor and permutation
cycles with closed-form positions, and the out-of-range clamp.  ``softmax`` (the online
recurrence of "Kernel optimisation guide", section on softmax optimisation) and
``row_sum`` (its section on warp-shuffle reduction) are pinned in
``tests/test_oracle_softmax.py``: exact decimal arithmetic at 50 digits, closed forms
(constant rows, two-element rows), shift invariance, independence of rows and strides,
integer sums, and planted mistakes.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle355.so")

_lib = None


def _configure(lib):
    dp, fp, vp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i = ctypes.c_int
    for name in ("oracle_gemm_f32", "oracle_gemm_f16", "oracle_gemm_bf16"):
        f = getattr(lib, name)
        f.argtypes = [i, i, i, vp, i, vp, i, dp, fp, i]
        f.restype = i
    lib.oracle_gemm_f64.argtypes = [i, i, i, dp, i, dp, i, dp, fp, i]
    lib.oracle_gemm_f64.restype = i
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i
    lib.oracle_gemm_ex.argtypes = [i, i, i, i, i, i, i, i, i, vp, i, vp, i, vp, dp, fp, i]
    lib.oracle_gemm_ex.restype = i
    lib.oracle_xor_words.argtypes = [vp, ctypes.c_int64]
    lib.oracle_xor_words.restype = ctypes.c_uint32
    lib.oracle_chase.argtypes = [vp, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int64]
    lib.oracle_chase.restype = ctypes.c_uint32
    lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_f16.restype = ctypes.c_uint16
    lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_gemm_ex16.argtypes = [i, i, i, i, i, i, i, i, i, vp, i, vp, i, vp, dp, vp, i]
    lib.oracle_gemm_ex16.restype = i
    lib.oracle_softmax.argtypes = [i, i, vp, i, dp, fp, i, dp, dp]
    lib.oracle_softmax.restype = i
    lib.oracle_row_sum.argtypes = [i, i, vp, i, dp, fp]
    lib.oracle_row_sum.restype = i
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = _configure(ctypes.CDLL(LIB_PATH))
    return _lib


def load_library(path: str):
    """Load an oracle build from another path (used by the planted-mistake tests)."""
    return _configure(ctypes.CDLL(path))


def num_threads() -> int:
    return _load().oracle_num_threads()


def _row_stride(x: np.ndarray) -> int:
    """Row stride in elements of a 2-D array whose rows are contiguous."""
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    item = x.itemsize
    if x.size == 0:
        return max(x.shape[1], 1)
    if x.shape[1] > 1 and x.strides[1] != item:
        raise ValueError("rows must be contiguous")
    if x.shape[0] <= 1:
        return max(x.shape[1], 1)
    if x.strides[0] % item:
        raise ValueError("row stride is not a whole number of elements")
    return x.strides[0] // item


_KIND = {"f32": (np.float32, "oracle_gemm_f32"),
         "f16": (np.uint16, "oracle_gemm_f16"),
         "bf16": (np.uint16, "oracle_gemm_bf16"),
         "f64": (np.float64, "oracle_gemm_f64")}


def gemm(A: np.ndarray, B: np.ndarray, dtype: str = "f32", lib=None):
    """Return (C64, C32): the binary64 sums and their binary32 roundings, both M x N.

    ``A`` (M x K) and ``B`` (K x N) are float32 arrays for ``"f32"``, uint16 bit
    patterns for ``"f16"``/``"bf16"``, float64 for ``"f64"``.  Rows must be contiguous;
    a row stride larger than the row length (a view into a padded buffer) is passed on
    as lda / ldb.
    """
    np_t, fname = _KIND[dtype]
    if A.dtype != np_t or B.dtype != np_t:
        raise TypeError(f"{dtype} oracle expects {np.dtype(np_t)} operands")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    lda = max(_row_stride(A), max(K, 1))
    ldb = max(_row_stride(B), max(N, 1))
    C64 = np.zeros((M, N), dtype=np.float64)
    C32 = np.zeros((M, N), dtype=np.float32)
    lib = lib or _load()
    rc = getattr(lib, fname)(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                             C64.ctypes.data, C32.ctypes.data, max(N, 1))
    if rc != 0:
        raise RuntimeError(f"{fname} failed ({rc})")
    return C64, C32


_DT = {"f32": (np.float32, 0), "f16": (np.uint16, 1), "bf16": (np.uint16, 2)}


def gemm_ex(A: np.ndarray, B: np.ndarray, dtype: str = "f32", trans_a: bool = False,
            trans_b: bool = False, neg_a: bool = False, neg_b: bool = False,
            C_in: np.ndarray | None = None, lib=None):
    """(C64, C32) of C = s op(A) op(B) (+ C_in), s = -1 when exactly one operand is
    negated ("Advanced CUDA features - starting from GEMM", tensor-core instruction
    table).  ``A`` and ``B`` are the stored matrices: A is M x K, or K x M when
    trans_a; B is K x N, or N x K when trans_b.  ``C_in`` (float32 M x N) is added when
    given."""
    np_t, code = _DT[dtype]
    if A.dtype != np_t or B.dtype != np_t:
        raise TypeError(f"{dtype} oracle expects {np.dtype(np_t)} operands")
    M, K = (A.shape[1], A.shape[0]) if trans_a else A.shape
    KB, N = (B.shape[1], B.shape[0]) if trans_b else B.shape
    if KB != K:
        raise ValueError("inner dimensions differ")
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    lda = max(A.shape[1], 1)
    ldb = max(B.shape[1], 1)
    C64 = np.zeros((M, N), dtype=np.float64)
    C32 = np.zeros((M, N), dtype=np.float32)
    cin = None
    if C_in is not None:
        cin = np.ascontiguousarray(C_in, dtype=np.float32)
        if cin.shape != (M, N):
            raise ValueError("C_in must be M x N")
    lib = lib or _load()
    rc = lib.oracle_gemm_ex(code, int(trans_a), int(trans_b), int(neg_a), int(neg_b),
                            int(cin is not None), M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                            None if cin is None else cin.ctypes.data, C64.ctypes.data,
                            C32.ctypes.data, max(N, 1))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_ex failed ({rc})")
    return C64, C32


def gemm_ex16(A: np.ndarray, B: np.ndarray, dtype: str, trans_a: bool = False,
              trans_b: bool = False, neg_a: bool = False, neg_b: bool = False,
              C_in: np.ndarray | None = None, lib=None):
    """(C64, C16) of the general form with C in the operands' 16-bit type: C16 holds the
    binary64 results rounded once (to nearest, ties to even) to binary16 / bfloat16, as
    uint16 bit patterns; ``C_in`` (uint16 bits, M x N) is added when given."""
    if dtype not in ("f16", "bf16"):
        raise ValueError("gemm_ex16 takes f16 or bf16 operands")
    np_t, code = _DT[dtype]
    if A.dtype != np_t or B.dtype != np_t:
        raise TypeError(f"{dtype} oracle expects uint16 operands")
    M, K = (A.shape[1], A.shape[0]) if trans_a else A.shape
    KB, N = (B.shape[1], B.shape[0]) if trans_b else B.shape
    if KB != K:
        raise ValueError("inner dimensions differ")
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    C64 = np.zeros((M, N), dtype=np.float64)
    C16 = np.zeros((M, N), dtype=np.uint16)
    cin = None
    if C_in is not None:
        cin = np.ascontiguousarray(C_in, dtype=np.uint16)
        if cin.shape != (M, N):
            raise ValueError("C_in must be M x N")
    lib = lib or _load()
    rc = lib.oracle_gemm_ex16(code, int(trans_a), int(trans_b), int(neg_a), int(neg_b),
                              int(cin is not None), M, N, K, A.ctypes.data, max(A.shape[1], 1),
                              B.ctypes.data, max(B.shape[1], 1),
                              cin.ctypes.data if cin is not None else None, C64.ctypes.data,
                              C16.ctypes.data, max(N, 1))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_ex16 failed ({rc})")
    return C64, C16


def f64_to_f16_bits(x, lib=None) -> np.ndarray:
    """binary64 values rounded once to binary16 (ties to even), as uint16 bit patterns."""
    lib = lib or _load()
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    return np.array([lib.oracle_f64_to_f16(float(v)) for v in x], dtype=np.uint16)


def f64_to_bf16_bits(x, lib=None) -> np.ndarray:
    """binary64 values rounded once to bfloat16 (ties to even), as uint16 bit patterns."""
    lib = lib or _load()
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    return np.array([lib.oracle_f64_to_bf16(float(v)) for v in x], dtype=np.uint16)


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(int(bits))


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits))


def stream_xor(words: np.ndarray, lib=None) -> int:
    """XOR of all 32-bit words of `words` (any shape, viewed as uint32)."""
    lib = lib or _load()
    w = np.ascontiguousarray(words).view(np.uint32).reshape(-1)
    return int(lib.oracle_xor_words(w.ctypes.data if w.size else None, w.size))


def chase(next_words: np.ndarray, start: int, hops: int, n: int | None = None, lib=None) -> int:
    """The index reached from `start` after `hops` steps cur = next[cur] over the first
    `n` words of `next_words` (default all), an index outside [0, n) replaced by n - 1."""
    lib = lib or _load()
    w = np.ascontiguousarray(next_words, dtype=np.uint32).reshape(-1)
    n = w.size if n is None else int(n)
    if not (1 <= n <= w.size) or not (0 <= start < n) or hops < 0:
        raise ValueError("chase: need 1 <= n <= len(next), 0 <= start < n, hops >= 0")
    return int(lib.oracle_chase(w.ctypes.data, n, start, hops))


def softmax(X: np.ndarray, lib=None):
    """Row-wise softmax of a 2-D float32 array by the online recurrence.

    Returns (Y64, Y32, m, l): the binary64 results, their binary32 roundings (both of
    X's shape, packed), and the per-row running maximum and running sum at the end of
    the pass."""
    lib = lib or _load()
    X = np.asarray(X)
    if X.dtype != np.float32 or X.ndim != 2:
        raise ValueError("softmax: expected a 2-D float32 array")
    rows, cols = X.shape
    ldx = _row_stride(X)
    ldy = max(cols, 1)
    Y64 = np.zeros((rows, cols), np.float64)
    Y32 = np.zeros((rows, cols), np.float32)
    m = np.zeros(rows, np.float64)
    l = np.zeros(rows, np.float64)
    ptr = X.ctypes.data if X.size else None
    st = lib.oracle_softmax(rows, cols, ptr, ldx, Y64.ctypes.data, Y32.ctypes.data, ldy,
                            m.ctypes.data, l.ctypes.data)
    if st:
        raise ValueError("oracle_softmax: bad arguments")
    return Y64, Y32, m, l


def row_sum(X: np.ndarray, lib=None):
    """Sums of the rows of a 2-D float32 array, in binary64 in increasing column order.
    Returns (S64, S32)."""
    lib = lib or _load()
    X = np.asarray(X)
    if X.dtype != np.float32 or X.ndim != 2:
        raise ValueError("row_sum: expected a 2-D float32 array")
    rows, cols = X.shape
    S64 = np.zeros(rows, np.float64)
    S32 = np.zeros(rows, np.float32)
    ptr = X.ctypes.data if X.size else None
    st = lib.oracle_row_sum(rows, cols, ptr, _row_stride(X), S64.ctypes.data, S32.ctypes.data)
    if st:
        raise ValueError("oracle_row_sum: bad arguments")
    return S64, S32
