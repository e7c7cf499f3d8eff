"""Helpers for the GPU parity tests: device buffers with NaN-poisoned padding and guard
regions, calls through the C ABI, and error metrics against the oracle."""

from __future__ import annotations

import numpy as np

from roofline_optimisation_amd import binding as gb
from roofline_optimisation_amd import inputs

SENTINEL = np.float32(7777.0)
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}
NP_STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}
CODE = {"f32": gb.F32, "f16": gb.F16, "bf16": gb.BF16}


def torch():
    import torch as _t
    return _t


def nan_fill(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else np.uint16(NAN_BITS[dtype])


def place(x: np.ndarray, ld: int, offset: int, guard_rows: int, fill) -> np.ndarray:
    """Flat buffer: `offset` fill elements, then x as rows of stride ld (padding = fill),
    then `guard_rows` rows of fill."""
    rows, cols = x.shape
    buf = np.full(offset + (rows + guard_rows) * ld + 8, fill, dtype=x.dtype)
    if rows and cols:
        buf[offset:offset + rows * ld].reshape(rows, ld)[:, :cols] = x
    return buf


def to_device(x: np.ndarray):
    t = torch()
    if x.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    return t.from_numpy(np.ascontiguousarray(x)).cuda()


def gpu_gemm(A: np.ndarray, B: np.ndarray, dtype: str, variant: int = gb.VARIANT_AUTO, *,
             pad=(0, 0, 0), offset: int = 0, guard_rows: int = 0, stream=None,
             entry: str = "variant"):
    """C = A.B on the GPU through the C ABI.  Returns (C as M x N float32, intact) where
    `intact` says every element of the C buffer outside the M x N result still holds
    the sentinel."""
    t = torch()
    M, K = A.shape
    N = B.shape[1]
    lda, ldb, ldc = max(K, 1) + pad[0], max(N, 1) + pad[1], max(N, 1) + pad[2]
    fill = nan_fill(dtype)
    dA = to_device(place(A, lda, offset, guard_rows, fill))
    dB = to_device(place(B, ldb, offset, guard_rows, fill))
    cbuf = np.full(offset + (M + guard_rows) * ldc + 8, SENTINEL, dtype=np.float32)
    dC = to_device(cbuf)
    es = dA.element_size()
    pa, pb, pc = dA.data_ptr() + offset * es, dB.data_ptr() + offset * es, dC.data_ptr() + offset * 4
    s = stream if stream is not None else t.cuda.current_stream()
    h = s.cuda_stream
    if entry == "typed":
        f = {"f32": gb.gemm_f32, "f16": gb.gemm_f16f32acc, "bf16": gb.gemm_bf16f32acc}[dtype]
        st = f(M, N, K, pa, lda, pb, ldb, pc, ldc, h)
    else:
        st = gb.gemm355_run_variant(variant, CODE[dtype], M, N, K, pa, lda, pb, ldb, pc, ldc, h)
    if st != gb.OK:
        raise gb.Gemm355Error(st, f"gemm {dtype} variant {variant} {M}x{N}x{K}")
    s.synchronize()
    out = dC.cpu().numpy()
    region = out[offset:offset + M * ldc].reshape(M, ldc) if M else np.zeros((0, ldc), np.float32)
    C = region[:, :N].copy()
    mask = np.ones(out.shape, bool)
    if M and N:
        mask[offset:offset + M * ldc].reshape(M, ldc)[:, :N] = False
    intact = bool(np.all(out[mask] == SENTINEL))
    return C, intact


def errors(C: np.ndarray, C64: np.ndarray) -> tuple[float, float]:
    d = C.astype(np.float64) - C64
    den = np.linalg.norm(C64)
    rel = float(np.linalg.norm(d) / den) if den > 0 else float(np.linalg.norm(d))
    return rel, float(np.abs(d).max()) if d.size else 0.0


def tolerance(dtype: str, dist: str, K: int) -> tuple[float, float]:
    """(max relative Frobenius error, max absolute error).

    FP32, U[-1,1]: 1e-5 and 1e-4 sqrt(K).  FP32, N(0,1): the absolute bound scales with
    the spread of the products, three times that of U[-1,1] products: 3e-4 sqrt(K).
    FP16/BF16 (against the oracle on the same rounded inputs): 1e-3 relative, and the
    FP32 element bound above: a product of two binary16 (11-bit) or bfloat16 (8-bit)
    significands is exact in binary32, so only the binary32 accumulation rounds, as in
    the FP32 case."""
    tabs = (1e-4 if dist == "uniform" else 3e-4) * np.sqrt(max(K, 1))
    return (1e-5 if dtype == "f32" else 1e-3), tabs


def sample_rows(M: int, n: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n, M), replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(rows))


__all__ = ["gpu_gemm", "errors", "tolerance", "sample_rows", "place", "to_device", "inputs"]
