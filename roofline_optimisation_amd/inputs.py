"""Seeded synthetic operands for the dense GEMM C = A.B (row-major A is MxK, B is KxN).

This module is shared by the GPU path's tests and bench and by the CPU oracle's
tests.  It only draws random numbers and rounds them to the storage precision of
the inputs; it holds none of the product's arithmetic.

Recipe (the pages measure on synthetic square sizes only, e.g. the 256^3 and
3072^3 runs printed on "Advanced CUDA features - starting from GEMM",
section "Shared Memory Tiling", performance test):

* ``numpy.random.default_rng(seed)`` (PCG64), reseeded for every case; A (MxK)
  is drawn first, then B (KxN), both in row-major order.
* ``"uniform"``: i.i.d. U[-1, 1] drawn in float64, rounded to float32 (RNE).
* ``"normal"``: i.i.d. N(0, 1) drawn in float64, rounded to float32 (RNE).
* ``"int"``: i.i.d. integers uniform on {-4, ..., 4}, stored exactly.
* FP16 inputs: the float32 values rounded to IEEE binary16 by numpy (RNE).
* BF16 inputs: the float32 values rounded to bfloat16 by round-to-nearest-even
  on the upper 16 bits of the binary32 pattern.

FP16/BF16 operands travel as ``uint16`` bit patterns.

Row-wise softmax and row-sum inputs (``make_logits``; the pages give the online softmax
and the shuffle reduction without workloads, so these are synthetic rows of logits):
``default_rng(seed)``, one rows x cols draw in row-major order, rounded to float32:
``"normal"`` N(0, 1); ``"uniform"`` U[-1, 1]; ``"int"`` integers on {-4, ..., 4};
``"wide"`` N(0, 1) x 40 (exp of the raw values would overflow binary32, so only a
max-shifted evaluation is finite); ``"ascending"`` / ``"descending"`` N(0, 1) x 4 sorted
along each row (a new running maximum at every element, or never after the first).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DTYPES = ("f32", "f16", "bf16")


# U[-1, 1] matrices larger than this many elements are drawn in pieces of this size, so
# a 2^30-element operand does not need its float64 draw in memory at once.  The values are
# the same: the generator hands out one double per element in row-major order whatever
# the size of each call.
UNIFORM_CHUNK = 1 << 24


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "uniform":
        n = int(np.prod(shape))
        if n <= UNIFORM_CHUNK:
            return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
        out = np.empty(n, dtype=np.float32)
        for s in range(0, n, UNIFORM_CHUNK):
            e = min(n, s + UNIFORM_CHUNK)
            out[s:e] = rng.uniform(-1.0, 1.0, size=e - s)  # float64 -> float32, RNE
        return out.reshape(shape)
    if dist == "normal":
        return rng.standard_normal(size=shape).astype(np.float32)
    if dist == "int":
        return rng.integers(-4, 5, size=shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_logits(rows: int, cols: int, seed: int, dist: str = "normal") -> np.ndarray:
    """A rows x cols float32 matrix of synthetic logits (see the module notes)."""
    rng = np.random.default_rng(seed)
    if dist in ("normal", "uniform", "int"):
        return _draw(rng, (rows, cols), dist)
    if dist == "wide":
        return (rng.standard_normal(size=(rows, cols)) * 40.0).astype(np.float32)
    if dist in ("ascending", "descending"):
        x = np.sort((rng.standard_normal(size=(rows, cols)) * 4.0).astype(np.float32), axis=1)
        return np.ascontiguousarray(x if dist == "ascending" else x[:, ::-1])
    raise ValueError(f"unknown distribution {dist!r}")


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (RNE) and return the bit patterns."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (RNE) and return the bit patterns.

    Works on the binary32 patterns in pieces of UNIFORM_CHUNK elements, in uint32: for a
    finite value the pattern is at most 0xFF7FFFFF, so adding the rounding bias (at most
    0x8000) cannot wrap."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.size, dtype=np.uint16)
    for s in range(0, u.size, UNIFORM_CHUNK):
        v = u[s:s + UNIFORM_CHUNK]
        out[s:s + UNIFORM_CHUNK] = (v + (np.uint32(0x7FFF) + ((v >> 16) & np.uint32(1)))) >> 16
    return out.reshape(x.shape)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Convert float32 values to the storage form of ``dtype`` (float32 or uint16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_operands(M: int, N: int, K: int, seed: int, dist: str = "uniform",
                  dtype: str = "f32") -> tuple[np.ndarray, np.ndarray]:
    """Draw A (MxK) then B (KxN) from a fresh generator, in ``dtype`` storage form."""
    rng = np.random.default_rng(seed)
    a = _draw(rng, (M, K), dist)
    b = _draw(rng, (K, N), dist)
    return to_storage(a, dtype), to_storage(b, dtype)


def draw_rows(M: int, K: int, seed: int, dist: str = "uniform", dtype: str = "f32",
              rows: int | None = None) -> np.ndarray:
    """The first ``rows`` rows of the A that ``make_operands`` draws (PCG64 streams are
    consumed row-major, so a prefix of rows is a prefix of the stream)."""
    rng = np.random.default_rng(seed)
    r = M if rows is None else min(rows, M)
    return to_storage(_draw(rng, (r, K), dist), dtype)


def embed(x: np.ndarray, ld: int, extra_rows: int = 0, fill=np.nan) -> np.ndarray:
    """Place a row-major matrix inside a larger (rows+extra_rows) x ld buffer filled with
    ``fill`` (NaN for float32, the quiet-NaN pattern for uint16 storage)."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError("ld smaller than the row length")
    if x.dtype == np.uint16:
        fillv = 0x7E00 if (isinstance(fill, float) and np.isnan(fill)) else fill
        out = np.full((rows + extra_rows, ld), fillv, dtype=np.uint16)
    else:
        out = np.full((rows + extra_rows, ld), fill, dtype=x.dtype)
    out[:rows, :cols] = x
    return out


@dataclass(frozen=True)
class Case:
    """One synthetic GEMM workload."""
    name: str
    dtype: str
    M: int
    N: int
    K: int
    seed: int
    dist: str


# The five workloads the measurements are quoted on (square FP32 256^3 and 3072^3 as on
# the pages, ragged FP32 shapes, FP16 4096^3, and the roofline sweep).
CASES = {
    "f32_256": Case("f32_256", "f32", 256, 256, 256, 0, "uniform"),
    "f32_256_int": Case("f32_256_int", "f32", 256, 256, 256, 0, "int"),
    "f32_3072": Case("f32_3072", "f32", 3072, 3072, 3072, 1, "uniform"),
    "f32_1000": Case("f32_1000", "f32", 1000, 1000, 1000, 2, "normal"),
    "f32_1023x997x515": Case("f32_1023x997x515", "f32", 1023, 997, 515, 2, "normal"),
    "f16_4096": Case("f16_4096", "f16", 4096, 4096, 4096, 3, "uniform"),
}

SWEEP_N = (128, 256, 512, 1024, 2048, 4096, 8192)
SWEEP_SEED = 4


def sweep_cases() -> list[Case]:
    """Square FP32 and BF16->FP32 GEMMs over SWEEP_N plus the tall-skinny 16384x4096x4096."""
    out = []
    for dt in ("f32", "bf16"):
        for n in SWEEP_N:
            out.append(Case(f"{dt}_sq{n}", dt, n, n, n, SWEEP_SEED, "uniform"))
        out.append(Case(f"{dt}_tall", dt, 16384, 4096, 4096, SWEEP_SEED, "uniform"))
    return out


def operands_for(case: Case) -> tuple[np.ndarray, np.ndarray]:
    return make_operands(case.M, case.N, case.K, case.seed, case.dist, case.dtype)
