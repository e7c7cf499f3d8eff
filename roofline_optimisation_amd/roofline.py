"""Roofline accounting for the dense GEMM C = A.B (host-side arithmetic for the bench).

Closed forms from "Advanced CUDA features - starting from GEMM" (roofline section):

* work: an n x n x n product costs about 2 n^3 floating-point operations (one multiply
  and one add per (i, j, k)); for M x N x K it is 2 M N K;
* no-reuse traffic (case A / case (4)): every multiply-add fetches its two operands
  from DRAM, 2 n^3 words, so 8 n^3 bytes for float and an intensity of 0.25 FLOP/B;
* ideal-reuse traffic (case B / case (2)): A and B are read once and C written once,
  3 n^2 words (12 n^2 bytes for float), intensity n / 6;
* the ridge point is peak FLOP/s divided by bandwidth; an algorithm is compute bound
  once its intensity reaches the ridge (n >= 6 * ridge for the ideal-reuse GEMM);
* Little's law (section on occupancy control): bytes in flight = latency x bandwidth
  per cycle; and the occupancy example, where shared memory per block limits the
  number of resident blocks.

The generalisation to M x N x K with separate input and output element sizes counts
each operand once: in_bytes * (MK + KN) + out_bytes * MN (no beta term, so C is
written but never read).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

# MI355X (gfx950) published dense peaks, 256 CUs at 2.4 GHz, HBM3E 8 TB/s.
MI355X = {
    "cus": 256,
    "clock_hz": 2.4e9,
    "hbm_Bps": 8.0e12,
    "peak_flops": {
        "f32_vector": 157.3e12,   # 256 FLOP/clk/CU (packed FP32 FMA)
        "f32_mfma": 157.3e12,     # v_mfma_f32_*_f32: 256 FLOP/clk/CU
        "f16_mfma": 2516.6e12,    # 4096 FLOP/clk/CU, dense
        "bf16_mfma": 2516.6e12,
        "f64_vector": 78.6e12,
    },
}


def flops(M: int, N: int, K: int) -> int:
    """2 M N K: one multiply and one add per (i, j, k)."""
    return 2 * M * N * K


def ideal_bytes(M: int, N: int, K: int, in_bytes: int = 4, out_bytes: int = 4) -> int:
    """Each operand read once, C written once."""
    return in_bytes * (M * K + K * N) + out_bytes * M * N


def noreuse_bytes(M: int, N: int, K: int, in_bytes: int = 4) -> int:
    """Two operand loads per multiply-add, nothing reused."""
    return 2 * in_bytes * M * N * K


def intensity(M: int, N: int, K: int, in_bytes: int = 4, out_bytes: int = 4) -> float:
    return flops(M, N, K) / ideal_bytes(M, N, K, in_bytes, out_bytes)


def ridge(peak_flops: float, bandwidth_Bps: float) -> float:
    """FLOP per byte at which the compute roof meets the bandwidth slope."""
    return peak_flops / bandwidth_Bps


def crossover_n(peak_flops: float, bandwidth_Bps: float, word_bytes: int = 4) -> int:
    """Smallest square n whose ideal-reuse intensity reaches the ridge.

    With equal input and output word sizes the intensity is 2n^3 / (3 w n^2) = 2n / (3w),
    i.e. n / 6 for 4-byte words."""
    r = ridge(peak_flops, bandwidth_Bps)
    return math.ceil(r * 3 * word_bytes / 2)


def attainable(oi: float, peak_flops: float, bandwidth_Bps: float) -> float:
    """Roofline: min(peak, intensity x bandwidth)."""
    return min(peak_flops, oi * bandwidth_Bps)


def compute_time(M: int, N: int, K: int, peak_flops: float) -> float:
    return flops(M, N, K) / peak_flops


def memory_time(nbytes: float, bandwidth_Bps: float) -> float:
    return nbytes / bandwidth_Bps


def littles_law_bytes(latency_cycles: float, bandwidth_Bps: float, clock_hz: float) -> float:
    """Bytes that must be in flight to sustain ``bandwidth_Bps``."""
    return latency_cycles * bandwidth_Bps / clock_hz


@dataclass(frozen=True)
class Occupancy:
    blocks: int
    warps: int
    fraction: float


def occupancy_from_smem(smem_per_block: int, smem_per_sm: int, max_warps: int,
                        warps_per_block: int, max_blocks: int | None = None) -> Occupancy:
    """Resident blocks limited by shared memory and by the warp slots."""
    by_smem = smem_per_sm // smem_per_block if smem_per_block else max_warps
    by_warps = max_warps // warps_per_block
    cap = by_warps if max_blocks is None else min(by_warps, max_blocks)
    blocks = min(by_smem, cap)
    warps = blocks * warps_per_block
    return Occupancy(blocks, warps, warps / max_warps)


def roofline_entry(M: int, N: int, K: int, seconds: float, dtype: str) -> dict:
    """TFLOP/s and fraction of the MI355X peak that bounds this GEMM."""
    in_b = 4 if dtype == "f32" else 2
    peak_key = {"f32": "f32_mfma", "f16": "f16_mfma", "bf16": "bf16_mfma"}[dtype]
    peak = MI355X["peak_flops"][peak_key]
    f = flops(M, N, K)
    nbytes = ideal_bytes(M, N, K, in_b, 4)
    oi = f / nbytes
    tf = f / seconds
    return {
        "tflops": tf / 1e12,
        "peak_tflops": peak / 1e12,
        "frac": tf / peak,
        "oi": oi,
        "attainable_tflops": attainable(oi, peak, MI355X["hbm_Bps"]) / 1e12,
        "ideal_bytes": nbytes,
        "ideal_GBps": nbytes / seconds / 1e9,
    }


def text_chart(points, roofs, bandwidth_Bps: float, x_range=(8.0, 4096.0), y_range=(0.25, 4096.0),
               width: int = 64, height: int = 20) -> list[str]:
    """A log-log roofline chart as text lines.

    ``points``: (intensity FLOP/B, achieved TFLOP/s, marker character); ``roofs``:
    (peak TFLOP/s, character) -- each roof is drawn as min(peak, intensity x bandwidth).
    Axes are log2 scaled over x_range (FLOP/B) and y_range (TFLOP/s); a point outside the
    ranges is clamped to the border.  Later points overwrite earlier ones."""
    lx0, lx1 = math.log2(x_range[0]), math.log2(x_range[1])
    ly0, ly1 = math.log2(y_range[0]), math.log2(y_range[1])

    def col(x):
        return min(width - 1, max(0, round((math.log2(x) - lx0) / (lx1 - lx0) * (width - 1))))

    def row(y):
        return min(height - 1, max(0, round((ly1 - math.log2(y)) / (ly1 - ly0) * (height - 1))))

    grid = [[" "] * width for _ in range(height)]
    for peak, ch in roofs:
        for c in range(width):
            x = 2.0 ** (lx0 + (lx1 - lx0) * c / (width - 1))
            grid[row(min(peak, x * bandwidth_Bps / 1e12))][c] = ch
    for x, y, ch in points:
        grid[row(max(y, y_range[0]))][col(x)] = ch
    out = []
    for r in range(height):
        y = 2.0 ** (ly1 - (ly1 - ly0) * r / (height - 1))
        label = f"{y:7.1f} |" if r % 4 == 0 or r == height - 1 else "        |"
        out.append(label + "".join(grid[r]))
    out.append("        +" + "-" * width)
    ticks = [" "] * (width + 9)
    for x in (8, 32, 128, 512, 2048):
        if x_range[0] <= x <= x_range[1]:
            t = str(x)
            c = 9 + col(x)
            for i, chx in enumerate(t):
                if c + i < len(ticks):
                    ticks[c + i] = chx
    out.append("".join(ticks).rstrip() + "   (FLOP/B, log scale; TFLOP/s log scale)")
    return out
