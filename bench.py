#!/usr/bin/env python3
"""Benchmark of libgemm355 on one MI355X: GEMM TFLOP/s (2MNK / t) and fraction of peak.

A step is one call of the FP32 entry point gemm_f32 on the 3072 x 3072 x 3072 workload
(row-major, packed strides, A and B i.i.d. U[-1,1] from seed 1), with the operands
already resident in HBM.  W untimed warm-up steps are followed by K timed steps on one
HIP stream, bracketed by device synchronisation; the per-step time comes from HIP
events recorded on that stream.  The defaults (W = 300, K = 200) time the sustained
rate: per-launch kernel traces show the chip's clocks settling over the first ~50
(FP32) to ~200 (FP16) back-to-back launches, so a short warm-up measures the power
management's transient instead of the kernel.  The FP16-input / FP32-accumulate 4096^3 workload
(seed 3) is measured the same way and reported beside it.

`--softmax PATH` measures the row-wise softmax and row sum instead (64 Mi binary32
logits per workload) and prints one JSON line for the 16384 x 4096 workload, with its
roofline against the 8 TB/s HBM peak and the CPU oracle's rate beside it.

The JSON line also carries
  * "roofline": the dominant kernel's achieved TFLOP/s against the MI355X peak for its
    arithmetic (FP32 on the matrix cores: 157.3 TFLOP/s), with HBM traffic from the
    committed rocprofv3 counter summary when it was taken on the current kernel source;
  * "cpu_baseline": the CPU oracle (plain C, fp64 accumulation, OpenMP over rows) timed
    on this host on one full step of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAKS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}  # TFLOP/s, dense, 2.4 GHz
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "roofline_optimisation_amd", "csrc")
KERNEL_SOURCES = {"f32": ["k_mfma_f32.hip", "f32_gemm.hpp", "common.hpp"],
                  "f16": ["k_mfma_f16.hip", "h16_gemm.hpp", "h16_dma.hpp", "common.hpp"],
                  "softmax": ["k_softmax.hip", "wave_reduce.hpp"]}
PMC_FILES = {"f32": "pmc_mfma_f32_n3072.txt", "f16": "pmc_mfma_f16_n4096.txt",
             "softmax": "pmc_softmax_16384x4096.txt"}
HBM_PEAK_GBS = 8000.0
# Row-wise softmax workloads: 64 Mi binary32 logits each, N(0, 1), seed 7 (the pages give
# the online softmax without sizes); the first is the one the JSON line reports.
SOFTMAX_SHAPES = ((16384, 4096), (65536, 1024), (4096, 16384), (2048, 32768), (512, 131072))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def strip_comments(src: str) -> str:
    """C++ source without its comments, blank lines and layout whitespace (string and
    character literals kept as they are), so that an edit of comments or indentation
    leaves the hash of a kernel's code unchanged."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            while i < n and src[i] != "\n":
                i += 1
        elif src.startswith("/*", i):
            e = src.find("*/", i + 2)
            i = n if e < 0 else e + 2
            out.append(" ")
        elif c in " \t":
            if out and out[-1] != " ":
                out.append(" ")
            i += 1
        else:
            out.append(c)
            i += 1
    lines = (ln.strip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def kernel_hash(kind: str) -> str:
    """Hash of the code (comments stripped) of the sources a kernel family is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kind: str):
    """HBM bytes per launch from the committed counter summary, or None if there is none
    or it was taken on a different kernel source."""
    path = os.path.join(PROFILES, PMC_FILES[kind])
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if ":" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_hash(kind):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_gemm(kind, M, N, K, seed, steps, warmup):
    import torch

    from roofline_optimisation_amd import binding as gb
    from roofline_optimisation_amd import inputs

    dt = kind
    A, B = inputs.make_operands(M, N, K, seed, "uniform", dt)
    if dt == "f32":
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        entry = gb.gemm_f32
    else:
        dA = torch.from_numpy(A.view("int16")).cuda()
        dB = torch.from_numpy(B.view("int16")).cuda()
        entry = gb.gemm_f16f32acc if dt == "f16" else gb.gemm_bf16f32acc
    dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    h = stream.cuda_stream
    args = (M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, h)
    desc = gb.gemm355_kernel_desc(-1, gb.DTYPE_CODES[dt], M, N, K, dA.data_ptr(), K,
                                  dB.data_ptr(), N, dC.data_ptr(), N)

    def step():
        st = entry(*args)
        if st != gb.OK:
            raise gb.Gemm355Error(st, entry.__name__)

    torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    return {"ms": ms, "wall_ms": wall * 1e3 / steps, "desc": desc, "A": A, "B": B, "dC": dC}


def cpu_baseline(A, B, M, N, K, min_seconds=10.0):
    """The oracle on this host's cores: full steps of the same workload, repeated until
    at least `min_seconds` of wall time, reported as the mean rate."""
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm(A, B, "f32")
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(2.0 * M * N * K * reps / dt / 1e12, 5), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} full steps of FP32 {M}x{N}x{K} (same seeded operands), "
                      f"{dt:.1f} s wall"}


def time_variant(variant, dtype, M, N, K, seed, reps=None):
    """Mean per-launch time (ms) of one kernel family on a seeded U[-1,1] workload, timed
    with HIP events on one stream after warm-up."""
    import torch

    from roofline_optimisation_amd import binding as gb
    from roofline_optimisation_amd import inputs

    A, B = inputs.make_operands(M, N, K, seed, "uniform", dtype)
    if dtype == "f32":
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    else:
        dA = torch.from_numpy(A.view("int16")).cuda()
        dB = torch.from_numpy(B.view("int16")).cuda()
    dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    code = gb.DTYPE_CODES[dtype]
    args = (variant, code, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
            stream.cuda_stream)
    desc = gb.gemm355_kernel_desc(variant, code, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N,
                                  dC.data_ptr(), N)

    def launch():
        st = gb.gemm355_run_variant(*args)
        if st != gb.OK:
            raise gb.Gemm355Error(st, "gemm355_run_variant")

    launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    launch()
    e1.record(stream)
    stream.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    if reps is None:
        reps = int(min(200, max(3, 100.0 / one)))  # about 100 ms of timed work
    # about 50 ms of untimed launches first: the clocks take that long to settle after
    # the host-side set-up of each case has left the GPU idle
    for _ in range(int(min(2000, max(2, 50.0 / one)))):
        launch()
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    stream.synchronize()
    return e0.elapsed_time(e1) / reps, desc, reps


def family_run(family, steps, warmup, dtype="f32", n=0, m=0):
    """`warmup` untimed and `steps` timed launches of one kernel family on the FP32 3072^3
    workload (seed 1) or an n^3 FP16/BF16 one (seed 3; m x n x n with m given), logged to
    stderr: the target of the counter passes."""
    import torch

    from roofline_optimisation_amd import binding as gb
    from roofline_optimisation_amd import inputs

    variant = gb.VARIANTS[family]
    n = n or (3072 if dtype == "f32" else 4096)
    M = m or n
    A, B = inputs.make_operands(M, n, n, 1 if dtype == "f32" else 3, "uniform", dtype)
    if dtype == "f32":
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    else:
        dA = torch.from_numpy(A.view("int16")).cuda()
        dB = torch.from_numpy(B.view("int16")).cuda()
    dC = torch.empty((M, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    args = (variant, gb.DTYPE_CODES[dtype], M, n, n, dA.data_ptr(), n, dB.data_ptr(), n,
            dC.data_ptr(), n, stream.cuda_stream)
    desc = gb.gemm355_kernel_desc(*args[:-1])

    def launch():
        st = gb.gemm355_run_variant(*args)
        if st != gb.OK:
            raise gb.Gemm355Error(st, "gemm355_run_variant")

    for _ in range(warmup):
        launch()
    stream.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    stream.synchronize()
    ms = e0.elapsed_time(e1) / max(steps, 1)
    log(f"[bench] family {family} ({desc}) {dtype} {M}x{n}x{n}: {warmup} + {steps} launches, "
        f"{ms:.4f} ms/launch, {2.0 * M * n * n / (ms * 1e-3) / 1e12:.2f} TFLOP/s")


RAGGED_K = ((4096, 4096, 4096), (4096, 4000, 4000), (4096, 4064, 4064), (4096, 4072, 4072),
            (4096, 4104, 4104), (4096, 4000, 4096), (4096, 4072, 4096), (4096, 4096, 4104),
            (2048, 2048, 2048), (2048, 2000, 2000), (2048, 2000, 2048), (2048, 2048, 2056))


def ragged_k_lines(warm=300, rounds=3, reps=100):
    """BF16 n x n x K (U[-1,1], seed 4; n = 4096 on the 256 x 256 direct-to-LDS tile, 2048
    on the 128 x 128 one) for K = n and K that are not whole ring trips, A's rows packed
    (lda = K) or padded to 2n halves, and K = n with rows of 2n + 8 halves (off the
    128-byte lines): every case warmed, then timed interleaved, median of `rounds` rounds
    of `reps` launches (HIP events).  Time per FLOP is relative to K = lda = n."""
    import torch

    from roofline_optimisation_amd import binding as gb
    from roofline_optimisation_amd import inputs

    stream = torch.cuda.Stream()
    runs = []
    for n, K, lda in RAGGED_K:
        A, B = inputs.make_operands(n, n, K, 4, "uniform", "bf16")
        dA = torch.zeros((n, lda), dtype=torch.int16, device="cuda")
        dA[:, :K] = torch.from_numpy(A.view("int16")).cuda()
        dB = torch.from_numpy(B.view("int16")).cuda()
        dC = torch.empty((n, n), dtype=torch.float32, device="cuda")
        args = (n, n, K, dA.data_ptr(), lda, dB.data_ptr(), n, dC.data_ptr(), n, stream.cuda_stream)
        desc = gb.gemm355_kernel_desc(gb.VARIANT_AUTO, gb.BF16, *args[:-1])

        def go(args=args):
            st = gb.gemm_bf16f32acc(*args)
            if st != gb.OK:
                raise gb.Gemm355Error(st, "gemm_bf16f32acc")
        runs.append(((n, K, lda), desc, go, (dA, dB, dC)))
    for key, desc, go, _ in runs:
        for _ in range(warm):
            go()
    stream.synchronize()
    times = {key: [] for key, *_ in runs}
    for _ in range(rounds):
        for key, desc, go, _ in runs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                go()
            e1.record(stream)
            stream.synchronize()
            times[key].append(e0.elapsed_time(e1) * 1e3 / reps)
    out = ["# BF16 n x n x K on one MI355X: K not a whole number of ring trips, and A's row alignment", "",
           f"U[-1,1] bfloat16 operands (seed 4), FP32 C, B and C packed, A's rows of lda halves; {warm} "
           f"warm-up launches per case, then all cases interleaved, median of {rounds} rounds of {reps} "
           f"launches; HIP events. k-steps are 32 wide, run in trips of 4 (256 x 256 tile) or 8 "
           f"(128 x 128 tile); the last trip's steps wholly past K are skipped. Time per FLOP is "
           f"relative to K = lda = n.", "",
           "| n | K | lda | k-steps run | kernel | µs | TFLOP/s | % of 2516.6 | time per FLOP vs K = n |",
           "|---|---|---|---|---|---|---|---|---|"]
    for (n, K, lda), desc, go, _ in runs:
        base = float(np.median(times[(n, n, n)])) / n
        us = float(np.median(times[(n, K, lda)]))
        tf = 2.0 * n * n * K / us / 1e6
        out.append(f"| {n} | {K} | {lda} | {-(-K // 32)} | `{md_cell(desc)}` | {us:.1f} | {tf:.0f} | "
                   f"{100 * tf / PEAKS['bf16']:.1f} | {us / K / base:.3f} |")
        log(f"[ragged-k] n={n} K={K} lda={lda}: {us:.1f} us, {tf:.0f} TFLOP/s")
    return out


def md_cell(text: str) -> str:
    """A markdown table cell: '|' inside the text escaped."""
    return text.replace("|", "\\|")


def schedule_lines(warm=300, rounds=3, reps=100):
    """The schedules of the FP16 direct-to-LDS kernel at 4096^3 and 8192^3 (U[-1,1] from
    seed 3): every case warmed, then timed interleaved, median of `rounds` rounds of
    `reps` launches (HIP events on one stream)."""
    import torch

    from roofline_optimisation_amd import binding as gb
    from roofline_optimisation_amd import inputs

    names = [("mfma", "dispatched: 256x256, 4 waves"),
             ("mfma_split", "split: 256x128, 4 compute + 4 producer waves"),
             ("mfma_w8", "w8: 256x256, 8 waves (2 per SIMD)"),
             ("mfma_t256x128", "t256x128: 256x128, 4 waves")]
    stream = torch.cuda.Stream()
    out = ["# Schedules of the FP16 direct-to-LDS GEMM kernel on one MI355X", "",
           f"U[-1,1] binary16 operands (seed 3), FP32 C; {warm} warm-up launches per case, then "
           f"all cases interleaved, median of {rounds} rounds of {reps} launches; HIP events.", "",
           "| n | schedule | kernel | µs | TFLOP/s | % of 2516.6 | vs dispatched |", "|---|---|---|---|---|---|---|"]
    for n in (4096, 8192):
        A, B = inputs.make_operands(n, n, n, 3, "uniform", "f16")
        dA = torch.from_numpy(A.view("int16")).cuda()
        dB = torch.from_numpy(B.view("int16")).cuda()
        dC = torch.empty((n, n), dtype=torch.float32, device="cuda")
        runs = []
        for fam, label in names:
            v = gb.VARIANTS[fam]
            args = (v, gb.F16, n, n, n, dA.data_ptr(), n, dB.data_ptr(), n, dC.data_ptr(), n,
                    stream.cuda_stream)
            desc = gb.gemm355_kernel_desc(*args[:-1])

            def go(args=args):
                st = gb.gemm355_run_variant(*args)
                if st != gb.OK:
                    raise gb.Gemm355Error(st, "gemm355_run_variant")
            runs.append((label, desc, go))
        for label, desc, go in runs:
            for _ in range(warm):
                go()
        stream.synchronize()
        times = {label: [] for label, _, _ in runs}
        for _ in range(rounds):
            for label, desc, go in runs:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    go()
                e1.record(stream)
                stream.synchronize()
                times[label].append(e0.elapsed_time(e1) * 1e3 / reps)
        base = float(np.median(times[runs[0][0]]))
        for label, desc, go in runs:
            us = float(np.median(times[label]))
            tf = 2.0 * n ** 3 / us / 1e6
            out.append(f"| {n} | {label} | `{md_cell(desc)}` | {us:.1f} | {tf:.0f} | {100 * tf / PEAKS['f16']:.1f} | "
                       f"{base / us:.3f}x |")
            log(f"[schedules] {n}^3 {label}: {us:.1f} us, {tf:.0f} TFLOP/s")
        del dA, dB, dC
    return out


# Calls for which the dispatcher takes the 192 x 256 or 256 x 192 direct-to-LDS tile (the
# last five with the 192 side m/n-contiguous, in LDS rows of 24 chunks), each with the 256 x 256 tile
# timed beside it: (dtype, M, N, K, gemm355_gemm_ex flags).
TILE_SHAPES = [("f16", 3072, 3072, 3072, ()), ("bf16", 3072, 3072, 3072, ()), ("f16", 3072, 4096, 4096, ()),
               ("f16", 4096, 4104, 4096, ()), ("f16", 4608, 4608, 4608, ()), ("f16", 6144, 6144, 4096, ()),
               ("f16", 3000, 3072, 1024, ()), ("bf16", 3072, 3072, 1000, ()),
               ("f16", 3072, 3072, 3072, ("TRANS_B",)), ("f16", 3072, 3072, 3072, ("NEG_A", "ACCUMULATE")),
               ("bf16", 3072, 3072, 3072, ("C_16",)), ("f16", 4096, 3072, 4096, ("TRANS_B",)),
               ("bf16", 4096, 3072, 4096, ("TRANS_B",)), ("f16", 3072, 3072, 3072, ("TRANS_A", "TRANS_B")),
               ("bf16", 3000, 3000, 1000, ("TRANS_A", "TRANS_B", "ACCUMULATE")),
               ("f16", 4096, 3072, 4096, ()), ("bf16", 4096, 3072, 4096, ()), ("f16", 3072, 3072, 3072, ("TRANS_A",)),
               ("bf16", 3072, 3072, 3072, ("TRANS_A",)), ("f16", 4608, 4608, 4608, ("TRANS_A",))]
# Calls for which the dispatcher takes the 128 x 128 direct-to-LDS tile on its 4-stage ring
# (two workgroups per CU), each with the register-staged kernel timed beside it.
RING4_SHAPES = [("f16", 2304, 2304, 2304, ()), ("f16", 2560, 2560, 2560, ()), ("bf16", 2560, 2560, 2560, ()),
                ("f16", 2816, 2816, 2816, ()), ("f16", 2304, 2304, 4096, ()), ("f16", 2560, 2560, 4096, ()),
                ("f16", 2048, 4096, 2048, ()), ("bf16", 2500, 2600, 1000, ()),
                ("f16", 2560, 2560, 2560, ("TRANS_A",)), ("f16", 2560, 2560, 2560, ("NEG_A", "ACCUMULATE"))]

# Calls of small grids that the dispatcher gives a direct-to-LDS tile and variant
# MFMA_STAGED_SMALL does not: the 64 x 64 tile (plain, general form, ragged, deep K), the
# 128 x 128 one for plain products whose grid leaves CUs idle, and the 4-stage ring for K
# from 128 to 255.
SMALL_SHAPES = [("bf16", 1024, 1024, 1024, ()), ("f16", 1024, 1024, 1024, ()), ("bf16", 512, 512, 512, ()),
                ("f16", 1024, 1024, 4096, ()), ("bf16", 1000, 1000, 1000, ()),
                ("f16", 1024, 1024, 1024, ("TRANS_A",)), ("bf16", 1024, 1024, 1024, ("C_16",)),
                ("f16", 1280, 1280, 1280, ("TRANS_B", "ACCUMULATE")), ("bf16", 1408, 1408, 1408, ("NEG_A",)),
                ("f16", 1536, 1536, 1536, ()), ("f16", 1792, 1792, 1792, ()), ("f16", 1536, 1536, 4096, ()),
                ("bf16", 1500, 1456, 1000, ()), ("f16", 1600, 1600, 1600, ()),
                ("bf16", 1024, 1024, 200, ("TRANS_A",)), ("f16", 2048, 2048, 136, ()),
                ("f16", 1792, 1792, 248, ("TRANS_B",)), ("bf16", 2048, 2048, 192, ("ACCUMULATE",))]


def _time_pair(dt, M, N, K, fl, alt, warm, rounds, reps, stream):
    """Median times (us) of one call on variant `alt` and as dispatched, through
    gemm355_gemm_ex: U[-1,1] operands (seed 3; a transposed operand is the same draw
    stored transposed), packed strides; both warmed, then timed interleaved, `rounds`
    rounds of `reps` launches (HIP events on `stream`).  Returns (alt us, dispatched us,
    alt kernel, dispatched kernel)."""
    import torch

    from roofline_optimisation_amd import binding as gb
    from roofline_optimisation_amd import inputs

    flags = 0
    for f in fl:
        flags |= getattr(gb, f)
    A, B = inputs.make_operands(M, N, K, 3, "uniform", dt)
    if "TRANS_A" in fl:
        A = np.ascontiguousarray(A.T)
    if "TRANS_B" in fl:
        B = np.ascontiguousarray(B.T)
    dA = torch.from_numpy(A.view("int16")).cuda()
    dB = torch.from_numpy(B.view("int16")).cuda()
    # an accumulated C grows by one product's worth per launch; well inside FP32's range
    dC = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    runs = []
    for v in (alt, gb.VARIANT_AUTO):
        args = (v, gb.DTYPE_CODES[dt], flags, M, N, K, dA.data_ptr(), A.shape[1], dB.data_ptr(), B.shape[1],
                dC.data_ptr(), N, stream.cuda_stream)

        def go(args=args):
            st = gb.gemm355_gemm_ex(*args)
            if st != gb.OK:
                raise gb.Gemm355Error(st, "gemm355_gemm_ex")
        runs.append((v, gb.gemm355_kernel_desc_ex(*args[:-1]), go))
    for _, _, go in runs:
        for _ in range(warm):
            go()
    stream.synchronize()
    times = {v: [] for v, _, _ in runs}
    for _ in range(rounds):
        for v, _, go in runs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                go()
            e1.record(stream)
            stream.synchronize()
            times[v].append(e0.elapsed_time(e1) * 1e3 / reps)
    del dA, dB, dC
    return (float(np.median(times[alt])), float(np.median(times[gb.VARIANT_AUTO])), runs[0][1], runs[1][1])


def tile_lines(warm=300, rounds=5, reps=100):
    """Tile classes against what the dispatcher took before them, on calls it gives them:
    the 192 x 256 and 256 x 192 tiles against the 256 x 256 one (variant MFMA_T256X256),
    the two-per-CU 128 x 128 direct-to-LDS tile against the register-staged kernel (variant
    MFMA_STAGED128), and the direct-to-LDS tiles of small grids against the register-staged
    and 128 x 128 ones (variant MFMA_STAGED_SMALL).  Rounds: ceil(tiles / slots), the waves
    of resident work each grid takes (256 slots for one workgroup per CU, 512 for two)."""
    import torch

    from roofline_optimisation_amd import binding as gb

    cdiv = lambda a, b: -(-a // b)
    stream = torch.cuda.Stream()
    head = (f"U[-1,1] operands (seed 3), packed strides, FP32 C (16-bit with C_16; C += with ACCUMULATE); "
            f"{warm} warm-up launches per case, then both cases interleaved, median of {rounds} rounds of "
            f"{reps} launches; HIP events.")
    out = ["# Tile classes of the 16-bit direct-to-LDS kernel on one MI355X", "", head, "",
           "## 192 x 256 and 256 x 192 against 256 x 256 tiles", "", "Rounds = ceil(tiles / 256 CUs).", "",
           "| dtype | M x N x K | flags | 256x256 tiles (rounds) | dispatched tiles (rounds) | 256x256 µs | "
           "dispatched µs | speedup | TFLOP/s | % of peak | dispatched kernel |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for dt, M, N, K, fl in TILE_SHAPES:
        sq, dis, _, kd = _time_pair(dt, M, N, K, fl, gb.VARIANT_MFMA_T256X256, warm, rounds, reps, stream)
        t256 = cdiv(M, 256) * cdiv(N, 256)
        t192 = cdiv(M, 256) * cdiv(N, 192) if "256x192" in kd else cdiv(M, 192) * cdiv(N, 256)
        tf = 2.0 * M * N * K / dis / 1e6
        fl_text = " \\| ".join(fl) or "plain"
        out.append(f"| {dt} | {M}x{N}x{K} | {fl_text} | {t256} ({cdiv(t256, 256)}) | {t192} ({cdiv(t192, 256)}) | "
                   f"{sq:.2f} | {dis:.2f} | {sq / dis:.3f}x | {tf:.0f} | {100 * tf / PEAKS[dt]:.1f} | "
                   f"`{md_cell(kd)}` |")
        log(f"[tiles] {dt} {M}x{N}x{K} {'|'.join(fl) or 'plain'}: 256x256 {sq:.2f} us, "
            f"dispatched {dis:.2f} us ({sq / dis:.3f}x)")
    out += ["", "## 128 x 128 direct-to-LDS tiles two per CU against the register-staged kernel", "",
            "Both run 128 x 128 tiles, two workgroups per CU (512 slots); the direct-to-LDS kernel on a 4-stage "
            "ring (64 KiB of LDS).", "",
            "| dtype | M x N x K | flags | 128x128 tiles (rounds) | register-staged µs | dispatched µs | speedup | "
            "TFLOP/s | % of peak | register-staged kernel | dispatched kernel |",
            "|---|---|---|---|---|---|---|---|---|---|---|"]
    for dt, M, N, K, fl in RING4_SHAPES:
        st, dis, ks, kd = _time_pair(dt, M, N, K, fl, gb.VARIANT_MFMA_STAGED128, warm, rounds, reps, stream)
        t128 = cdiv(M, 128) * cdiv(N, 128)
        tf = 2.0 * M * N * K / dis / 1e6
        fl_text = " \\| ".join(fl) or "plain"
        out.append(f"| {dt} | {M}x{N}x{K} | {fl_text} | {t128} ({cdiv(t128, 512)}) | {st:.2f} | {dis:.2f} | "
                   f"{st / dis:.3f}x | {tf:.0f} | {100 * tf / PEAKS[dt]:.1f} | `{md_cell(ks)}` | `{md_cell(kd)}` |")
        log(f"[tiles] {dt} {M}x{N}x{K} {'|'.join(fl) or 'plain'}: staged {st:.2f} us, "
            f"dispatched {dis:.2f} us ({st / dis:.3f}x)")
    out += ["", "## Direct-to-LDS tiles of small grids against the kernels they replaced", "",
            "The 64 x 64 direct-to-LDS tile (8-stage ring, or 4-stage for K from 128 to 255) where the 128 x 128 "
            "grid leaves CUs idle and the 64 x 64 one fits one round of two per CU; the 128 x 128 direct-to-LDS tile "
            "for plain products past that; the 4-stage ring for K from 128 to 255.  Before: variant "
            "`mfma_staged_small`.", "",
            "| dtype | M x N x K | flags | before µs | dispatched µs | speedup | TFLOP/s | % of peak | "
            "kernel before | dispatched kernel |",
            "|---|---|---|---|---|---|---|---|---|---|"]
    for dt, M, N, K, fl in SMALL_SHAPES:
        st, dis, ks, kd = _time_pair(dt, M, N, K, fl, gb.VARIANT_MFMA_STAGED_SMALL, warm, rounds, reps, stream)
        tf = 2.0 * M * N * K / dis / 1e6
        fl_text = " \\| ".join(fl) or "plain"
        out.append(f"| {dt} | {M}x{N}x{K} | {fl_text} | {st:.2f} | {dis:.2f} | {st / dis:.3f}x | {tf:.0f} | "
                   f"{100 * tf / PEAKS[dt]:.1f} | `{md_cell(ks)}` | `{md_cell(kd)}` |")
        log(f"[tiles] {dt} {M}x{N}x{K} {'|'.join(fl) or 'plain'}: before {st:.2f} us, "
            f"dispatched {dis:.2f} us ({st / dis:.3f}x)")
    return out


def general_form_lines():
    """Markdown lines timing gemm355_gemm_ex (transposed / negated operands, accumulation)
    at the headline sizes, against the plain product."""
    import numpy as np
    import torch

    from roofline_optimisation_amd import binding as gb
    from roofline_optimisation_amd import inputs

    lines = ["", "## General form C = s op(A) op(B) (+ C) (`gemm355_gemm_ex`)", "",
             "op(A) = A^T means A is stored K x M, op(B) = B^T means B is stored N x K.  TFLOP/s",
             "counts 2MNK (the addition of the old C is not counted).  Negated and accumulating",
             "calls run the kernels' signed variants, which store sign * acc (+ C); \"16-bit C\" keeps",
             "C in the operands' type (GEMM355_C_16: half the bytes written).  Every case is",
             "warmed, then the cases are timed interleaved (3 rounds of 100 launches after 20",
             "untimed ones); the table gives the median round.", "",
             "| dtype | n | layout | mode | kernel path | time (us) | TFLOP/s | % of peak | vs plain NN |",
             "|---|---|---|---|---|---|---|---|---|"]
    stream = torch.cuda.Stream()
    for dt, n, seed in (("f32", 3072, 1), ("f16", 4096, 3)):
        A, B = inputs.make_operands(n, n, n, seed, "uniform", dt)
        conv = (lambda x: torch.from_numpy(x).cuda()) if dt == "f32" else \
            (lambda x: torch.from_numpy(x.view("int16")).cuda())
        dA, dB = conv(np.ascontiguousarray(A)), conv(np.ascontiguousarray(B))
        dAt, dBt = conv(np.ascontiguousarray(A.T)), conv(np.ascontiguousarray(B.T))
        dC = torch.zeros((n, n), dtype=torch.float32, device="cuda")
        dC16 = torch.zeros((n, n), dtype=torch.int16, device="cuda")
        modes = [("plain", 0), ("negated", gb.NEG_A), ("accumulate", gb.ACCUMULATE)]
        if dt != "f32":
            modes += [("16-bit C", gb.C_16), ("16-bit C, accumulate", gb.C_16 | gb.ACCUMULATE)]
        cases = []
        for layout, (ta, tb) in (("NN", (0, 0)), ("NT", (0, 1)), ("TN", (1, 0)), ("TT", (1, 1))):
            for mode, extra in modes:
                flags = (gb.TRANS_A if ta else 0) | (gb.TRANS_B if tb else 0) | extra
                a = dAt if ta else dA
                b = dBt if tb else dB
                c = dC16 if extra & gb.C_16 else dC
                cases.append((layout, mode, (gb.VARIANT_AUTO, gb.DTYPE_CODES[dt], flags, n, n, n,
                                             a.data_ptr(), n, b.data_ptr(), n, c.data_ptr(), n,
                                             stream.cuda_stream)))

        def go(args, reps):
            for _ in range(reps):
                st = gb.gemm355_gemm_ex(*args)
                if st != gb.OK:
                    raise gb.Gemm355Error(st, "gemm355_gemm_ex")
        # the clock settles over the first few hundred launches: warm every case, then
        # time the cases interleaved, 3 rounds of 100 launches each, and keep the median
        for _, _, args in cases:
            go(args, 30)
        times = {i: [] for i in range(len(cases))}
        for _ in range(3):
            for i, (_, _, args) in enumerate(cases):
                go(args, 20)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                go(args, 100)
                e1.record(stream)
                stream.synchronize()
                times[i].append(e0.elapsed_time(e1) / 100)
        base = sorted(times[0])[1]
        for i, (layout, mode, _) in enumerate(cases):
            ms = sorted(times[i])[1]
            tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
            path = {"plain": "plain", "16-bit C": "16-bit C variant",
                    "16-bit C, accumulate": "16-bit C variant"}.get(mode, "signed / accumulating variant")
            lines.append(f"| {dt} | {n} | {layout} | {mode} | {path} | {ms * 1e3:.1f} | {tf:.1f} | "
                         f"{100 * tf / PEAKS[dt]:.1f} | {base / ms:.2f} |")
            log(f"[report] ex {dt} {n} {layout} {mode}: {ms * 1e3:.1f} us {tf:.1f} TFLOP/s")
        del dA, dB, dAt, dBt, dC, dC16
    return lines


def time_launches(go, stream, warm=50, rounds=3, reps=100):
    """Median over `rounds` of the mean per-launch time (ms) of `reps` back-to-back calls
    of go(), timed with HIP events on `stream`, after `warm` untimed calls."""
    import torch
    for _ in range(warm):
        go()
    times = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            go()
        e1.record(stream)
        stream.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    return sorted(times)[len(times) // 2]


SOFTMAX_ROTATE = 5  # buffer pairs cycled per workload: 5 x 2 x 256 MiB, ten times the MALL


def softmax_measure(warm=50, reps=100):
    """Per-launch time and algorithmic bandwidth of gemm355_softmax_f32 (4 bytes read and
    4 written per element) and gemm355_row_sum_f32 (4 bytes read per element, 4 written
    per row) on every softmax workload.

    The primary figures cycle through SOFTMAX_ROTATE input / output buffer pairs (the
    same seeded values, different addresses), so that no launch finds its data in the
    256 MB last-level cache (MALL) and the rate is HBM's.  The secondary figures re-use
    one pair, as a loop over a single resident tensor would: then part of the traffic
    is served by the MALL."""
    import torch

    from roofline_optimisation_amd import binding as gb
    from roofline_optimisation_amd import inputs

    stream = torch.cuda.Stream()
    h = stream.cuda_stream
    out = []
    for rows, cols in SOFTMAX_SHAPES:
        X = inputs.make_logits(rows, cols, 7, "normal")
        dX0 = torch.from_numpy(X).cuda()
        dX = [dX0] + [dX0.clone() for _ in range(SOFTMAX_ROTATE - 1)]
        dY = [torch.empty_like(dX0) for _ in range(SOFTMAX_ROTATE)]
        dS = [torch.empty(rows, dtype=torch.float32, device="cuda") for _ in range(SOFTMAX_ROTATE)]
        torch.cuda.synchronize()
        state = {"i": 0, "rotate": True}

        def nxt():
            i = state["i"]
            if state["rotate"]:
                state["i"] = (i + 1) % SOFTMAX_ROTATE
            return i

        def sm():
            i = nxt()
            st = gb.gemm355_softmax_f32(rows, cols, dX[i].data_ptr(), cols, dY[i].data_ptr(), cols, h)
            if st != gb.OK:
                raise gb.Gemm355Error(st, "gemm355_softmax_f32")

        def rs():
            i = nxt()
            st = gb.gemm355_row_sum_f32(rows, cols, dX[i].data_ptr(), cols, dS[i].data_ptr(), h)
            if st != gb.OK:
                raise gb.Gemm355Error(st, "gemm355_row_sum_f32")
        n = rows * cols
        res = {}
        for name, fn, nbytes in (("sm", sm, 8.0 * n), ("rs", rs, 4.0 * n + 4 * rows)):
            state.update(i=0, rotate=True)
            ms = time_launches(fn, stream, warm, 3, reps)
            state.update(i=0, rotate=False)
            ms_warm = time_launches(fn, stream, 0, 3, reps)
            res[name] = (ms, nbytes / (ms * 1e-3) / 1e9, nbytes / (ms_warm * 1e-3) / 1e9)
        r = {"rows": rows, "cols": cols, "ms": res["sm"][0], "gbs": res["sm"][1],
             "gbs_warm": res["sm"][2], "ms_sum": res["rs"][0], "gbs_sum": res["rs"][1],
             "gbs_sum_warm": res["rs"][2],
             "path": "two passes (row streamed twice)" if cols > 32768 else "row held in registers",
             "X": X if (rows, cols) == SOFTMAX_SHAPES[0] else None}
        log(f"[softmax] {rows}x{cols}: {r['ms'] * 1e3:.1f} us, {r['gbs']:.0f} GB/s "
            f"({100 * r['gbs'] / HBM_PEAK_GBS:.1f}% of 8 TB/s; one resident pair: {r['gbs_warm']:.0f}); "
            f"row sum {r['ms_sum'] * 1e3:.1f} us, {r['gbs_sum']:.0f} GB/s (resident: {r['gbs_sum_warm']:.0f})")
        out.append(r)
        del dX, dY, dS, dX0
    return out


def softmax_lines(res):
    lines = ["", "## Row-wise softmax and row sum (`gemm355_softmax_f32`, `gemm355_row_sum_f32`)", "",
             "Binary32 logits, N(0, 1), seed 7, packed rows, 64 Mi elements per workload.",
             "Algorithmic bytes: softmax 4 read + 4 written per element; row sum 4 read per",
             "element + 4 written per row.  Per-launch time: median of 3 rounds of 100 launches",
             f"after 50 warm-up launches, HIP events on the launch stream, cycling through {SOFTMAX_ROTATE}",
             "buffer pairs (same values, 2.5 GiB in all) so the data comes from HBM; the 'resident'",
             "columns re-use one pair, whose 256 MiB the 256 MB MALL then partly serves.", "",
             "| rows x cols | softmax path | softmax (us) | GB/s | % of 8 TB/s | resident GB/s | row sum (us) | GB/s | % of 8 TB/s | resident GB/s |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for r in res:
        lines.append(f"| {r['rows']} x {r['cols']} | {r['path']} | {r['ms'] * 1e3:.1f} | {r['gbs']:.0f} | "
                     f"{100 * r['gbs'] / HBM_PEAK_GBS:.1f} | {r['gbs_warm']:.0f} | {r['ms_sum'] * 1e3:.1f} | "
                     f"{r['gbs_sum']:.0f} | {100 * r['gbs_sum'] / HBM_PEAK_GBS:.1f} | {r['gbs_sum_warm']:.0f} |")
    return lines


def softmax_cpu_baseline(X, min_seconds=10.0):
    """The oracle's softmax on this host: the first 1024 rows of the workload, repeated
    until at least `min_seconds` of wall time, as algorithmic GB/s (8 bytes per element)."""
    import oracle
    sample = np.ascontiguousarray(X[:1024])
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.softmax(sample)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    n = sample.size * reps
    return {"value": round(8.0 * n / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} passes over the first 1024 rows ({sample.shape[0]}x{sample.shape[1]}) "
                      f"of the same seeded workload, {dt:.1f} s wall"}


def memory_slope_lines():
    """Markdown lines for the memory-slope probe: HBM read bandwidth against resident waves
    per CU and bytes in flight per wave, dependent-load latency, and the Little's-law
    in-flight requirement that follows from them."""
    import numpy as np
    import torch

    from roofline_optimisation_amd import binding as gb
    from roofline_optimisation_amd import roofline as rl

    stream = torch.cuda.Stream()
    h = stream.cuda_stream
    n_bytes = 2 << 30                      # 2 GiB: 8x the 256 MB MALL
    src = torch.empty(n_bytes // 4, dtype=torch.int32, device="cuda")
    src.random_()
    part = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def read_rate(vec, unroll, threads, lds, grid, reps=4):
        def go():
            st = gb.gemm355_stream(gb.STREAM_READ_XOR, src.data_ptr(), part.data_ptr(), n_bytes,
                                   vec, unroll, threads, lds, grid, h)
            if st != gb.OK:
                raise gb.Gemm355Error(st, "gemm355_stream")
        go()
        stream.synchronize()
        e0.record(stream)
        for _ in range(reps):
            go()
        e1.record(stream)
        stream.synchronize()
        return n_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    # resident waves per CU set by workgroup size and LDS reservation (160 KiB per CU)
    occ = [(1, 64, 163840), (2, 128, 163840), (4, 256, 163840), (8, 256, 81920),
           (16, 256, 40960), (32, 256, 20480)]
    ilp = [(4, 1), (16, 1), (16, 4)]
    rows, best = [], 0.0
    for waves, threads, lds in occ:
        wg_per_cu = 163840 // lds
        grid = 256 * wg_per_cu
        for vec, unroll in ilp:
            gbps = read_rate(vec, unroll, threads, lds, grid)
            inflight = waves * 64 * vec * unroll
            rows.append((waves, vec, unroll, inflight, gbps))
            best = max(best, gbps)
            log(f"[report] stream read: {waves} waves/CU vec {vec} unroll {unroll}: {gbps:.0f} GB/s")

    # copy (read + write) at the same occupancies, 16-byte vectors, one load in flight,
    # with ordinary and with non-temporal stores
    dst = torch.empty_like(src)
    copy_rows = []
    for waves, threads, lds in occ:
        grid = 256 * (163840 // lds)
        rates = []
        for mode in (gb.STREAM_COPY, gb.STREAM_COPY_NT):
            def go():
                st = gb.gemm355_stream(mode, src.data_ptr(), dst.data_ptr(), n_bytes, 16, 1,
                                       threads, lds, grid, h)
                if st != gb.OK:
                    raise gb.Gemm355Error(st, "gemm355_stream")
            go()
            stream.synchronize()
            e0.record(stream)
            for _ in range(3):
                go()
            e1.record(stream)
            stream.synchronize()
            rates.append(2 * n_bytes * 3 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        copy_rows.append((waves, rates[0], rates[1]))
        log(f"[report] stream copy: {waves} waves/CU: {rates[0]:.0f} GB/s, non-temporal stores "
            f"{rates[1]:.0f} GB/s (read + write)")
    del dst

    # dependent-load latency: one lane walks a random cycle through stride-aligned word
    # positions of a table; `warm` walks the whole cycle first, `flush` streams the 2 GiB
    # source first so that no level of cache holds the table
    def chase(table_bytes, nodes, stride, hops, warm=False, flush=False):
        nw = table_bytes // 4
        gen = torch.Generator(device="cuda")
        gen.manual_seed(5)
        pos = torch.randperm(nw // stride, device="cuda", generator=gen)[:nodes].to(torch.int64) * stride
        table = torch.zeros(nw, dtype=torch.int32, device="cuda")
        table[pos] = torch.roll(pos, -1).to(torch.int32)
        out = torch.zeros(2, dtype=torch.int64, device="cuda")
        start = int(pos[0])
        def walk(k):
            st = gb.gemm355_chase(table.data_ptr(), nw, start, k, out.data_ptr(), h)
            if st != gb.OK:
                raise gb.Gemm355Error(st, "gemm355_chase")
        res = []
        for _ in range(3):
            if warm:
                walk(nodes)
            if flush:
                read_rate(16, 1, 256, 20480, 2048, reps=1)
            e0.record(stream)
            walk(hops)
            e1.record(stream)
            stream.synchronize()
            res.append((e0.elapsed_time(e1) * 1e6 / hops, int(out[1].item()) / hops))
        del table
        return min(res)
    lat_l2 = chase(64 << 20, 2048, 1024, 4000, warm=True)           # 256 KB of lines
    lat_mall = chase(64 << 20, 65536, 256, 65536, warm=True)        # 8 MB of lines > L2
    lat_hbm = chase(2 << 30, 65536, 1024, 4000, flush=True)
    for name, lat in (("L2", lat_l2), ("MALL", lat_mall), ("HBM", lat_hbm)):
        log(f"[report] chase {name}: {lat[0]:.0f} ns/hop {lat[1]:.0f} cycles")

    need = best * 1e9 * lat_hbm[0] * 1e-9                     # bytes in flight (chip)
    clock_ghz = lat_hbm[1] / lat_hbm[0]
    need_cycles = rl.littles_law_bytes(lat_hbm[1], best * 1e9, clock_ghz * 1e9)
    sat = min((r for r in rows if r[4] >= 0.9 * best), key=lambda r: r[3])
    lines = ["", "## Memory slope (Little's law and occupancy probe)", "",
             "HBM read bandwidth of `gemm355_stream` (mode READ_XOR) over a 2 GiB source (8x the 256 MB",
             "MALL), against resident waves per CU (set by workgroup size and LDS reservation out of",
             "160 KiB per CU) and bytes in flight per wave (64 lanes x vector bytes x loads issued before",
             "first use).  Mean of 4 passes after one warm pass.", "",
             "| waves/CU | occupancy (of 32) | vec B | loads in flight | in-flight B per CU | GB/s | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|"]
    for waves, vec, unroll, inflight, gbps in rows:
        lines.append(f"| {waves} | {100 * waves / 32:.1f} % | {vec} | {unroll} | {inflight} | {gbps:.0f} | "
                     f"{100 * gbps / 8000:.1f} |")
    lines += ["", "Copy (`gemm355_stream` modes COPY and COPY_NT, 16-byte vectors, one load in flight per "
              "lane; read + write bytes; COPY_NT stores non-temporally):", "",
              "| waves/CU | occupancy (of 32) | COPY GB/s | % of best COPY | COPY_NT GB/s | % of 8 TB/s |",
              "|---|---|---|---|---|---|"]
    cbest = max(g for _, g, _ in copy_rows)
    for waves, gbps, gnt in copy_rows:
        lines.append(f"| {waves} | {100 * waves / 32:.1f} % | {gbps:.0f} | {100 * gbps / cbest:.0f} % | "
                     f"{gnt:.0f} | {100 * gnt / 8000:.1f} |")
    lines += ["", "Dependent-load latency (`gemm355_chase`: one lane walks a random cycle; minimum of 3 runs):", "",
              "| level | table, cycle | preparation | ns per hop | shader cycles per hop |", "|---|---|---|---|---|",
              f"| L2 | 64 MiB, 2048 nodes (256 KB of lines), 4000 hops | one warm walk | {lat_l2[0]:.0f} | {lat_l2[1]:.0f} |",
              f"| MALL | 64 MiB, 65536 nodes (8 MB of lines > 4 MB L2), 65536 hops | one warm walk | {lat_mall[0]:.0f} | {lat_mall[1]:.0f} |",
              f"| HBM | 2 GiB, 65536 nodes 4 KiB apart, 4000 hops | 2 GiB streamed first | {lat_hbm[0]:.0f} | {lat_hbm[1]:.0f} |", "",
              f"Little's law with these numbers: best measured read rate {best:.0f} GB/s x HBM latency "
              f"{lat_hbm[0]:.0f} ns = {need / 1e6:.2f} MB in flight for the chip "
              f"({need / 256 / 1e3:.1f} KB per CU; {need_cycles / 1e6:.2f} MB by the page's cycles x "
              f"bytes-per-cycle form at the chase's {clock_ghz:.2f} GHz).  The smallest configuration "
              f"within 90 % of the best rate: {sat[0]} waves/CU with {sat[3]} B in flight per CU "
              f"({sat[3] * 256 / 1e6:.2f} MB for the chip), {sat[4]:.0f} GB/s."]
    del src
    return lines


def write_report(path):
    from roofline_optimisation_amd import inputs
    from roofline_optimisation_amd import roofline as rl

    names = {0: "naive", 1: "lds_tiled", 2: "regblock", 3: "mfma"}
    lines = ["# libgemm355 measurements on one MI355X", "",
             "Made by `python3 bench.py --no-cpu-baseline --warmup 50 --steps 50 --report PATH` from the",
             "repository root (the report's own cases; `--steps` and `--warmup` set only the JSON line's run).", "",
             "Per-launch time from HIP events on one stream (mean over >= 3 launches after about 50 ms",
             "of untimed launches of the same case),",
             "U[-1,1] operands, packed row-major strides.  TFLOP/s = 2MNK / t.  Peaks: FP32 157.3,",
             "FP16/BF16 2516.6 TFLOP/s (2.4 GHz datasheet); attainable = min(peak, OI x 8 TB/s)",
             "with OI = 2MNK / ideal bytes (each operand read once, C written once).", "",
             "## Kernel families, FP32", "",
             "| workload | family | kernel | reps | time (us) | TFLOP/s | % of FP32 peak |",
             "|---|---|---|---|---|---|---|"]
    for (n, seed) in ((256, 0), (3072, 1)):
        for v in (0, 1, 2, 3):
            ms, desc, reps = time_variant(v, "f32", n, n, n, seed)
            tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
            lines.append(f"| FP32 {n}^3 | {names[v]} | {md_cell(desc)} | {reps} | {ms * 1e3:.1f} | {tf:.2f} | "
                         f"{100 * tf / PEAKS['f32']:.1f} |")
            log(f"[report] f32 {n} {names[v]}: {ms * 1e3:.1f} us {tf:.2f} TFLOP/s")
    lines += ["", "## Roofline sweep (dispatched kernels)", "",
              "| dtype | M x N x K | kernel | time (us) | TFLOP/s | % of peak | OI (FLOP/B) | "
              "attainable TFLOP/s | bound |", "|---|---|---|---|---|---|---|---|---|"]
    chart_points = []
    for c in inputs.sweep_cases():
        ms, desc, reps = time_variant(-1, c.dtype, c.M, c.N, c.K, c.seed)
        tf = 2.0 * c.M * c.N * c.K / (ms * 1e-3) / 1e12
        e = rl.roofline_entry(c.M, c.N, c.K, ms * 1e-3, c.dtype)
        chart_points.append((e["oi"], tf, "f" if c.dtype == "f32" else "b"))
        bound = "HBM" if e["attainable_tflops"] < e["peak_tflops"] else "compute"
        lines.append(f"| {c.dtype} | {c.M}x{c.N}x{c.K} | {md_cell(desc)} | {ms * 1e3:.1f} | {tf:.1f} | "
                     f"{100 * e['frac']:.1f} | {e['oi']:.1f} | {e['attainable_tflops']:.0f} | {bound} |")
        log(f"[report] {c.name}: {ms * 1e3:.1f} us {tf:.1f} TFLOP/s")
    lines += ["", "Roofline chart of the sweep (f: FP32 points, b: BF16 points; roofs min(peak, OI x 8 TB/s): "
              "'=' BF16 2516.6 TFLOP/s, '-' FP32 157.3 TFLOP/s):", "", "```"]
    lines += rl.text_chart(chart_points, [(PEAKS["bf16"], "="), (PEAKS["f32"], "-")], 8e12)
    lines += ["```"]
    # Context only, not a target: the analytic figures "Advanced CUDA features - starting
    # from GEMM" works through (roofline section) for its RTX 4000 Ada, recomputed from
    # the peak and bandwidth it states.
    ada_peak, ada_bw = 26.7e12, 360e9
    lines += ["", "## Context: the pages' analytic RTX 4000 Ada figures (not a target)", "",
              f"Peak {ada_peak / 1e12:.1f} TFLOP/s FP32, {ada_bw / 1e9:.0f} GB/s: ridge "
              f"{rl.ridge(ada_peak, ada_bw):.2f} FLOP/B, compute-bound time for the 3072^3 product "
              f"{rl.compute_time(3072, 3072, 3072, ada_peak) * 1e3:.2f} ms (this library on one MI355X: "
              f"see the FP32 3072^3 rows above)."]
    lines += general_form_lines()
    lines += softmax_lines(softmax_measure())
    lines += memory_slope_lines()
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--only", choices=["f32", "f16", "bf16"], default=None,
                    help="measure one workload only (for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--report", default=None, metavar="PATH",
                    help="also time every kernel family on the 256^3 and 3072^3 FP32 workloads "
                         "and the square FP32/BF16 sweep plus the tall-skinny shape, and write a "
                         "markdown table to PATH (the JSON line is unchanged)")
    ap.add_argument("--memory-slope", default=None, metavar="PATH",
                    help="only run the memory-slope probe (HBM read rate against occupancy and "
                         "bytes in flight, dependent-load latency) and write its markdown table "
                         "to PATH; no GEMM timing, no JSON line")
    ap.add_argument("--softmax", default=None, metavar="PATH",
                    help="only measure the row-wise softmax and row sum on their 64 Mi-element "
                         "workloads, write the markdown table to PATH and print one JSON line "
                         "for the 16384 x 4096 workload; no GEMM timing")
    ap.add_argument("--family", choices=["naive", "lds_tiled", "regblock", "mfma", "mfma_split",
                                         "mfma_w8", "mfma_t256x128", "mfma_t256x256", "mfma_staged128", "mfma_staged_small"], default=None,
                    help="only launch one kernel family (--warmup untimed and --steps timed "
                         "launches, for counter passes) on the FP32 3072^3 workload, or with "
                         "--family-dtype f16/bf16 on the n^3 16-bit workload (seed 3); no JSON line")
    ap.add_argument("--family-dtype", choices=["f32", "f16", "bf16"], default="f32")
    ap.add_argument("--family-n", type=int, default=0,
                    help="square size for --family (default 3072 for f32, 4096 for f16/bf16)")
    ap.add_argument("--family-m", type=int, default=0,
                    help="rows of A and C for --family (default --family-n: a square product)")
    ap.add_argument("--schedules", default=None, metavar="PATH",
                    help="only time the schedules of the FP16 direct-to-LDS kernel (dispatched, "
                         "producer/consumer split, eight waves, 256 x 128 tiles) at 4096^3 and "
                         "8192^3, interleaved, and write the markdown table to PATH")
    ap.add_argument("--tiles", default=None, metavar="PATH",
                    help="only time the 192 x 256 direct-to-LDS tile against the 256 x 256 one, and "
                         "the two-per-CU 128 x 128 direct-to-LDS tile against the register-staged "
                         "kernel, on calls the dispatcher gives them, interleaved, and write the "
                         "markdown tables to PATH")
    ap.add_argument("--ragged-k", default=None, metavar="PATH",
                    help="only time BF16 n x n x K on the direct-to-LDS kernel (n = 4096 and "
                         "2048; K not a whole number of ring trips, A's rows packed, padded or "
                         "off the 128-byte lines), interleaved, and write the markdown table "
                         "(time per FLOP against K = n) to PATH")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the GEMMs, copy this many MiB device-to-device once (a plain "
                         "copy of known size, used to scale the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): "
              "this library is a single-GPU GEMM (a multi-GPU product would give each GPU a "
              "block of rows of A and C and all of B, and run this same call on each)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    from roofline_optimisation_amd import roofline as rl

    if args.memory_slope:
        lines = ["# libgemm355 memory-slope probe on one MI355X"] + memory_slope_lines()
        with open(args.memory_slope, "w") as f:
            f.write("\n".join(lines) + "\n")
        log(f"[bench] memory-slope table written to {args.memory_slope}")
        return

    def calibration_copy():
        if args.calib_copy_mib:
            nel = args.calib_copy_mib * (1 << 20) // 4
            src = torch.ones(nel, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
            log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")

    if args.family:
        family_run(args.family, args.steps, args.warmup, args.family_dtype, args.family_n, args.family_m)
        calibration_copy()
        return

    if args.ragged_k:
        with open(args.ragged_k, "w") as f:
            f.write("\n".join(ragged_k_lines(warm=max(args.warmup, 1))) + "\n")
        log(f"[bench] ragged-K table written to {args.ragged_k}")
        return

    if args.tiles:
        with open(args.tiles, "w") as f:
            f.write("\n".join(tile_lines(warm=max(args.warmup, 1))) + "\n")
        log(f"[bench] tile table written to {args.tiles}")
        return

    if args.schedules:
        with open(args.schedules, "w") as f:
            f.write("\n".join(schedule_lines(warm=max(args.warmup, 1))) + "\n")
        log(f"[bench] schedule table written to {args.schedules}")
        return

    if args.softmax:
        warm, reps = min(args.warmup, 50), max(1, min(args.steps, 100))
        res = softmax_measure(warm=warm, reps=reps)
        with open(args.softmax, "w") as f:
            f.write("\n".join(["# libgemm355 row-wise softmax on one MI355X"] + softmax_lines(res)) + "\n")
        calibration_copy()
        r = res[0]
        tr = measured_traffic("softmax")
        line = {
            "metric": "row-wise softmax, algorithmic HBM bandwidth (8 bytes per element), 1 MI355X",
            "value": round(r["gbs"], 1), "unit": "GB/s", "n_gpus": 1, "steps": 3 * reps, "warmup": warm,
            "ms_per_step": round(r["ms"], 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"softmax_f32_{r['rows']}x{r['cols']}", "rows": r["rows"],
                       "cols": r["cols"], "dist": "N(0,1)", "seed": 7,
                       "buffers": f"{SOFTMAX_ROTATE} input/output pairs cycled (data from HBM)",
                       "resident_one_pair_gbs": round(r["gbs_warm"], 1)},
            "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(r["gbs"] / HBM_PEAK_GBS, 4), "traffic": tr,
                         "algorithmic_bytes": 8 * r["rows"] * r["cols"],
                         "kernel": "softmax_rows_kernel<32, 2, 1, vec> (32 elements per lane, 2 waves per row)"},
        }
        if not args.no_cpu_baseline:
            log("[softmax] timing the CPU oracle (at least 10 s)")
            line["cpu_baseline"] = softmax_cpu_baseline(r["X"])
        print(json.dumps(line), flush=True)
        return

    results = {}
    # BF16 4096^3 (the FP16 workload's values rounded to bfloat16) only on request: the
    # same kernel as FP16, for comparing clock and matrix-core use between the formats
    for kind, n, seed in (("f32", 3072, 1), ("f16", 4096, 3), ("bf16", 4096, 3)):
        if (args.only and args.only != kind) or (not args.only and kind == "bf16"):
            continue
        log(f"[bench] {kind} {n}^3: warmup {args.warmup}, steps {args.steps}")
        r = time_gemm(kind, n, n, n, seed, args.steps, args.warmup)
        tf = 2.0 * n ** 3 / (r["ms"] * 1e-3) / 1e12
        r["tflops"] = tf
        results[kind] = r
        log(f"[bench] {kind} {n}^3 {r['desc']}: {r['ms']:.4f} ms/launch, {tf:.1f} TFLOP/s "
            f"({100 * tf / PEAKS[kind]:.1f}% of {PEAKS[kind]})")

    if args.report:
        write_report(args.report)

    calibration_copy()

    def roof(kind, n):
        r = results[kind]
        tr = measured_traffic(kind) if kind in PMC_FILES else None
        in_b = 4 if kind == "f32" else 2
        return {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": PEAKS[kind],
                "unit": "TFLOP/s", "frac": round(r["tflops"] / PEAKS[kind], 4),
                "traffic": tr, "algorithmic_flops": 2 * n ** 3,
                "ideal_bytes": rl.ideal_bytes(n, n, n, in_b, 4), "kernel": r["desc"]}

    main_kind = "f32" if "f32" in results else ("f16" if "f16" in results else "bf16")
    n = 3072 if main_kind == "f32" else 4096
    r = results[main_kind]
    line = {
        "metric": "GEMM TFLOPS (2MNK/s) + % of peak: FP32 n=3072, FP16->FP32 n=4096, 1 MI355X",
        "value": round(r["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16->f32", "bf16": "bf16->f32"}[main_kind],
        "data": "synthetic",
        "config": {"workload": f"gemm_{main_kind}_{n}", "M": n, "N": n, "K": n,
                   "layout": "row-major, packed strides", "dist": "U[-1,1]",
                   "seed": 1 if main_kind == "f32" else 3, "kernel": r["desc"]},
        "roofline": roof(main_kind, n),
    }
    if main_kind == "f32" and "f16" in results:
        f = results["f16"]
        line["fp16_n4096"] = {"value": round(f["tflops"], 2), "unit": "TFLOP/s",
                              "ms_per_step": round(f["ms"], 5), "frac": round(f["tflops"] / PEAKS["f16"], 4),
                              "roofline": roof("f16", 4096)}
    if not args.no_cpu_baseline and main_kind == "f32":
        log("[bench] timing the CPU oracle (full steps, at least 10 s)")
        line["cpu_baseline"] = cpu_baseline(r["A"], r["B"], n, n, n)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
