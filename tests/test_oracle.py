"""Pins of the CPU oracle against facts fixed outside it.

Every pin is a function ``pin_*(lib)`` so that the planted-mistake test can run the
same checks against deliberately broken builds of the oracle and show each mistake
is caught.  The facts used:

* hand-worked products stored under ``tests/golden/`` (definition C_ij = sum_k A_ik B_kj);
* identity and permutation matrices (exact by construction);
* small-integer inputs, whose product is an exact integer, against numpy int64 matmul;
* exact rational brute force (``fractions.Fraction``) for every M, N, K in 1..8;
* the transpose identity (B^T A^T)^T = A B, bit for bit (same products, same k order);
* strides: padded buffers whose padding is NaN give the packed result;
* the forward error bound against numpy's binary64 matmul (an independent routine);
* exhaustive binary16 / bfloat16 decoding against numpy's own conversions;
* degenerate sizes (K = 0 gives +0.0; M = 0 or N = 0 is a no-op; negative sizes fail).
"""

from __future__ import annotations

import ctypes
import os
import re
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from roofline_optimisation_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U53 = 2.0 ** -53


def gamma(n: int, u: float = U53) -> float:
    """Higham's gamma_n = n u / (1 - n u), the recursive-summation constant."""
    return n * u / (1.0 - n * u)


def read_matrices(path: str) -> dict[str, np.ndarray]:
    """Parse a fixture of blocks 'NAME rows cols' followed by rows of numbers."""
    mats: dict[str, np.ndarray] = {}
    lines = [ln.split("#", 1)[0].strip() for ln in open(path)]
    lines = [ln for ln in lines if ln]
    i = 0
    while i < len(lines):
        name, r, c = lines[i].split()
        r, c = int(r), int(c)
        rows = [[float(v) for v in lines[i + 1 + k].split()] for k in range(r)]
        mats[name] = np.array(rows, dtype=np.float64).reshape(r, c)
        i += 1 + r
    return mats


# --------------------------------------------------------------------------- pins

def pin_hand_worked(lib):
    for fname in ("hand_product_2x3x2.txt", "hand_product_3x2x4_signed.txt"):
        m = read_matrices(os.path.join(GOLDEN, fname))
        for dt in ("f32", "f16", "bf16"):
            A = inputs.to_storage(m["A"].astype(np.float32), dt)
            B = inputs.to_storage(m["B"].astype(np.float32), dt)
            c64, c32 = oracle.gemm(A, B, dt, lib=lib)
            assert np.array_equal(c64, m["C"]), (fname, dt, c64)
            assert np.array_equal(c32, m["C"].astype(np.float32)), (fname, dt)


def pin_identity(lib):
    rng = np.random.default_rng(11)
    A = rng.uniform(-1, 1, (5, 7)).astype(np.float32)
    c64, c32 = oracle.gemm(A, np.eye(7, dtype=np.float32), lib=lib)
    assert np.array_equal(c32, A) and np.array_equal(c64, A.astype(np.float64))
    c64, c32 = oracle.gemm(np.eye(5, dtype=np.float32), A, lib=lib)
    assert np.array_equal(c32, A)


def pin_permutation(lib):
    rng = np.random.default_rng(12)
    B = rng.uniform(-1, 1, (6, 9)).astype(np.float32)
    perm = np.array([3, 0, 5, 1, 4, 2])
    P = np.zeros((6, 6), np.float32)
    P[np.arange(6), perm] = 1.0                      # (P B)[r] = B[perm[r]]
    _, c32 = oracle.gemm(P, B, lib=lib)
    assert np.array_equal(c32, B[perm])
    A = rng.uniform(-1, 1, (4, 9)).astype(np.float32)
    q = np.array([8, 2, 6, 0, 1, 7, 3, 5, 4])
    Q = np.zeros((9, 9), np.float32)
    Q[q, np.arange(9)] = 1.0                         # (A Q)[:, c] = A[:, q[c]]
    _, c32 = oracle.gemm(A, Q, lib=lib)
    assert np.array_equal(c32, A[:, q])


def pin_small_integers(lib):
    # every partial sum is an integer of magnitude <= 16 K < 2^24: exact in any order
    for (M, N, K, seed) in ((1, 1, 1, 0), (7, 5, 3, 1), (37, 53, 129, 2), (64, 48, 4096, 3)):
        for dt in ("f32", "f16", "bf16"):
            A, B = inputs.make_operands(M, N, K, seed, "int", dt)
            Ai, Bi = inputs.make_operands(M, N, K, seed, "int", "f32")
            exact = Ai.astype(np.int64) @ Bi.astype(np.int64)
            c64, c32 = oracle.gemm(A, B, dt, lib=lib)
            assert np.array_equal(c64, exact.astype(np.float64)), (M, N, K, dt)
            assert np.array_equal(c32, exact.astype(np.float32)), (M, N, K, dt)


def _fraction_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational to binary32, round-to-nearest-even (normal range)."""
    if q == 0:
        return np.float32(0.0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    scaled = a / Fraction(2) ** (e - 23)             # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(s * float(m) * 2.0 ** (e - 23))


def pin_brute_force(lib):
    rng = np.random.default_rng(13)
    for M in range(1, 9):
        for N in range(1, 9):
            for K in range(1, 9):
                A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
                B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
                c64, c32 = oracle.gemm(A, B, lib=lib)
                Af = [[Fraction(float(v)) for v in row] for row in A]
                Bf = [[Fraction(float(v)) for v in row] for row in B]
                for i in range(M):
                    for j in range(N):
                        ex = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
                        mag = sum(abs(Af[i][k] * Bf[k][j]) for k in range(K))
                        err = abs(Fraction(float(c64[i, j])) - ex)
                        assert err <= Fraction(gamma(K - 1)) * mag, (M, N, K, i, j)
                        assert c32[i, j] == _fraction_to_f32(ex), (M, N, K, i, j)


def pin_transpose_identity(lib):
    A, B = inputs.make_operands(33, 21, 45, 5, "uniform", "f32")
    c64, _ = oracle.gemm(A, B, lib=lib)
    t64, _ = oracle.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), lib=lib)
    assert np.array_equal(t64.T, c64)


def pin_strides(lib):
    for dt in ("f32", "f16", "bf16"):
        A, B = inputs.make_operands(19, 23, 17, 6, "uniform", dt)
        c64, c32 = oracle.gemm(A, B, dt, lib=lib)
        Ap = inputs.embed(A, 29, extra_rows=3)[:19, :17]
        Bp = inputs.embed(B, 31, extra_rows=2)[:17, :23]
        p64, p32 = oracle.gemm(Ap, Bp, dt, lib=lib)
        assert np.array_equal(p64, c64) and not np.isnan(p64).any(), dt


def _decode(bits: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f32":
        return bits.astype(np.float64)
    if dt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_error_bound_vs_numpy(lib):
    for dt, (M, N, K) in (("f32", (64, 80, 300)), ("f16", (40, 72, 512)), ("bf16", (48, 40, 257))):
        A, B = inputs.make_operands(M, N, K, 7, "uniform", dt)
        c64, c32 = oracle.gemm(A, B, dt, lib=lib)
        a, b = _decode(A, dt), _decode(B, dt)
        ref = a @ b
        bound = 2 * gamma(K) * (np.abs(a) @ np.abs(b))
        assert np.all(np.abs(c64 - ref) <= bound), dt
        assert np.array_equal(c32, c64.astype(np.float32))


def pin_decoders(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = lib.oracle_f16_to_f64
    got = np.array([f(int(b)) for b in bits])
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan])
    g = lib.oracle_bf16_to_f64
    got = np.array([g(int(b)) for b in bits])
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan])


def pin_degenerate(lib):
    A = np.ones((3, 0), np.float32)
    B = np.ones((0, 4), np.float32)
    c64, c32 = oracle.gemm(A, B, lib=lib)
    assert c64.shape == (3, 4) and np.all(c64 == 0) and not np.signbit(c64).any()
    c64, _ = oracle.gemm(np.ones((0, 5), np.float32), np.ones((5, 4), np.float32), lib=lib)
    assert c64.shape == (0, 4)
    c64, _ = oracle.gemm(np.ones((3, 5), np.float32), np.ones((5, 0), np.float32), lib=lib)
    assert c64.shape == (3, 0)
    # all products cancel to an exact zero: +0.0, never -0.0
    c64, _ = oracle.gemm(np.array([[1.0, -1.0]], np.float32), np.array([[1.0], [1.0]], np.float32), lib=lib)
    assert c64[0, 0] == 0 and not np.signbit(c64[0, 0])
    buf = (ctypes.c_double * 4)()
    fbuf = (ctypes.c_float * 4)()
    assert lib.oracle_gemm_f32(-1, 1, 1, None, 1, None, 1, buf, fbuf, 1) == -1
    assert lib.oracle_gemm_f32(2, 2, 3, None, 2, None, 2, buf, fbuf, 2) == -1   # lda < K


PINS = [pin_hand_worked, pin_identity, pin_permutation, pin_small_integers, pin_brute_force,
        pin_transpose_identity, pin_strides, pin_error_bound_vs_numpy, pin_decoders,
        pin_degenerate]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_thread_count_does_not_change_result(tmp_path):
    """The row loop is split over threads; each element's sum is still in increasing k."""
    A, B = inputs.make_operands(97, 61, 389, 8, "normal", "f32")
    code = (
        "import sys, numpy as np; sys.path.insert(0, %r); import oracle;"
        "from roofline_optimisation_amd import inputs;"
        "A,B=inputs.make_operands(97,61,389,8,'normal','f32');"
        "c,_=oracle.gemm(A,B); np.save(%r, c)"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for t in (1, 3):
        out = str(tmp_path / f"c{t}.npy")
        env = dict(os.environ, OMP_NUM_THREADS=str(t))
        subprocess.run(["python", "-c", code % (root, out)], check=True, env=env)
        outs.append(np.load(out))
    c, _ = oracle.gemm(A, B)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], c)


# ----------------------------------------------------------- planted mistakes

# Each mutation is a plausible slip in oracle.c; at least one pin must fail on it.
MUTATIONS = {
    "drop_last_k": ("for (int k = 0; k < K; ++k)", "for (int k = 0; k < K - 1; ++k)"),
    "sign_flip": ("r[j] += a * brow[j]", "r[j] -= a * brow[j]"),
    "transposed_b": ("r[j] += a * brow[j]", "r[j] += a * B[(size_t)j * ldb + k]"),
    "no_row_reset": ("for (int j = 0; j < N; ++j) r[j] = 0.0;", ""),
    "ignores_lda": ("dec(src, (size_t)r * ld + c)", "dec(src, (size_t)r * cols + c)"),
    "f16_bias": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "f16_subnormal": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "bf16_shift": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    "c32_truncates": ("c32[j] = (float)r[j];", "c32[j] = nextafterf((float)r[j], 0.0f);"),
    "skips_first_k": ("const double a = arow[k];", "const double a = k ? arow[k] : 0.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    csrc = tmp_path / "mut.c"
    csrc.write_text(mutated)
    so = tmp_path / "libmut.so"
    from oracle import build as ob
    subprocess.run(["gcc", *ob.CFLAGS, str(csrc), "-o", str(so), "-lm"], check=True)
    # run the pins against the mutant in a child process: a mutant may read out of bounds
    here = os.path.dirname(os.path.abspath(__file__))
    code = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle, test_oracle\n"
        "lib = oracle.load_library(%r)\n"
        "for pin in test_oracle.PINS:\n"
        "    try:\n"
        "        pin(lib)\n"
        "    except (AssertionError, RuntimeError):\n"
        "        print('CAUGHT', pin.__name__)\n"
    ) % (os.path.dirname(here), here, str(so))
    res = subprocess.run(["python", "-c", code], capture_output=True, text=True, timeout=600)
    caught = [ln.split()[1] for ln in res.stdout.splitlines() if ln.startswith("CAUGHT")]
    assert res.returncode == 0, res.stderr[-2000:]
    assert caught, f"no pin caught the planted mistake {name}"


def test_mutation_anchors_are_distinct():
    """Guard the mutation table itself: each anchor names real code."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    for name, (old, _) in MUTATIONS.items():
        assert re.escape(old) and old in src, name
