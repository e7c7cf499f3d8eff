"""Pins of the oracle's general form C = s op(A) op(B) (+ C_in).

The operation is the one the tensor-core instruction table of "Advanced CUDA features -
starting from GEMM" lists for its warp-group MMA (D = A*B + D; A, B transposed or
negated; D scaled by 0 or 1).  Each pin checks ``oracle.gemm_ex`` against something
computed another way:
  * exact rational arithmetic (fractions.Fraction) with explicit index maps, for every
    one of the 32 flag combinations and several tiny shapes;
  * a non-symmetric permutation matrix, whose transpose moves rows the other way;
  * small-integer operands against numpy int64 products of explicitly transposed
    operands (bit-exact);
  * planted mistakes in oracle.c, each caught by at least one pin.
"""

from __future__ import annotations

import itertools
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle

FLAGS = list(itertools.product([False, True], repeat=5))  # ta, tb, na, nb, acc


def stored(op: np.ndarray, trans: bool) -> np.ndarray:
    """The stored matrix whose op() is `op`."""
    return np.ascontiguousarray(op.T) if trans else np.ascontiguousarray(op)


def _rne32(q: Fraction) -> float:
    """Round an exact rational to the nearest binary32 (ties to even)."""
    f = float(q)                        # nearest binary64
    lo = np.float32(f)
    cands = {np.float32(lo), np.nextafter(lo, np.float32(np.inf)), np.nextafter(lo, np.float32(-np.inf))}
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.frombuffer(np.float32(c).tobytes(), np.uint32)[0]) & 1))
    return float(best)


def pin_ex_brute_force(lib):
    rng = np.random.default_rng(21)
    for (M, N, K) in [(1, 1, 1), (2, 3, 4), (3, 2, 5), (4, 4, 1), (1, 5, 3)]:
        opA = rng.uniform(-1, 1, (M, K)).astype(np.float32)
        opB = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        Cin = rng.uniform(-1, 1, (M, N)).astype(np.float32)
        for ta, tb, na, nb, acc in FLAGS:
            C64, C32 = oracle.gemm_ex(stored(opA, ta), stored(opB, tb), "f32", ta, tb, na, nb,
                                      Cin if acc else None, lib=lib)
            s = -1 if na != nb else 1
            for i in range(M):
                for j in range(N):
                    exact = Fraction(0)
                    mag = Fraction(0)
                    for k in range(K):
                        t = Fraction(float(opA[i, k])) * Fraction(float(opB[k, j]))
                        exact += t
                        mag += abs(t)
                    exact = s * exact + (Fraction(float(Cin[i, j])) if acc else 0)
                    bound = (K + 1) * 2.0 ** -53 * (float(mag) + (abs(float(Cin[i, j])) if acc else 0))
                    assert abs(C64[i, j] - float(exact)) <= bound + 1e-300, (M, N, K, ta, tb, na, nb, acc)
                    want = _rne32(exact)
                    got = float(C32[i, j])
                    assert got == want or abs(got - want) <= float(np.spacing(np.float32(want))), \
                        (M, N, K, ta, tb, na, nb, acc, got, want)


def pin_ex_permutation(lib):
    # P[i][perm[i]] = 1: (P B)[i] = B[perm[i]];  (P^T B)[i] = B[inv[i]]
    perm = np.array([2, 0, 3, 1, 4])
    inv = np.argsort(perm)
    P = np.zeros((5, 5), np.float32)
    P[np.arange(5), perm] = 1
    B = np.arange(5 * 3, dtype=np.float32).reshape(5, 3) - 7
    _, plain = oracle.gemm_ex(P, B, lib=lib)
    assert np.array_equal(plain, B[perm])
    _, tr = oracle.gemm_ex(P, B, trans_a=True, lib=lib)      # stored P, op(A) = P^T
    assert np.array_equal(tr, B[inv])
    # B stored transposed: op(B) = S^T for stored S = B^T
    _, tb = oracle.gemm_ex(P, np.ascontiguousarray(B.T), trans_b=True, lib=lib)
    assert np.array_equal(tb, B[perm])
    _, neg = oracle.gemm_ex(P, B, neg_b=True, C_in=np.ones((5, 3), np.float32), lib=lib)
    assert np.array_equal(neg, 1 - B[perm])


def pin_ex_integers(lib):
    rng = np.random.default_rng(22)
    for dt in ("f32", "f16", "bf16"):
        M, N, K = 7, 9, 13
        ia = rng.integers(-4, 5, (M, K))
        ib = rng.integers(-4, 5, (K, N))
        ic = rng.integers(-50, 51, (M, N))
        def enc(x):
            if dt == "f32":
                return x.astype(np.float32)
            if dt == "f16":
                return x.astype(np.float16).view(np.uint16)
            return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        for ta, tb, na, nb, acc in FLAGS:
            s = -1 if na != nb else 1
            want = s * (ia @ ib) + (ic if acc else 0)
            _, C32 = oracle.gemm_ex(enc(stored(ia, ta)), enc(stored(ib, tb)), dt, ta, tb, na, nb,
                                    ic.astype(np.float32) if acc else None, lib=lib)
            assert np.array_equal(C32, want.astype(np.float32)), (dt, ta, tb, na, nb, acc)


PINS = [pin_ex_brute_force, pin_ex_permutation, pin_ex_integers]


@pytest.fixture(scope="module")
def oracle_lib():
    return oracle._load()


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_plain_form_equals_gemm(oracle_lib):
    """No flags: the same products in the same order as oracle.gemm, bit for bit."""
    rng = np.random.default_rng(23)
    A = rng.uniform(-1, 1, (33, 17)).astype(np.float32)
    B = rng.uniform(-1, 1, (17, 29)).astype(np.float32)
    a64, a32 = oracle.gemm(A, B)
    b64, b32 = oracle.gemm_ex(A, B)
    assert np.array_equal(a64, b64) and np.array_equal(a32, b32)


MUTATIONS = {
    "ex_ignores_transpose": ("trans ? dec(src, (size_t)c * ld + r) : dec(src, (size_t)r * ld + c);",
                             "dec(src, (size_t)r * ld + c);"),
    "ex_sign_from_a_only": ("((neg_a != 0) != (neg_b != 0)) ? -1.0 : 1.0",
                            "(neg_a != 0) ? -1.0 : 1.0"),
    "ex_drops_c": ("if (accumulate) v += (double)Cin[(size_t)i * ldc + j];",
                   "if (0) v += (double)Cin[(size_t)i * ldc + j];"),
    "ex_sign_on_c_too": ("double v = s * C64[(size_t)i * ldc + j];\n            if (accumulate) v += (double)Cin[(size_t)i * ldc + j];",
                         "double v = C64[(size_t)i * ldc + j];\n            if (accumulate) v += (double)Cin[(size_t)i * ldc + j];\n            v *= s;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    csrc = tmp_path / "mut.c"
    csrc.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    from oracle import build as ob
    subprocess.run(["gcc", *ob.CFLAGS, str(csrc), "-o", str(so), "-lm"], check=True)
    here = os.path.dirname(os.path.abspath(__file__))
    code = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle, test_oracle_ex as t\n"
        "lib = oracle.load_library(%r)\n"
        "for pin in t.PINS:\n"
        "    try:\n"
        "        pin(lib)\n"
        "    except AssertionError:\n"
        "        print('CAUGHT', pin.__name__)\n"
    ) % (os.path.dirname(here), here, str(so))
    res = subprocess.run(["python", "-c", code], capture_output=True, text=True, timeout=300)
    caught = [ln.split()[1] for ln in res.stdout.splitlines() if ln.startswith("CAUGHT")]
    assert res.returncode == 0, res.stderr[-2000:]
    assert caught, f"no pin caught the planted mistake {name}"
