"""Pins of the oracle's row-wise softmax (the online recurrence of "Kernel optimisation
guide", section on softmax optimisation) and row sum (its section on warp-shuffle
reduction).

The pages print no worked softmax values, so each pin checks ``oracle.softmax`` /
``oracle.row_sum`` against something computed another way:
  * the definition y_i = e^{x_i} / sum_j e^{x_j} evaluated with Python's ``decimal`` at
    50 significant digits (no max shift: decimal's exponent range is wide enough), on
    rows whose maximum rises at every element, never after the first, or at random,
    and on rows whose raw exponentials overflow binary64;
  * closed forms: a constant row gives exactly 1/n (m = the constant, l = n); one
    element gives 1; a two-element row is the logistic function of the difference; an
    element 2000 above the rest takes everything;
  * shift invariance (integer rows shifted by an integer give bit-identical results);
  * independence of rows and of the row stride (NaN padding never read);
  * sums of small integers exactly; sums of binary32 values against exact rationals;
  * planted mistakes in oracle.c, each caught by at least one pin.
"""

from __future__ import annotations

import math
import os
import shutil
import subprocess
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from roofline_optimisation_amd import inputs

U53 = 2.0 ** -53


def exact_softmax(row):
    """The definition at 50 digits: returns (y as Decimals, max, sum of e^{x - max})."""
    with localcontext() as ctx:
        ctx.prec = 50
        xs = [Decimal(float(v)) for v in row]
        es = [x.exp() for x in xs]
        tot = sum(es, Decimal(0))
        mx = max(xs)
        lsum = sum(((x - mx).exp() for x in xs), Decimal(0))
        return [e / tot for e in es], mx, lsum


def f32_near(got: float, exact: Decimal) -> bool:
    """binary32 result equal to the RNE of `exact`, or within one ulp of it (the result
    is rounded twice: to binary64, then to binary32)."""
    want = np.float32(float(exact))
    return got == float(want) or abs(got - float(want)) <= float(np.spacing(want))


def pin_softmax_decimal(lib):
    for dist, seed in (("normal", 31), ("wide", 32), ("ascending", 33), ("descending", 34),
                       ("uniform", 35)):
        for cols in (1, 2, 3, 7, 16, 33):
            X = inputs.make_logits(3, cols, seed + cols, dist)
            Y64, Y32, m, l = oracle.softmax(X, lib=lib)
            assert np.isfinite(Y64).all() and np.isfinite(l).all() and np.isfinite(m).all(), (dist, cols)
            for r in range(X.shape[0]):
                ys, mx, lsum = exact_softmax(X[r])
                assert m[r] == float(mx), (dist, cols, r)
                assert abs(Decimal(l[r]) - lsum) <= Decimal((4 * cols + 8) * U53) * lsum, (dist, cols, r)
                for i, y in enumerate(ys):
                    bound = Decimal((4 * cols + 8) * U53) * y + Decimal(1e-300)
                    assert abs(Decimal(Y64[r, i]) - y) <= bound, (dist, cols, r, i, Y64[r, i], y)
                    assert f32_near(float(Y32[r, i]), y), (dist, cols, r, i)


def pin_softmax_closed_forms(lib):
    for n in (1, 2, 3, 5, 8, 64, 100, 1000):
        for c in (0.0, 3.5, -100.0, 1e4):
            X = np.full((2, n), c, np.float32)
            Y64, Y32, m, l = oracle.softmax(X, lib=lib)
            assert np.all(Y64 == 1.0 / n) and np.all(Y32 == np.float32(1.0 / n)), (n, c)
            assert np.all(m == np.float32(c)) and np.all(l == n), (n, c)
    # two elements: the logistic function of the difference
    rng = np.random.default_rng(36)
    for _ in range(50):
        a, b = rng.standard_normal(2).astype(np.float32) * 5
        Y64, _, _, _ = oracle.softmax(np.array([[a, b]], np.float32), lib=lib)
        want = 1.0 / (1.0 + math.exp(float(b) - float(a)))
        assert abs(Y64[0, 0] - want) <= 8 * U53 * want, (a, b)
        assert abs(Y64[0, 1] - (1.0 - want)) <= 8 * U53 + 8 * U53 * (1 - want), (a, b)
    # one element far above the rest takes everything (e^-2000 underflows binary64)
    X = np.full((1, 9), -2000.0, np.float32)
    X[0, 4] = 0.0
    Y64, Y32, m, l = oracle.softmax(X, lib=lib)
    assert Y64[0, 4] == 1.0 and np.all(np.delete(Y64[0], 4) == 0.0) and l[0] == 1.0


def pin_softmax_shift_and_rows(lib):
    X = inputs.make_logits(5, 300, 37, "int")
    base, b32, bm, bl = oracle.softmax(X, lib=lib)
    for c in (1.0, -37.0, 1000.0):
        Y64, _, m, l = oracle.softmax(X + np.float32(c), lib=lib)
        assert np.array_equal(Y64, base) and np.array_equal(l, bl) and np.array_equal(m, bm + c), c
    # each row on its own, and inside a NaN-padded buffer, gives the same bits
    W = inputs.make_logits(6, 45, 38, "normal")
    full, _, _, _ = oracle.softmax(W, lib=lib)
    for r in range(W.shape[0]):
        one, _, _, _ = oracle.softmax(W[r:r + 1].copy(), lib=lib)
        assert np.array_equal(one[0], full[r]), r
    padded = inputs.embed(W, 45 + 11)
    Yp, _, _, _ = oracle.softmax(padded[:, :45], lib=lib)
    assert np.array_equal(Yp, full) and not np.isnan(Yp).any()
    # every row sums to 1 (exactly summed), and permuting a row permutes its outputs
    assert np.all(np.abs(np.array([math.fsum(r) for r in full]) - 1.0) <= (4 * 45 + 8) * U53)
    perm = np.random.default_rng(39).permutation(45)
    Yq, _, _, _ = oracle.softmax(np.ascontiguousarray(W[:, perm]), lib=lib)
    assert np.all(np.abs(Yq - full[:, perm]) <= (8 * 45 + 16) * U53 * full[:, perm])


def pin_row_sum(lib):
    # small integers: every partial sum is an integer, so the sums are exact
    X = inputs.make_logits(7, 1001, 40, "int")
    S64, S32 = oracle.row_sum(X, lib=lib)
    want = [sum(int(v) for v in r) for r in X]
    assert list(S64) == want and list(S32) == [float(w) for w in want]
    # binary32 values against their exact rational sum
    for cols in (1, 2, 17, 640):
        X = inputs.make_logits(4, cols, 41 + cols, "uniform")
        S64, S32 = oracle.row_sum(X, lib=lib)
        for r in range(4):
            ex = sum((Fraction(float(v)) for v in X[r]), Fraction(0))
            mag = sum(abs(float(v)) for v in X[r])
            assert abs(Fraction(S64[r]) - ex) <= Fraction(max(cols - 1, 0) * U53 * mag), (cols, r)
            with localcontext() as ctx:
                ctx.prec = 50
                exd = Decimal(ex.numerator) / Decimal(ex.denominator)
            assert f32_near(float(S32[r]), exd), (cols, r)
    # an empty row sums to +0.0; a padded buffer is read only within the rows
    S64, _ = oracle.row_sum(np.zeros((3, 0), np.float32), lib=lib)
    assert np.all(S64 == 0.0) and not np.signbit(S64).any()
    X = inputs.make_logits(5, 33, 42, "normal")
    a, _ = oracle.row_sum(X, lib=lib)
    b, _ = oracle.row_sum(inputs.embed(X, 40)[:, :33], lib=lib)
    assert np.array_equal(a, b)


PINS = [pin_softmax_decimal, pin_softmax_closed_forms, pin_softmax_shift_and_rows, pin_row_sum]


@pytest.fixture(scope="module")
def oracle_lib():
    return oracle._load()


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_argument_errors(oracle_lib):
    lib = oracle_lib
    assert lib.oracle_softmax(-1, 3, None, 3, None, None, 3, None, None) == 1
    assert lib.oracle_softmax(2, 3, None, 2, None, None, 3, None, None) == 1
    assert lib.oracle_softmax(2, 3, None, 3, None, None, 2, None, None) == 1
    assert lib.oracle_row_sum(2, 3, None, 2, None, None) == 1
    assert lib.oracle_softmax(0, 3, None, 3, None, None, 3, None, None) == 0


MUTATIONS = {
    "softmax_no_rescale": ("l *= exp(m - v);", "(void)0;"),
    "softmax_rescale_sign": ("l *= exp(m - v);", "l *= exp(v - m);"),
    "softmax_max_not_updated": ("m = v;", "(void)v;"),
    "softmax_normalise_unshifted": ("const double y = exp((double)x[i] - m) / l;",
                                    "const double y = exp((double)x[i]) / l;"),
    "softmax_row_stride": ("const float *x = X + (size_t)r * ldx;\n        double m = -INFINITY;",
                           "const float *x = X + (size_t)r * cols;\n        double m = -INFINITY;"),
    "row_sum_drops_last": ("for (int i = 0; i < cols; ++i) s += (double)x[i];",
                           "for (int i = 0; i + 1 < cols; ++i) s += (double)x[i];"),
    "row_sum_binary32": ("double s = 0.0;", "float s = 0.0f;"),
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
        "import oracle, test_oracle_softmax as t\n"
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
