"""Pins of the oracle's general form with C stored in the operands' 16-bit type
(``oracle.gemm_ex16``: D = A*B + D of the tensor-core instruction table of "Advanced
CUDA features - starting from GEMM", whose type for D the table leaves open, kept in
binary16 / bfloat16), and of its rounding of binary64 values to those formats.

  * binary16 rounding against numpy's float64 -> float16 conversion (which rounds the
    binary64 value directly, to nearest with ties to even) on random values across the
    whole range, on every midpoint between neighbouring binary16 values, and on values
    just beside those midpoints;
  * bfloat16 rounding against an exact rational reference written here (the two
    neighbours on the bfloat16 grid, nearest wins, ties to the even one), on random
    values, midpoints, subnormals, overflow, and double-rounding traps (a value that
    rounds differently through binary32 first);
  * small-integer products: C16 is the rounding of the exact integer;
  * sums just above a 16-bit midpoint that binary32 would put on it (rounded once);
  * accumulation reads the old C in the 16-bit type;
  * planted mistakes in oracle.c, each caught.
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
from roofline_optimisation_amd import inputs


def ref_round_bits(v: float, p: int, emin: int, ebias: int) -> int:
    """Exact rational reference: the bit pattern of v rounded to nearest, ties to even,
    on the grid of a binary format with p significant bits, smallest normal exponent
    emin and exponent bias ebias (8-bit exponent field for bfloat16, 5-bit for binary16)."""
    ebits = 8 if ebias == 127 else 5
    emax = (1 << ebits) - 2 - ebias
    sign = 0x8000 if np.signbit(v) else 0
    x = abs(Fraction(v))
    if x == 0:
        return sign
    lead = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** lead > x:
        lead -= 1
    q = max(lead, emin) - (p - 1)
    unit = Fraction(2) ** q
    k = x / unit                     # position on the grid
    lo = k.numerator // k.denominator
    rem = k - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * unit
    maxfin = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > maxfin:
        return sign | (((1 << ebits) - 1) << (p - 1))
    if lo < (1 << (p - 1)) and q == emin - (p - 1):     # subnormal (or rounded up to min normal)
        return sign | int(lo) if lo < (1 << (p - 1)) else sign | (1 << (p - 1))
    lead2 = lead if lo < (1 << p) else lead + 1
    lead2 = max(lead2, emin)
    mant = int(r / Fraction(2) ** (lead2 - (p - 1))) - (1 << (p - 1))
    return sign | ((lead2 + ebias) << (p - 1)) | mant


def decode16(bits: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_cases(rng):
    vals = [rng.uniform(1, 2, 4000) * 2.0 ** rng.integers(-30, 17, 4000) * rng.choice([-1, 1], 4000)]
    h = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = (np.arange(0, 0x7C00, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    mid = (h + nxt) / 2                                   # exact in binary64
    vals += [mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)]
    vals += [np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                       3 * 2.0 ** -26, 2.0 ** -26, 1e-300, 6.1e-5])]
    return np.concatenate(vals)


def pin_f16_rounding(lib):
    x = f16_cases(np.random.default_rng(70))
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = oracle.f64_to_f16_bits(x, lib=lib)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(x[i], hex(got[i]), hex(want[i])) for i in bad[:5]]
    # the exact reference agrees with numpy on a sample (both are direct roundings)
    for v in x[::97]:
        assert ref_round_bits(float(v), 11, -14, 15) == int(np.float16(v).view(np.uint16)), v


def pin_bf16_rounding(lib):
    rng = np.random.default_rng(71)
    x = [rng.uniform(1, 2, 3000) * 2.0 ** rng.integers(-140, 128, 3000) * rng.choice([-1, 1], 3000)]
    ones = 1.0 + np.arange(0, 256) * 2.0 ** -8          # every midpoint and grid point near 1
    x += [ones, -ones, np.nextafter(ones, 2), np.nextafter(ones, 0)]
    x += [np.array([0.0, -0.0, 1 + 2.0 ** -8 + 2.0 ** -30, 1 + 3 * 2.0 ** -8, 3.3895313892515355e38,
                    3.3961775292304e38, 3.40e38, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135,
                    2.0 ** -126, (2 - 2.0 ** -7) * 2.0 ** -127])]
    x = np.concatenate(x)
    got = oracle.f64_to_bf16_bits(x, lib=lib)
    for v, g in zip(x, got):
        assert int(g) == ref_round_bits(float(v), 8, -126, 127), (v, hex(int(g)))
    # a double-rounding trap: through binary32 this would tie and go to even (1.0)
    assert oracle.f64_to_bf16_bits([1 + 2.0 ** -8 + 2.0 ** -30], lib=lib)[0] == 0x3F81


def pin_ex16_integers(lib):
    rng = np.random.default_rng(72)
    for dt, (p, emin, bias) in (("f16", (11, -14, 15)), ("bf16", (8, -126, 127))):
        M, N, K = 6, 7, 40
        ia = rng.integers(-4, 5, (M, K))
        ib = rng.integers(-4, 5, (K, N))
        ic = rng.integers(-60, 61, (M, N))
        enc = (lambda z: inputs.to_storage(z.astype(np.float32), dt))
        for ta, tb, na, nb, acc in itertools.product([False, True], repeat=5):
            s = -1 if na != nb else 1
            want = s * (ia @ ib) + (ic if acc else 0)
            SA = enc(ia.T.copy() if ta else ia)
            SB = enc(ib.T.copy() if tb else ib)
            C64, C16 = oracle.gemm_ex16(SA, SB, dt, ta, tb, na, nb, enc(ic) if acc else None, lib=lib)
            assert np.array_equal(C64, want.astype(np.float64)), (dt, ta, tb, na, nb, acc)
            ref = np.array([[ref_round_bits(float(w), p, emin, bias) for w in row] for row in want])
            # values, not zero signs: a negated product summing to 0 is -0.0
            assert np.array_equal(decode16(C16, dt), decode16(ref.astype(np.uint16), dt)), \
                (dt, ta, tb, na, nb, acc)


def pin_ex16_values(lib):
    """Random operands: C16 is the direct rounding of the binary64 value s sum + old C."""
    for dt, (p, emin, bias) in (("f16", (11, -14, 15)), ("bf16", (8, -126, 127))):
        A, B = inputs.make_operands(9, 11, 13, 73, "uniform", dt)
        Cin = inputs.to_storage(np.random.default_rng(74).uniform(-2, 2, (9, 11)).astype(np.float32), dt)
        C64, C16 = oracle.gemm_ex16(A, B, dt, False, False, True, False, Cin, lib=lib)
        plain, _ = oracle.gemm_ex(A, B, dt)
        assert np.array_equal(C64, -plain + decode16(Cin, dt)), dt
        ref = np.array([[ref_round_bits(float(v), p, emin, bias) for v in row] for row in C64])
        assert np.array_equal(C16, ref.astype(np.uint16)), dt


def pin_ex16_single_rounding(lib):
    """Sums that sit just above a midpoint of the 16-bit grid but on it in binary32:
    1 + 2^-11 + 2^-24 (binary16) and 1 + 2^-8 + 2^-30 (bfloat16) round up when rounded
    once, to 1.0 when rounded through binary32 first."""
    for dt, terms, want in (("f16", [1.0, 2.0 ** -11, 2.0 ** -24], 0x3C01),
                            ("bf16", [1.0, 2.0 ** -8, 2.0 ** -30], 0x3F81)):
        A = inputs.to_storage(np.array([terms], np.float32), dt)
        B = inputs.to_storage(np.ones((3, 1), np.float32), dt)
        _, C16 = oracle.gemm_ex16(A, B, dt, lib=lib)
        assert int(C16[0, 0]) == want, (dt, hex(int(C16[0, 0])))


PINS = [pin_f16_rounding, pin_bf16_rounding, pin_ex16_integers, pin_ex16_values,
        pin_ex16_single_rounding]


@pytest.fixture(scope="module")
def oracle_lib():
    return oracle._load()


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


MUTATIONS = {
    "round_truncates": ("return ldexp(nearbyint(ldexp(v, -q)), q);", "return ldexp(trunc(ldexp(v, -q)), q);"),
    "round_ties_away": ("return ldexp(nearbyint(ldexp(v, -q)), q);", "return ldexp(round(ldexp(v, -q)), q);"),
    "no_subnormal_floor": ("    if (lead < emin) lead = emin;\n    const int q", "    const int q"),
    "through_binary32": ("C16[at] = dtype == 1 ? oracle_f64_to_f16(v) : oracle_f64_to_bf16(v);",
                         "C16[at] = dtype == 1 ? oracle_f64_to_f16((float)v) : oracle_f64_to_bf16((float)v);"),
    "old_c_wrong_type": ("v += dtype == 1 ? oracle_f16_to_f64(Cin[at]) : oracle_bf16_to_f64(Cin[at]);",
                         "v += oracle_f16_to_f64(Cin[at]);"),
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
        "import oracle, test_oracle_ex16 as t\n"
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
