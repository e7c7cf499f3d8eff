"""The seeded input generator: determinism, stream prefixes and storage rounding."""

import hashlib

import numpy as np
import pytest

from roofline_optimisation_amd import inputs

# SHA-256 prefixes of A||B recorded when the recipe was fixed; a change here means the
# synthetic workloads changed.
DIGESTS = {
    "f32_256": "56ac2f22bd24a1a6",
    "f32_256_int": "fba5c0e5c109c05a",
    "f32_1023x997x515": "9f1a72b5f3dc0cfb",
}


@pytest.mark.parametrize("name", sorted(DIGESTS))
def test_digests(name):
    A, B = inputs.operands_for(inputs.CASES[name])
    assert hashlib.sha256(A.tobytes() + B.tobytes()).hexdigest()[:16] == DIGESTS[name]


def test_half_digests():
    A, B = inputs.make_operands(64, 32, 48, 3, "uniform", "f16")
    assert hashlib.sha256(A.tobytes() + B.tobytes()).hexdigest()[:16] == "66b12c3ed295e6f5"
    A, B = inputs.make_operands(64, 32, 48, 4, "uniform", "bf16")
    assert hashlib.sha256(A.tobytes() + B.tobytes()).hexdigest()[:16] == "b294174e5808473f"


@pytest.mark.parametrize("dist", ["uniform", "normal", "int"])
def test_draw_rows_is_a_prefix(dist):
    A, _ = inputs.make_operands(50, 7, 33, 9, dist, "f32")
    assert np.array_equal(inputs.draw_rows(50, 33, 9, dist, "f32", rows=17), A[:17])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_uniform_pieces_equal_one_draw(monkeypatch, dtype):
    """Large U[-1,1] matrices are drawn in pieces; the values must be those of one draw
    (here with pieces of 1000 elements, not a divisor of either operand's size)."""
    A1, B1 = inputs.make_operands(61, 47, 83, 11, "uniform", dtype)
    monkeypatch.setattr(inputs, "UNIFORM_CHUNK", 1000)
    A2, B2 = inputs.make_operands(61, 47, 83, 11, "uniform", dtype)
    assert np.array_equal(A1, A2) and np.array_equal(B1, B2)
    assert np.array_equal(inputs.draw_rows(61, 83, 11, "uniform", dtype, rows=29), A1[:29])


def test_ranges():
    A, B = inputs.make_operands(100, 90, 80, 1, "uniform")
    assert A.dtype == np.float32 and A.min() >= -1 and A.max() <= 1
    A, _ = inputs.make_operands(100, 90, 80, 1, "int")
    assert set(np.unique(A).tolist()) <= set(range(-4, 5))


def test_bf16_round_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing just above 1
    x = np.array([one, one + ulp / 2, one + 1.5 * ulp, one + 0.75 * ulp, -one - ulp / 4,
                  3.0e38], np.float32)
    bits = inputs.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back[0] == 1.0
    assert back[1] == 1.0                 # tie -> even
    assert back[2] == one + 2 * ulp       # tie -> even (odd neighbour below)
    assert back[3] == one + ulp           # above half -> up
    assert back[4] == -1.0
    assert np.isfinite(back[5])


def test_bf16_pieces_match_wide_arithmetic(monkeypatch):
    """The piecewise uint32 rounding equals RNE done in uint64 on the whole array, for
    every sign and exponent (extreme finite values and infinities included)."""
    rng = np.random.default_rng(5)
    x = np.concatenate([
        (rng.standard_normal(5000) * np.exp(rng.uniform(-80, 80, 5000))).astype(np.float32),
        np.array([np.finfo(np.float32).max, -np.finfo(np.float32).max, np.inf, -np.inf,
                  0.0, -0.0, 1e-45, -1e-45], np.float32)])
    u = x.view(np.uint32).astype(np.uint64)
    ref = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    monkeypatch.setattr(inputs, "UNIFORM_CHUNK", 777)
    assert np.array_equal(inputs.f32_to_bf16_bits(x), ref)


def test_f16_matches_numpy():
    x = np.random.default_rng(0).uniform(-1, 1, 1000).astype(np.float32)
    assert np.array_equal(inputs.f32_to_f16_bits(x).view(np.float16), x.astype(np.float16))


def test_embed():
    x = np.arange(6, dtype=np.float32).reshape(2, 3)
    e = inputs.embed(x, 5, extra_rows=1)
    assert e.shape == (3, 5) and np.array_equal(e[:2, :3], x) and np.isnan(e[:, 3:]).all()
    h = inputs.embed(np.ones((2, 2), np.uint16), 3)
    assert h[0, 2] == 0x7E00


def test_make_logits_recipe():
    a = inputs.make_logits(4, 9, 5, "normal")
    assert a.dtype == np.float32 and a.shape == (4, 9)
    assert np.array_equal(a, inputs.make_logits(4, 9, 5, "normal"))
    assert np.array_equal(a, np.random.default_rng(5).standard_normal((4, 9)).astype(np.float32))
    up = inputs.make_logits(3, 20, 6, "ascending")
    assert np.all(np.diff(up, axis=1) >= 0)
    down = inputs.make_logits(3, 20, 6, "descending")
    assert np.array_equal(down, up[:, ::-1])
    w = inputs.make_logits(2, 1000, 7, "wide")
    assert np.abs(w).max() > 89.0  # e^x would overflow binary32
    i = inputs.make_logits(2, 50, 8, "int")
    assert np.array_equal(i, np.round(i)) and np.abs(i).max() <= 4
    with pytest.raises(ValueError):
        inputs.make_logits(1, 1, 0, "bogus")
