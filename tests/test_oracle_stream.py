"""Pins of the memory-slope probe oracle (XOR of a word stream, dependent-index walk).

The probes of the Little's-law and occupancy section of "Advanced CUDA features -
starting from GEMM" move data; what they must return is fixed by definition.  Each pin
checks the oracle against something computed another way: the closed form of
0 ^ 1 ^ ... ^ m, per-bit parity counted with numpy, cancellation of duplicated words,
closed-form positions on successor and permutation cycles, and the out-of-range clamp
(through a table longer than the n words the walk may use).  Planted mistakes in
oracle.c must each be caught by at least one pin.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle


def xor_upto(m: int) -> int:
    """0 ^ 1 ^ ... ^ m, by the period-4 closed form."""
    return [m, 1, m + 1, 0][m % 4]


def pin_xor_closed_form(lib):
    for n in (1, 2, 3, 4, 5, 6, 7, 8, 1000, 4099, 1 << 20):
        got = oracle.stream_xor(np.arange(n, dtype=np.uint32), lib=lib)
        assert got == xor_upto(n - 1), (n, got)
    assert oracle.stream_xor(np.zeros(0, np.uint32), lib=lib) == 0


def pin_xor_bit_parity(lib):
    rng = np.random.default_rng(11)
    w = rng.integers(0, 2**32, size=100_003, dtype=np.uint64).astype(np.uint32)
    bits = np.unpackbits(w.view(np.uint8).reshape(-1, 4), axis=1, bitorder="little")
    parity = bits.sum(axis=0) % 2                      # bit 8*byte + k of each word
    expect = int(sum(int(p) << i for i, p in enumerate(parity)))
    assert oracle.stream_xor(w, lib=lib) == expect


def pin_xor_pairs_cancel(lib):
    rng = np.random.default_rng(12)
    w = rng.integers(0, 2**32, size=5000, dtype=np.uint64).astype(np.uint32)
    both = rng.permutation(np.concatenate([w, w]))
    assert oracle.stream_xor(both, lib=lib) == 0
    extra = np.uint32(0xDEADBEEF)
    assert oracle.stream_xor(np.concatenate([both, [extra]]), lib=lib) == int(extra)


def pin_chase_successor(lib):
    n = 1000
    nxt = ((np.arange(n) + 1) % n).astype(np.uint32)
    for start, hops in ((0, 1), (5, 999), (17, 1000), (999, 12345)):
        assert oracle.chase(nxt, start, hops, lib=lib) == (start + hops) % n


def pin_chase_permutation_cycle(lib):
    rng = np.random.default_rng(13)
    n = 4096
    order = rng.permutation(n)
    nxt = np.zeros(n, np.uint32)
    nxt[order] = np.roll(order, -1)
    for p, hops in ((0, 1), (10, 4095), (100, 4096), (7, 10_000)):
        assert oracle.chase(nxt, int(order[p]), hops, lib=lib) == int(order[(p + hops) % n])
    assert oracle.chase(nxt, 3, 0, lib=lib) == 3


def pin_chase_clamp(lib):
    # the table is 16 words long but the walk may only use the first 8: an entry of 12
    # must become 7, not the (in-memory) word 12
    nxt = np.array([12, 0, 0, 0, 0, 0, 0, 2, 0, 0, 0, 0, 5, 0, 0, 0], np.uint32)
    assert oracle.chase(nxt, 0, 1, n=8, lib=lib) == 7
    assert oracle.chase(nxt, 0, 2, n=8, lib=lib) == 2
    # 0 -> 3 (0xFFFFFFFF clamped to n - 1) -> 1 -> 3
    nxt2 = np.array([0xFFFFFFFF, 3, 3, 1], np.uint32)
    assert oracle.chase(nxt2, 0, 3, lib=lib) == 3


PINS = [pin_xor_closed_form, pin_xor_bit_parity, pin_xor_pairs_cancel, pin_chase_successor,
        pin_chase_permutation_cycle, pin_chase_clamp]


@pytest.fixture(scope="module")
def oracle_lib():
    return oracle._load()


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


# Plausible slips in the probe functions of oracle.c; at least one pin must fail on each.
MUTATIONS = {
    "xor_as_or": ("for (int64_t i = 0; i < n; ++i) x ^= w[i];", "for (int64_t i = 0; i < n; ++i) x |= w[i];"),
    "xor_drops_last": ("for (int64_t i = 0; i < n; ++i) x ^= w[i];", "for (int64_t i = 0; i + 1 < n; ++i) x ^= w[i];"),
    "chase_extra_hop": ("for (int64_t h = 0; h < hops; ++h) {", "for (int64_t h = 0; h <= hops; ++h) {"),
    "chase_no_clamp": ("cur = (int64_t)v < n ? v : (uint32_t)(n - 1);", "cur = v;"),
    "chase_clamps_to_zero": ("cur = (int64_t)v < n ? v : (uint32_t)(n - 1);", "cur = (int64_t)v < n ? v : 0;"),
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
        "import oracle, test_oracle_stream as t\n"
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
