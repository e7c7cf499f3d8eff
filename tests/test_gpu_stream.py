"""GPU parity of the memory-slope probes (Little's law and occupancy section of "Advanced
CUDA features - starting from GEMM") against the oracle, through the C ABI.

  * copy: the destination equals the source bit for bit, and the guard words on both
    sides of it keep their sentinel;
  * read XOR: the XOR of the per-workgroup entries equals the oracle's XOR of the whole
    source (which workgroup reads which word is not unique, the total is), and exactly
    `grid` entries are written;
  * chase: the index reached after `hops` dependent loads equals the oracle's walk,
    including the clamp of out-of-range entries.
Every configuration knob (vector width, loads in flight, workgroup size, LDS
reservation, grid) is exercised, with sizes that leave a ragged tail.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from roofline_optimisation_amd import binding as gb

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A
GUARD = 64  # words


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def words(n, seed):
    return np.random.default_rng(seed).integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)


def dev(a):
    import torch
    return torch.from_numpy(a.view(np.int32).copy()).cuda()


CONFIGS = [  # vec, unroll, threads, lds_bytes, grid
    (4, 1, 64, 0, 1), (16, 4, 256, 0, 256), (16, 8, 1024, 0, 7), (8, 2, 128, 40960, 300),
    (16, 1, 64, 163840, 256), (4, 8, 512, 20480, 1000), (8, 4, 256, 81920, 33),
]
SIZES = [0, 4, 4 * 1000, 16 * 64 * 8 * 3 + 4 * 37, (1 << 22) + 4 * 5]


@pytest.mark.parametrize("mode", [gb.STREAM_COPY, gb.STREAM_COPY_NT], ids=["copy", "copy_nt"])
@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "v{}u{}t{}l{}g{}".format(*c))
@pytest.mark.parametrize("n_bytes", SIZES)
def test_copy_bit_exact(cfg, n_bytes, mode):
    import torch
    vec, unroll, threads, lds, grid = cfg
    n = n_bytes // 4
    src = words(n, n + vec)
    d_src = dev(src)
    buf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.int32, device="cuda")
    dst_ptr = buf.data_ptr() + 4 * GUARD
    st = gb.gemm355_stream(mode, d_src.data_ptr() if n else 0, dst_ptr, n_bytes, vec,
                           unroll, threads, lds, grid, torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK
    torch.cuda.synchronize()
    out = buf.cpu().numpy().view(np.uint32)
    assert np.array_equal(out[GUARD:GUARD + n], src), f"copy {cfg} {n_bytes}"
    assert np.all(out[:GUARD] == SENTINEL) and np.all(out[GUARD + n:] == SENTINEL)


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "v{}u{}t{}l{}g{}".format(*c))
@pytest.mark.parametrize("n_bytes", SIZES)
def test_read_xor_matches_oracle(cfg, n_bytes):
    import torch
    vec, unroll, threads, lds, grid = cfg
    n = n_bytes // 4
    src = words(max(n, 1), 2 * n + vec)[:n]
    d_src = dev(src) if n else None
    buf = torch.full((grid + GUARD,), SENTINEL, dtype=torch.int32, device="cuda")
    st = gb.gemm355_stream(gb.STREAM_READ_XOR, d_src.data_ptr() if n else 0, buf.data_ptr(),
                           n_bytes, vec, unroll, threads, lds, grid,
                           torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK
    torch.cuda.synchronize()
    out = buf.cpu().numpy().view(np.uint32)
    total = int(np.bitwise_xor.reduce(out[:grid])) if grid > 1 else int(out[0])
    assert total == oracle.stream_xor(src), f"xor {cfg} {n_bytes}"
    assert np.all(out[grid:] == SENTINEL)


def chain(n_words, nodes, seed, stride=64):
    """A cycle through `nodes` random, stride-aligned word positions of an n_words table."""
    rng = np.random.default_rng(seed)
    pos = rng.choice(n_words // stride, size=nodes, replace=False).astype(np.int64) * stride
    table = np.zeros(n_words, np.uint32)
    table[pos] = np.roll(pos, -1)
    return table, pos


@pytest.mark.parametrize("n_words,nodes,hops", [(1 << 16, 256, 1), (1 << 16, 256, 1000),
                                                 (1 << 22, 4096, 5000), (1 << 20, 1, 3)])
def test_chase_matches_oracle(n_words, nodes, hops):
    import torch
    table, pos = chain(n_words, nodes, n_words + nodes)
    d = dev(table)
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    start = int(pos[0])
    st = gb.gemm355_chase(d.data_ptr(), n_words, start, hops, out.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK
    torch.cuda.synchronize()
    final, cycles = (int(v) for v in out.cpu().numpy())
    assert final == oracle.chase(table, start, hops)
    assert final == int(pos[hops % nodes])
    assert cycles > 0


def test_chase_clamps_out_of_range_entries():
    import torch
    # a table of 32 words of which the walk may use 8: entry 0 holds 20 and must become 7
    table = np.zeros(32, np.uint32)
    table[0], table[7], table[20] = 20, 3, 5
    d = dev(table)
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    for hops in (1, 2, 3):
        st = gb.gemm355_chase(d.data_ptr(), 8, 0, hops, out.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        assert st == gb.OK
        torch.cuda.synchronize()
        assert int(out.cpu()[0]) == oracle.chase(table, 0, hops, n=8)
