"""Pins of the gfx950 lane layouts the kernels rely on, measured on the device.

Layouts asserted (A is M x k, B is k x N, D = A.B, W = 32 or 16 rows per block):
  * A operand: lane l supplies row l mod W of A;
  * B operand: lane l supplies column l mod W of B;
  * the k slots of A-lane l and B-lane l' coincide element by element whenever
    l div W == l' div W (the kernels only rely on this consistency);
  * accumulator: 32 x 32 blocks: register r of lane l is D[8(r/4) + 4(l/32) + r%4][l%32];
    16 x 16 blocks: register r of lane l is D[4(l/16) + r][l%16];
  * ds_read_b64_tr_b16: within each 16-lane group, output lane j receives as element e
    halfword j%4 of the 8 bytes addressed by source lane 4e + (j%16)/4.
"""

from __future__ import annotations

import os

import numpy as np
import pytest

from roofline_optimisation_amd import binding as gb

pytestmark = pytest.mark.gpu

KINDS = {0: "32x32x2_f32", 1: "16x16x4_f32", 2: "32x32x16_f16", 3: "16x16x32_f16",
         4: "32x32x16_bf16", 5: "16x16x32_bf16"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_probe(kind, a, b):
    """a, b: (nruns, 64, E) float32 arrays -> (nruns, 64, R) accumulators."""
    import torch
    E, R = gb.gemm355_probe_mfma_shape(kind)
    nruns = a.shape[0]
    da = torch.from_numpy(np.ascontiguousarray(a, np.float32).reshape(-1)).cuda()
    db = torch.from_numpy(np.ascontiguousarray(b, np.float32).reshape(-1)).cuda()
    dd = torch.zeros(nruns * 64 * R, dtype=torch.float32, device="cuda")
    st = gb.gemm355_probe_mfma(kind, nruns, da.data_ptr(), db.data_ptr(), dd.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK
    torch.cuda.synchronize()
    return dd.cpu().numpy().reshape(nruns, 64, R)


def out_coords(kind):
    """(row, col) of accumulator register r of lane l, as two (64, R) arrays."""
    _, R = gb.gemm355_probe_mfma_shape(kind)
    l = np.arange(64)[:, None]
    r = np.arange(R)[None, :]
    if R == 16:
        return 8 * (r // 4) + 4 * (l // 32) + r % 4 + 0 * l, (l % 32) + 0 * r
    return 4 * (l // 16) + r + 0 * l, (l % 16) + 0 * r


@pytest.mark.parametrize("kind", sorted(KINDS), ids=lambda k: KINDS[k])
def test_rows_and_output_layout(kind):
    E, R = gb.gemm355_probe_mfma_shape(kind)
    W = 32 if R == 16 else 16
    a = np.zeros((64 * E, 64, E), np.float32)
    for p in range(64):
        for e in range(E):
            a[p * E + e, p, e] = 1.0
    b = np.ones_like(a)
    d = run_probe(kind, a, b)
    rows, _ = out_coords(kind)
    for p in range(64):
        for e in range(E):
            lit = d[p * E + e] != 0
            assert np.all(d[p * E + e][lit] == 1.0)
            assert np.array_equal(lit, rows == p % W), (KINDS[kind], p, e)


@pytest.mark.parametrize("kind", sorted(KINDS), ids=lambda k: KINDS[k])
def test_columns(kind):
    E, R = gb.gemm355_probe_mfma_shape(kind)
    W = 32 if R == 16 else 16
    b = np.zeros((64 * E, 64, E), np.float32)
    for q in range(64):
        for e in range(E):
            b[q * E + e, q, e] = 1.0
    d = run_probe(kind, np.ones_like(b), b)
    _, cols = out_coords(kind)
    for q in range(64):
        for e in range(E):
            assert np.array_equal(d[q * E + e] != 0, cols == q % W), (KINDS[kind], q, e)


@pytest.mark.parametrize("kind", sorted(KINDS), ids=lambda k: KINDS[k])
def test_k_slots_consistent(kind):
    E, R = gb.gemm355_probe_mfma_shape(kind)
    W = 32 if R == 16 else 16
    rows, cols = out_coords(kind)
    cases = []
    rng = np.random.default_rng(kind)
    for _ in range(48):
        p, q = rng.integers(0, 64, size=2)
        e, e2 = rng.integers(0, E, size=2)
        cases.append((p, e, q, e2))
    a = np.zeros((len(cases), 64, E), np.float32)
    b = np.zeros_like(a)
    for i, (p, e, q, e2) in enumerate(cases):
        a[i, p, e] = 1.0
        b[i, q, e2] = 1.0
    d = run_probe(kind, a, b)
    for i, (p, e, q, e2) in enumerate(cases):
        at = (rows == p % W) & (cols == q % W)
        same = (p // W == q // W) and (e == e2)
        assert np.all(d[i][~at] == 0)
        assert np.all(d[i][at] == (1.0 if same else 0.0)), (KINDS[kind], p, e, q, e2)


@pytest.mark.parametrize("kind", sorted(KINDS), ids=lambda k: KINDS[k])
def test_random_block_product(kind):
    """Load a random integer block product in the pinned layout and compare."""
    E, R = gb.gemm355_probe_mfma_shape(kind)
    W = 32 if R == 16 else 16
    G = 64 // W                    # lane groups
    Kb = G * E                     # k extent of one instruction
    rng = np.random.default_rng(100 + kind)
    Am = rng.integers(-3, 4, size=(W, Kb)).astype(np.float32)
    Bm = rng.integers(-3, 4, size=(Kb, W)).astype(np.float32)
    a = np.zeros((1, 64, E), np.float32)
    b = np.zeros_like(a)
    for l in range(64):
        for e in range(E):
            k = (l // W) * E + e
            a[0, l, e] = Am[l % W, k]
            b[0, l, e] = Bm[k, l % W]
    d = run_probe(kind, a, b)[0]
    rows, cols = out_coords(kind)
    ref = Am @ Bm
    assert np.array_equal(d, ref[rows, cols])


def tr16_expected(addrs):
    """The mapping the 16-bit kernel relies on: within each 16-lane group, output lane j
    receives as element e the halfword j % 4 of the 8 bytes read by source lane
    4 e + (j % 16) / 4 of the same group."""
    out = np.zeros((64, 4), np.int64)
    for j in range(64):
        g = j // 16
        for e in range(4):
            src = 16 * g + 4 * e + (j % 16) // 4
            out[j, e] = addrs[src] // 2 + j % 4
    return out


@pytest.mark.parametrize("pattern", ["linear", "rows576", "reversed", "gemm_b_fragment"])
def test_ds_read_tr16_mapping(pattern):
    import torch
    if pattern == "linear":
        addrs = [8 * l for l in range(64)]
    elif pattern == "rows576":
        addrs = [576 * (l % 16 // 4) + 8 * (l % 4) + 32 * (l // 16) for l in range(64)]
    elif pattern == "reversed":
        addrs = [8 * (63 - l) for l in range(64)]
    else:
        # the kernel's B-fragment address structure (group g reads rows 8 (g/2) + e,
        # columns 16 (g%2) + 4 q), with a 320-byte row stride so it fits the probe's 4 KiB
        addrs = []
        for l in range(64):
            g, s = l // 16, l % 16
            addrs.append((8 * (g // 2) + s // 4) * 320 + 2 * (16 * (g % 2) + 4 * (s % 4)))
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    st = gb.gemm355_probe_ds_read_tr16(addrs, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64).reshape(64, 4)
    assert np.array_equal(got, tr16_expected(addrs)), pattern


def test_ds_read_tr16_mapping_recorded():
    """Records where each output halfword of ds_read_b64_tr_b16 comes from, for linear
    lane addresses (lane l at byte 8l) and for a row-strided pattern; asserts only that
    the results are halfwords of the addressed region."""
    import torch
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    lines = []
    patterns = {
        "linear": [8 * l for l in range(64)],
        "rows256": [256 * (l % 16) + 8 * (l // 16) for l in range(64)],
    }
    for name, addrs in patterns.items():
        st = gb.gemm355_probe_ds_read_tr16(addrs, out.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
        assert st == gb.OK
        torch.cuda.synchronize()
        v = out.cpu().numpy().astype(np.int64).reshape(64, 4)
        allowed = set()
        for a in addrs:
            allowed |= {a // 2 + i for i in range(4)}
        assert set(v.reshape(-1).tolist()) <= allowed, name
        lines.append(f"pattern {name}: lane: (src_lane, src_elem) x4")
        src_of = {}
        for l, a in enumerate(addrs):
            for i in range(4):
                src_of[a // 2 + i] = (l, i)
        for l in range(64):
            lines.append(f"  {l:2d}: " + " ".join(f"({src_of[int(x)][0]:2d},{src_of[int(x)][1]})"
                                                 for x in v[l]))
    text = "\n".join(lines)
    print(text)
    out_dir = os.environ.get("GEMM355_PROBE_OUT")
    if out_dir:
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, "ds_read_tr16_mapping.txt"), "w") as f:
            f.write(text + "\n")


def gll_expected(chunks, base):
    """The placement the direct-to-LDS tile loads rely on: lane l's 16 bytes, read from
    16-byte chunk chunks[l] of the source, land at LDS bytes base + 16 l .. base + 16 l + 15
    (the LDS address is the wave-uniform base plus 16 times the lane index)."""
    out = np.zeros(512, np.int64)
    for l, c in enumerate(chunks):
        for i in range(4):
            out[base // 4 + 4 * l + i] = 4 * c + i + 1
    return out


@pytest.mark.parametrize("pattern,base", [("linear", 0), ("reversed", 0), ("strided", 512),
                                          ("linear", 1024), ("scattered", 256)])
def test_global_load_lds_placement(pattern, base):
    import torch
    if pattern == "linear":
        chunks = list(range(64))
    elif pattern == "reversed":
        chunks = [63 - l for l in range(64)]
    elif pattern == "strided":
        chunks = [37 * l for l in range(64)]
    else:
        chunks = np.random.default_rng(7).permutation(4096)[:64].tolist()
    # source word w holds w + 1, so a zero in the output means "not written"
    src = torch.arange(1, 4 * 4096 + 1, dtype=torch.int32, device="cuda")
    out = torch.full((512,), -1, dtype=torch.int32, device="cuda")
    st = gb.gemm355_probe_global_load_lds(src.data_ptr(), chunks, base, out.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64)
    exp = gll_expected(chunks, base)
    if not np.array_equal(got, exp):
        where = {int(v): i for i, v in enumerate(got) if v > 0}
        landed = [where.get(4 * c + 1, -1) for c in chunks]
        pytest.fail(f"{pattern}/{base}: lane -> LDS word of its first element: {landed}")
