"""The bench's roofline accounting reproduces the numbers printed on the pages."""

import os

import pytest

from roofline_optimisation_amd import roofline as rl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_kv(name):
    out = {}
    for ln in open(os.path.join(GOLDEN, name)):
        ln = ln.split("#", 1)[0].split()
        if ln:
            out[ln[0]] = (float(ln[1]), int(ln[2]) if len(ln) > 2 else None)
    return out


G = load_kv("ada_roofline_n3072.txt")


def printed(key, value):
    ref, dec = G[key]
    assert round(value, dec) == pytest.approx(ref), (key, value, ref)


def test_ridge_and_crossover():
    peak, bw = G["peak_flops"][0], G["dram_Bps"][0]
    printed("ridge_flop_per_B", rl.ridge(peak, bw))
    assert rl.crossover_n(peak, bw) == G["crossover_n"][0]
    n = int(G["crossover_n"][0])
    assert n / 6 >= rl.ridge(peak, bw) > (n - 1) / 6


def test_n3072_limits():
    n = int(G["n"][0])
    peak, bw, l2 = G["peak_flops"][0], G["dram_Bps"][0], G["l2_Bps"][0]
    assert rl.flops(n, n, n) == 2 * n ** 3
    assert f"{rl.flops(n, n, n):.3e}" == "5.798e+10"
    printed("compute_ms", rl.compute_time(n, n, n, peak) * 1e3)
    printed("ideal_MB", rl.ideal_bytes(n, n, n) / 1e6)
    printed("ideal_dram_ms", rl.memory_time(rl.ideal_bytes(n, n, n), bw) * 1e3)
    # the page's 231.87 GB is a slip; the closed form gives 231.93e9 B exactly
    assert rl.noreuse_bytes(n, n, n) == 8 * n ** 3 == 231_928_233_984
    gb = G["noreuse_GB_printed"][0] * 1e9
    printed("noreuse_dram_ms", rl.memory_time(gb, bw) * 1e3)
    printed("noreuse_l2_ms", rl.memory_time(gb, l2) * 1e3)
    # the summary table's "~296x" and "~42x" are the ratios cut to whole numbers
    comp = rl.compute_time(n, n, n, peak)
    assert int(rl.memory_time(gb, bw) / comp) == G["ratio_dram"][0]
    assert int(rl.memory_time(gb, l2) / comp) == G["ratio_l2"][0]


def test_intensities():
    printed("oi_naive", rl.flops(7, 7, 7) / rl.noreuse_bytes(7, 7, 7))
    for n in (6, 445, 3072):
        assert rl.intensity(n, n, n) == pytest.approx(n / 6)


def test_littles_law():
    lat, clk, bw = G["latency_cycles"][0], G["clock_hz"][0], G["dram_Bps"][0]
    printed("bytes_per_cycle", bw / clk)
    printed("inflight_bytes", rl.littles_law_bytes(lat, bw, clk))


def test_occupancy_table():
    for ln in open(os.path.join(GOLDEN, "occupancy_table.txt")):
        ln = ln.split("#", 1)[0].split()
        if not ln:
            continue
        smem, blocks, warps, pct = int(ln[0]), int(ln[1]), int(ln[2]), float(ln[3])
        occ = rl.occupancy_from_smem(smem, 102400, 48, 2, max_blocks=24)
        assert (occ.blocks, occ.warps) == (blocks, warps)
        assert round(occ.fraction * 100, 1) == pytest.approx(round(pct, 1), abs=0.05)


def test_mi355x_ridges():
    # FP32: 157.3 TF / 8 TB/s = 19.66 FLOP/B -> ideal-reuse crossover n = 118
    p = rl.MI355X["peak_flops"]
    assert rl.ridge(p["f32_vector"], rl.MI355X["hbm_Bps"]) == pytest.approx(19.6625)
    assert rl.crossover_n(p["f32_vector"], rl.MI355X["hbm_Bps"]) == 118
    # the published peaks follow from unit counts and clock
    cus, clk = rl.MI355X["cus"], rl.MI355X["clock_hz"]
    assert cus * clk * 256 == pytest.approx(p["f32_mfma"], rel=1e-3)
    assert cus * clk * 4096 == pytest.approx(p["f16_mfma"], rel=1e-3)


def test_roofline_entry():
    e = rl.roofline_entry(3072, 3072, 3072, 0.5e-3, "f32")
    assert e["tflops"] == pytest.approx(2 * 3072 ** 3 / 0.5e-3 / 1e12)
    assert e["oi"] == pytest.approx(512)
    e = rl.roofline_entry(4096, 4096, 4096, 100e-6, "f16")
    assert e["ideal_bytes"] == 2 * 2 * 4096 ** 2 + 4 * 4096 ** 2


def test_text_chart_places_points_and_roofs():
    lines = rl.text_chart([(1024.0, 1000.0, "b"), (8.0, 0.25, "f")], [(2516.6, "="), (157.3, "-")],
                          8e12, width=40, height=12)
    assert len(lines) == 14 and all(len(l) >= 9 for l in lines[:12])
    body = [l[9:] for l in lines[:12]]
    # the lowest-intensity, lowest-rate point sits in the bottom-left corner
    assert body[11][0] == "f"
    # the FP32 roof is flat at 157.3 to the right of its ridge (19.7 FLOP/B)
    r157 = [i for i, l in enumerate(body) if l.rstrip().endswith("-")]
    assert r157 and all(body[r157[0]][c] in "-b" for c in range(20, 40))
    assert any("b" in l for l in body)


def test_kernel_hash_ignores_comments_only():
    """The counter summaries are matched to the kernel code by a hash of the sources with
    comments stripped: comment edits keep it, any code edit (strings included) moves it."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "bench_host", os.path.join(os.path.dirname(os.path.dirname(__file__)), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    src = 'int f(int x) {  // add one\n  /* block\n comment */ return x + 1;\n}\nconst char* s = "a//b";\n'
    same = '// header\nint f(int x) {\n\n  return x + 1; /* c */\n}\nconst char* s = "a//b";  // tail\n'
    assert bench.strip_comments(src) == bench.strip_comments(same)
    assert "a//b" in bench.strip_comments(src)
    for edit in (src.replace("x + 1", "x + 2"), src.replace("a//b", "a/b"),
                 src.replace("x) {", "x) {\n  x++;")):
        assert bench.strip_comments(edit) != bench.strip_comments(src)
    for kind in bench.KERNEL_SOURCES:
        assert len(bench.kernel_hash(kind)) == 16
