"""Every kernel instance compiles for gfx950 without register spills or scratch memory
and without packed FP32 instructions, m0 is written only by the direct-to-LDS load
sequences, and the accumulators of the inline-assembly MFMAs are touched by nothing but
those MFMAs between the wait states that fence them (checked on the CPU with hipcc)."""

import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from roofline_optimisation_amd import build as gbuild

HIPCC = gbuild.HIPCC


@pytest.fixture(scope="module")
def compiled():
    """{source: (gfx950 assembly, resource-usage remarks)}: every HIP source compiled once,
    device code only."""
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    def one(src):
        r = subprocess.run([HIPCC, *gbuild.HIPFLAGS, "--cuda-device-only", "-S", src, "-o", "-",
                            "-Rpass-analysis=kernel-resource-usage"],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, (r.stdout, r.stderr)
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        return dict(ex.map(one, gbuild.sources()))


@pytest.fixture(scope="module")
def remarks(compiled):
    return {os.path.basename(src): rem for src, (_, rem) in compiled.items()}


def parse(text):
    """(function, {field: value}) for every kernel the remarks describe."""
    kernels, cur = [], None
    for ln in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", ln)
        if m:
            cur = (m.group(1), {})
            kernels.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?):\s+(\d+)", ln)
        if m and cur:
            cur[1][m.group(1).strip()] = int(m.group(2))
    return kernels


def test_no_spills_or_scratch(remarks):
    n = 0
    for fname, text in remarks.items():
        for name, f in parse(text):
            n += 1
            assert f.get("VGPRs Spill", 0) == 0, (fname, name, f)
            assert f.get("SGPRs Spill", 0) == 0, (fname, name, f)
            assert f.get("ScratchSize [bytes/lane]", 0) == 0, (fname, name, f)
    assert n >= 40


def test_lds_within_160k(remarks):
    for fname, text in remarks.items():
        for name, f in parse(text):
            assert f.get("LDS Size [bytes/block]", 0) <= 160 * 1024, (fname, name, f)


@pytest.fixture(scope="module")
def assembly(compiled):
    """{source: gfx950 assembly} for every HIP source."""
    return {src: asm for src, (asm, _) in compiled.items()}


def test_no_packed_fp32_instructions(assembly):
    for src, asm in assembly.items():
        bad = re.findall(r"\bv_pk_(?:fma|mul|add)_f32\b", asm)
        assert not bad, (src, bad[:3])


def test_inline_mfma_accumulators_fenced(assembly):
    """The direct-to-LDS kernels issue their MFMAs as inline assembly, so the compiler
    inserts no wait states for them.  In every kernel whose MFMAs are inline assembly,
    every compiler-generated instruction that names an accumulator register (a copy, a
    zeroing write, a store) lies either before the two-`s_nop 7` block that precedes the
    first MFMA or after the four-`s_nop 7` block that follows the last one, and no branch
    between them leaves that region except to the start of the closing block (so the
    skipped k-steps of a ragged-K tail still pass it)."""
    kernels = 0
    for src, asm in assembly.items():
        for body in re.split(r"\n(?=_Z\S+:)", asm):
            lines = [ln.strip() for ln in body.splitlines() if ln.strip()]
            in_asm, items = False, []  # (instruction, from inline assembly)
            labels = {}  # block label -> index of the instruction that follows it
            for ln in lines:
                if ln.startswith(";;#ASMSTART"):
                    in_asm = True
                elif ln.startswith(";;#ASMEND"):
                    in_asm = False
                elif re.match(r"\.LBB\w+:", ln):
                    labels[ln.split(":")[0]] = len(items)
                elif not ln.startswith((";", ".")) and not ln.endswith(":"):
                    items.append((ln, in_asm))
            mfma = [i for i, (ln, a) in enumerate(items) if a and ln.startswith("v_mfma")]
            if not mfma:
                continue
            kernels += 1
            first, last = mfma[0], mfma[-1]
            nops = [i for i, (ln, a) in enumerate(items) if a and ln.startswith("s_nop 7")]
            pre = [i for i in nops if i < first]
            post = [i for i in nops if i > last]
            assert len(pre) >= 2 and len(post) >= 4, (src, body[:80])
            lo, hi = pre[-2], post[3]
            for i in range(lo, hi):
                ln, a = items[i]
                if a:
                    continue
                assert not re.search(r"\ba(?:\d+|\[\d+:\d+\])", ln), (src, body[:60], ln)
                # every path out of the fenced region passes the closing wait-state block:
                # a branch inside it lands inside it or at the block's start at the latest
                m = re.match(r"s_(?:c?branch\w*)\s+(\.LBB\w+)$", ln)
                if m:
                    assert lo <= labels[m.group(1)] <= post[0], (src, body[:60], ln)
    assert kernels >= 40


def test_m0_only_in_lds_load_sequences(assembly):
    """The direct-to-LDS loads set m0 from inline assembly without declaring it: in every
    kernel that contains such a sequence no other instruction may read or write m0, and
    every m0 write is followed by one wait state and a buffer load with the lds flag."""
    kernels = 0
    for src, asm in assembly.items():
        for body in re.split(r"\n(?=_Z\S+:)", asm):
            if "offen lds" not in body:
                continue
            kernels += 1
            lines = [ln.strip() for ln in body.splitlines()
                     if ln.strip() and not ln.strip().startswith((";", ".", "//"))]
            seqs = 0
            for i, ln in enumerate(lines):
                if re.search(r"\bm0\b", ln):
                    assert re.match(r"s_mov_b32 m0, s\d+$", ln), (src, ln)
                    assert lines[i + 1] == "s_nop 0", (src, lines[i + 1])
                    assert re.match(r"buffer_load_dwordx4 v\d+, s\[\d+:\d+\], s\d+ offen lds$",
                                    lines[i + 2]), (src, lines[i + 2])
                    seqs += 1
                elif ln.endswith(" lds"):
                    assert lines[i - 1] == "s_nop 0", (src, ln)
            assert seqs > 0
    assert kernels >= 2
