"""The C ABI from plain C: a C11 client (tests/c_abi_client.c) that includes every public
header beside HIP's own runtime header compiles with gcc -Wall -Wextra -Werror, links
libgemm355.so, and gets the documented results from the calls that need no GPU."""

import os
import shutil
import subprocess

import pytest

from roofline_optimisation_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def client_output(tmp_path_factory):
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("gcc or the HIP headers are not available")
    if not os.path.exists(gb.LIB_PATH):
        pytest.fail("libgemm355.so is not built (run __graft_entry__.build())")
    libdir = os.path.dirname(gb.LIB_PATH)
    exe = str(tmp_path_factory.mktemp("c_client") / "c_abi_client")
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c_abi_client.c"), "-L", libdir, "-lgemm355",
                        f"-Wl,-rpath,{libdir}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    return dict(ln.split(" ", 1) for ln in r.stdout.splitlines())


def test_host_queries(client_output):
    out = client_output
    assert out["version"] == str(gb.gemm355_version())
    assert out["status_invalid"] == "invalid argument"
    assert out["variant_mfma"] == "mfma"
    assert out["select_f32_3072"] == str(gb.VARIANT_MFMA)
    assert out["desc_f32_3072"] == "mfma_f32 192x192x32 w2x6 dwordx4"
    assert out["desc_f16_4096"] == "mfma_f16 256x256x32 w2x2 lds-dma"
    assert out["desc_ex_f16_ta"] == "mfma_f16 256x256x32 w2x2 lds-dma"
    assert out["probe_shape_rc"] == "-1"


def test_argument_errors_before_any_hip_call(client_output):
    out = client_output
    invalid, unsupported = str(gb.ERR_INVALID_ARG), str(gb.ERR_UNSUPPORTED)
    for key in ("f32_negative_m", "f32_short_lda", "f16_null_a", "bf16_m0_null_b", "variant_bad",
                "ex_bad_flags", "softmax_short_ld", "row_sum_null", "stream_bad_mode"):
        assert out[key] == invalid, (key, out[key])
    assert out["lds_tiled_f16"] == unsupported
    assert out["bf16_m0"] == str(gb.OK)
