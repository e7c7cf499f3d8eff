"""libgemm355: dense GEMM C = A.B for AMD Instinct MI355X (gfx950).

The product runs in hand-written HIP kernels behind the C ABI declared in
``include/gemm355.h`` (``libgemm355.so``, built by ``build.py``).  ``binding`` is the
thin ctypes layer over it; ``inputs`` draws the seeded synthetic operands;
``roofline`` holds the FLOP and byte accounting used to report results against the
MI355X roofline.
"""

from .binding import (  # noqa: F401
    BF16, F16, F32, OK, VARIANTS, Gemm355Error, gemm355_kernel_desc, gemm355_run_variant,
    gemm355_select_variant, gemm355_status_string, gemm355_variant_name, gemm355_version,
    gemm_bf16f32acc, gemm_f16f32acc, gemm_f32, lib, matmul,
)
