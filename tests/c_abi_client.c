/* A plain C (C11) client of libgemm355: includes every public header next to HIP's own
 * runtime header, links the library, and exercises the calls that need no GPU (the host
 * queries and the argument checks made before any HIP call).  Each line it prints is
 * "name value"; tests/test_c_client.py compiles it, runs it and checks the lines. */
#include <stdint.h>
#include <stdio.h>

#include <hip/hip_runtime_api.h>

#include "gemm355.h"
#include "gemm355_probe.h"
#include "gemm355_softmax.h"
#include "gemm355_stream.h"

int main(void) {
    /* a 16-byte-aligned address that is never dereferenced: every call below returns
     * before touching memory */
    float *p = (float *)(uintptr_t)(1u << 20);
    const uint16_t *h = (const uint16_t *)(uintptr_t)(1u << 20);
    hipStream_t s = NULL;
    int ept = 0, rpl = 0;

    printf("version %d\n", gemm355_version());
    printf("status_invalid %s\n", gemm355_status_string(GEMM355_ERR_INVALID_ARG));
    printf("variant_mfma %s\n", gemm355_variant_name(GEMM355_VARIANT_MFMA));
    printf("f32_negative_m %d\n", (int)gemm_f32(-1, 4, 4, p, 4, p, 4, p, 4, s));
    printf("f32_short_lda %d\n", (int)gemm_f32(4, 4, 8, p, 7, p, 4, p, 4, s));
    printf("f16_null_a %d\n", (int)gemm_f16f32acc(4, 4, 4, NULL, 4, h, 4, p, 4, s));
    /* M = 0: nothing to do; A and C have no elements and may be NULL, B may not */
    printf("bf16_m0 %d\n", (int)gemm_bf16f32acc(0, 4, 4, NULL, 4, h, 4, NULL, 4, s));
    printf("bf16_m0_null_b %d\n", (int)gemm_bf16f32acc(0, 4, 4, NULL, 4, NULL, 4, NULL, 4, s));
    printf("variant_bad %d\n",
           (int)gemm355_run_variant(42, GEMM355_F32, 4, 4, 4, p, 4, p, 4, p, 4, s));
    printf("lds_tiled_f16 %d\n",
           (int)gemm355_run_variant(GEMM355_VARIANT_LDS_TILED, GEMM355_F16, 4, 4, 4, h, 4, h, 4, p, 4, s));
    printf("ex_bad_flags %d\n",
           (int)gemm355_gemm_ex(GEMM355_VARIANT_AUTO, GEMM355_F16, 1u << 10, 4, 4, 4, h, 4, h, 4, p, 4, s));
    printf("select_f32_3072 %d\n",
           gemm355_select_variant(GEMM355_F32, 3072, 3072, 3072, p, 3072, p, 3072, p, 3072));
    printf("desc_f32_3072 %s\n",
           gemm355_kernel_desc(GEMM355_VARIANT_AUTO, GEMM355_F32, 3072, 3072, 3072, p, 3072, p, 3072, p, 3072));
    printf("desc_f16_4096 %s\n",
           gemm355_kernel_desc(GEMM355_VARIANT_AUTO, GEMM355_F16, 4096, 4096, 4096, h, 4096, h, 4096, p, 4096));
    printf("desc_ex_f16_ta %s\n",
           gemm355_kernel_desc_ex(GEMM355_VARIANT_AUTO, GEMM355_F16, GEMM355_TRANS_A, 4096, 4096, 4096,
                                  h, 4096, h, 4096, p, 4096));
    printf("softmax_short_ld %d\n", (int)gemm355_softmax_f32(4, 8, p, 7, p, 8, s));
    printf("row_sum_null %d\n", (int)gemm355_row_sum_f32(4, 8, NULL, 8, p, s));
    printf("stream_bad_mode %d\n", (int)gemm355_stream(99, p, p, 1024, 16, 1, 256, 0, 0, s));
    printf("probe_shape_rc %d\n", gemm355_probe_mfma_shape(-7, &ept, &rpl));
    return 0;
}
