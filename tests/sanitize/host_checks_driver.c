/*
 * Sanitizer driver for the host side of libkq.so (test infrastructure): built
 * against a copy of the library whose host code carries
 * -fsanitize=address,undefined (device code unchanged) by
 * tests/test_sanitizers.py, and run on the CPU with no GPU. Every call below
 * fails its argument checks before any HIP call, or is host-only
 * (kq_factors_from_lu, kq_calib_workspace_bytes, kq_status_string), so the
 * checks' own arithmetic (size products, alignment, limits) runs under the
 * sanitizers, including at the extremes of int64 sizes.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kq.h"

#define P(x) ((void *)(uintptr_t)(x))
static const void *GOOD = P(0x10000);  /* never dereferenced */
static int failures = 0;

static void expect(const char *what, kq_status got, kq_status want) {
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, (int)got, (int)want);
        ++failures;
    }
}

int main(void) {
    const int64_t BIG = INT64_MAX / 2;
    expect("quantize d%32", kq_quantize_mxfp4(GOOD, 4, 33, 33, P(0x10000), P(0x10000), NULL), KQ_ERR_SHAPE);
    expect("quantize huge", kq_quantize_mxfp4(GOOD, BIG, 64, 64, P(0x10000), P(0x10000), NULL), KQ_ERR_SHAPE);
    expect("quantize huge lda", kq_quantize_mxfp4(GOOD, 4, 64, BIG, P(0x10000), P(0x10000), NULL), KQ_ERR_SHAPE);
    expect("quantize null", kq_quantize_mxfp4(NULL, 4, 64, 64, P(0x10000), P(0x10000), NULL), KQ_ERR_NULL);
    expect("quantize align", kq_quantize_mxfp4(P(0x10002), 4, 64, 64, P(0x10000), P(0x10000), NULL), KQ_ERR_ALIGN);
    expect("quantize m=0", kq_quantize_mxfp4(NULL, 0, 64, 64, NULL, NULL, NULL), KQ_OK);
    expect("fused null factors", kq_transform_quantize_mxfp4(GOOD, 4, 64, 64, NULL, P(0x10000), P(0x10000), NULL, NULL),
           KQ_ERR_NULL);
    expect("fused bad form", kq_transform_quantize_mxfp4_form(GOOD, 4, 64, 64, GOOD, P(0x10000), P(0x10000), NULL, 7,
                                                             NULL), KQ_ERR_UNSUPPORTED);
    expect("fused huge", kq_transform_quantize_mxfp4(GOOD, BIG, 64, 64, GOOD, P(0x10000), P(0x10000), NULL, NULL),
           KQ_ERR_SHAPE);
    expect("y16 null", kq_transform_quantize_mxfp4_y16(GOOD, 4, 64, 64, GOOD, P(0x10000), P(0x10000), NULL, NULL),
           KQ_ERR_NULL);
    expect("smooth align", kq_smoothquant_quantize_mxfp4(GOOD, 4, 64, 64, P(0x10004), P(0x10000), P(0x10000), NULL),
           KQ_ERR_ALIGN);
    expect("f32 ldx", kq_quantize_mxfp4_f32(GOOD, 4, 64, 66, P(0x10000), P(0x10000), NULL), KQ_ERR_ALIGN);
    expect("fold shape", kq_inverse_fold_weights(GOOD, 4, 40, GOOD, P(0x10000), NULL), KQ_ERR_SHAPE);
    expect("hadamard n", kq_hadamard_quantize_mxfp4(GOOD, 4, 96, 96, 48, P(0x10000), P(0x10000), NULL, NULL),
           KQ_ERR_SHAPE);
    expect("hadamard n big", kq_hadamard_quantize_mxfp4(GOOD, 4, 32768, 32768, 32768, P(0x10000), P(0x10000), NULL,
                                                        NULL), KQ_ERR_UNSUPPORTED);
    expect("gemm k", kq_mxfp4_gemm(GOOD, GOOD, GOOD, GOOD, 4, 4, 48, P(0x10000), 4, NULL), KQ_ERR_SHAPE);
    expect("gemm huge", kq_mxfp4_gemm_packed(GOOD, GOOD, GOOD, GOOD, BIG, BIG, 256, P(0x10000), BIG, NULL),
           KQ_ERR_UNSUPPORTED);
    expect("pack k", kq_pack_mxfp4_scales(GOOD, 4, 100, P(0x10000), NULL), KQ_ERR_SHAPE);
    expect("lowrank r", kq_mxfp4_gemm_packed_lowrank(GOOD, GOOD, GOOD, GOOD, 4, 4, 256, GOOD, GOOD, GOOD, 48,
                                                     P(0x10000), 4, NULL), KQ_ERR_SHAPE);
    expect("project null", kq_lowrank_project_bf16(NULL, 4, 64, 64, GOOD, 32, P(0x10000), NULL), KQ_ERR_NULL);
    expect("dequant k", kq_dequantize_mxfp4_bf16(GOOD, GOOD, 4, 48, P(0x10000), NULL), KQ_ERR_SHAPE);
    expect("gemm_f32 C", kq_gemm_f32(0, 0, 4, 4, 4, 1.0f, GOOD, 4, GOOD, 4, 1.0f, NULL, 4, P(0x10000), 4, NULL),
           KQ_ERR_NULL);
    expect("w4a4 fused k", kq_transform_quantize_mxfp4_gemm(GOOD, 4, 48, 48, GOOD, GOOD, GOOD, 4, P(0x10000), 4,
                                                           NULL), KQ_ERR_SHAPE);
    /* every GEMM-family entry point at sizes whose products overflow int64 */
    expect("gemm huge m", kq_mxfp4_gemm(GOOD, GOOD, GOOD, GOOD, BIG, 4, 64, P(0x10000), 4, NULL), KQ_ERR_UNSUPPORTED);
    expect("gemm huge ldo", kq_mxfp4_gemm(GOOD, GOOD, GOOD, GOOD, 4, 4, 64, P(0x10000), BIG, NULL),
           KQ_ERR_UNSUPPORTED);
    expect("gemm wide huge", kq_mxfp4_gemm_wide(GOOD, GOOD, GOOD, GOOD, 4, BIG, 64, P(0x10000), BIG, NULL),
           KQ_ERR_UNSUPPORTED);
    expect("gemm packed huge k", kq_mxfp4_gemm_packed(GOOD, GOOD, GOOD, GOOD, 4, 4, (int64_t)1 << 40, P(0x10000), 4,
                                                      NULL), KQ_ERR_UNSUPPORTED);
    expect("gemm packed bf16 huge", kq_mxfp4_gemm_packed_bf16(GOOD, GOOD, GOOD, GOOD, BIG, BIG, 256, P(0x10000), BIG,
                                                              NULL), KQ_ERR_UNSUPPORTED);
    expect("gemm packed lowrank huge", kq_mxfp4_gemm_packed_lowrank(GOOD, GOOD, GOOD, GOOD, BIG, 4, 256, GOOD, GOOD,
                                                                    GOOD, 32, P(0x10000), 4, NULL),
           KQ_ERR_UNSUPPORTED);
    expect("gemm lowrank huge r", kq_mxfp4_gemm_lowrank(GOOD, GOOD, GOOD, GOOD, 4, 4, 64, GOOD, GOOD, GOOD,
                                                        (int64_t)1 << 40, P(0x10000), 4, NULL), KQ_ERR_UNSUPPORTED);
    expect("project huge", kq_lowrank_project(GOOD, BIG, 64, 64, GOOD, GOOD, 32, P(0x10000), NULL),
           KQ_ERR_UNSUPPORTED);
    expect("project bf16 huge ldx", kq_lowrank_project_bf16(GOOD, 4, 64, BIG, GOOD, 32, P(0x10000), NULL),
           KQ_ERR_UNSUPPORTED);
    expect("dequant huge", kq_dequantize_mxfp4_bf16(GOOD, GOOD, BIG, 64, P(0x10000), NULL), KQ_ERR_UNSUPPORTED);
    expect("pack huge", kq_pack_mxfp4_scales(GOOD, BIG, 256, P(0x10000), NULL), KQ_ERR_UNSUPPORTED);
    expect("gemm_f32 huge", kq_gemm_f32(0, 0, BIG, BIG, 4, 1.0f, GOOD, 4, GOOD, BIG, 0.0f, NULL, BIG, P(0x10000), BIG,
                                        NULL), KQ_ERR_UNSUPPORTED);
    expect("w4a4 fused huge lda", kq_transform_quantize_mxfp4_gemm(GOOD, 4, 64, BIG, GOOD, GOOD, GOOD, 4, P(0x10000), 4,
                                                                  NULL), KQ_ERR_UNSUPPORTED);
    expect("calib huge", kq_calib_workspace_bytes((int64_t)1 << 40, (int64_t)1 << 40, (int64_t)1 << 40, &(int64_t){0}),
           KQ_ERR_UNSUPPORTED);
    expect("packed huge", kq_transform_quantize_mxfp4_packed(GOOD, (int64_t)1 << 30, 256, 256, GOOD, P(0x10000),
                                                             P(0x10000), NULL, NULL), KQ_ERR_UNSUPPORTED);
    expect("packed overflow", kq_transform_quantize_mxfp4_packed(GOOD, BIG, 256, 256, GOOD, P(0x10000), P(0x10000),
                                                                 NULL, NULL), KQ_ERR_SHAPE);
    expect("lowrank split r", kq_mxfp4_gemm_packed_lowrank_split(GOOD, GOOD, GOOD, GOOD, 4, 4, 256, GOOD, GOOD, GOOD, 48,
                                                                  P(0x10000), 4, NULL),
           KQ_ERR_SHAPE);
    expect("lowrank split huge", kq_mxfp4_gemm_packed_lowrank_split(GOOD, GOOD, GOOD, GOOD, BIG, 4, 256, GOOD, GOOD, GOOD,
                                                                     32, P(0x10000), 4, NULL),
           KQ_ERR_UNSUPPORTED);
    expect("project split huge", kq_lowrank_project_bf16_split(GOOD, BIG, 64, 64, GOOD, 32, P(0x10000), P(0x10000), NULL),
           KQ_ERR_UNSUPPORTED);
    expect("project mx split huge", kq_lowrank_project_split(GOOD, BIG, 64, 64, GOOD, GOOD, 32, P(0x10000), P(0x10000),
                                                             NULL),
           KQ_ERR_UNSUPPORTED);
    expect("project mx split r", kq_lowrank_project_split(GOOD, 4, 64, 64, GOOD, GOOD, 40, P(0x10000), P(0x10000), NULL),
           KQ_ERR_SHAPE);
    expect("y16 huge", kq_transform_quantize_mxfp4_y16(GOOD, BIG, 64, 64, GOOD, P(0x10000), P(0x10000), P(0x10000),
                                                       NULL), KQ_ERR_SHAPE);
    expect("smooth huge", kq_smoothquant_quantize_mxfp4(GOOD, 4, BIG / 64 * 32, BIG, GOOD, P(0x10000), P(0x10000),
                                                        NULL), KQ_ERR_SHAPE);
    expect("f32 huge", kq_quantize_mxfp4_f32(GOOD, BIG, 64, 64, P(0x10000), P(0x10000), NULL), KQ_ERR_SHAPE);
    expect("fold huge", kq_inverse_fold_weights(GOOD, BIG, 64, GOOD, P(0x10000), NULL), KQ_ERR_SHAPE);
    expect("hadamard huge", kq_hadamard_quantize_mxfp4(GOOD, BIG, 64, 64, 32, P(0x10000), P(0x10000), NULL, NULL),
           KQ_ERR_SHAPE);
    int64_t bytes = 0;
    expect("calib bytes", kq_calib_workspace_bytes(4096, 1152, 1152, &bytes), KQ_OK);
    if (bytes <= 0) ++failures;
    expect("calib bytes huge", kq_calib_workspace_bytes(1 << 30, 4096, 16, &bytes), KQ_ERR_UNSUPPORTED);
    expect("calib noalloc limit",
           kq_calib_step_noalloc(GOOD, GOOD, 4096, 1152, 1152, P(0x10000), P(0x10000), P(0x10000), 1, 1e-3f, 0.9f,
                                 0.999f, 1e-8f, P(0x10000), 1, P(0x10000), NULL, NULL),
           KQ_ERR_UNSUPPORTED);
    /* host-only: Eq. 6 factors on exact-size host buffers */
    const int64_t nblk = 37;
    double *abc = malloc(sizeof(double) * nblk * 15);
    float *fac = malloc(sizeof(float) * nblk * 20);
    for (int64_t i = 0; i < nblk * 15; ++i) abc[i] = (i % 3 == 0) ? 0.5 + 0.01 * (double)i : 0.25 - 0.003 * (double)i;
    expect("factors_from_lu", kq_factors_from_lu(abc, nblk, fac), KQ_OK);
    abc[3 * 7] = 0.0;
    expect("factors_from_lu a=0", kq_factors_from_lu(abc, nblk, fac), KQ_ERR_SHAPE);
    free(abc);
    free(fac);
    for (int s = 0; s <= 5; ++s)
        if (strncmp(kq_status_string((kq_status)s), "KQ_", 3) != 0) ++failures;
    if (kq_last_hip_error() != 0) ++failures;
    if (failures) {
        fprintf(stderr, "%d host-check failures\n", failures);
        return 1;
    }
    printf("libkq host-check sanitizer driver: ok\n");
    return 0;
}
