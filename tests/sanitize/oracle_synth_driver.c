/*
 * Sanitizer driver for the CPU oracle (oracle/kq_oracle.c) and the input
 * generator (synth/synth.c): test infrastructure, built with
 * -fsanitize=address,undefined by tests/test_sanitizers.py and run on the
 * CPU. Every buffer is allocated at its exact size, so any read or write past
 * an operand's end, any use after free and any undefined arithmetic in either
 * file aborts the run. Shapes cover one block, ragged leading dimensions,
 * more threads than rows, and the full-width Hadamard.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle/kq_oracle.c */
double kqo_bf16_to_double(uint16_t bits);
void kqo_quantize_bf16(const uint16_t *A, int64_t m, int64_t d, int64_t lda, uint8_t *codes, uint8_t *scales,
                       int nthreads);
void kqo_quantize_f32(const float *X, int64_t m, int64_t d, int64_t ldx, uint8_t *codes, uint8_t *scales,
                      int nthreads);
void kqo_quantize_f64(const double *Y, int64_t m, int64_t d, int64_t ldy, uint8_t *codes, uint8_t *scales,
                      int nthreads);
int kqo_transform_quantize(const uint16_t *A, int64_t m, int64_t d, int64_t lda, const float *factors,
                           uint8_t *codes, uint8_t *scales, double *y_out, int nthreads);
void kqo_smoothquant_quantize(const uint16_t *A, int64_t m, int64_t d, int64_t lda, const float *inv_scale,
                              uint8_t *codes, uint8_t *scales, int nthreads);
int kqo_inverse_fold(const float *W, int64_t o, int64_t d, const float *factors, double *Wf, int nthreads);
void kqo_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t m, int64_t d, double *out);
int kqo_gemm_dequant(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                     const uint8_t *scales_w, int64_t nout, int64_t k, const int64_t *rows, int64_t nrows,
                     double *O, int nthreads);
int kqo_hadamard_quantize(const uint16_t *A, int64_t m, int64_t d, int64_t lda, int64_t n, uint8_t *codes,
                          uint8_t *scales, double *y_out, int nthreads);
int kqo_hadamard_f64(const double *X, int64_t m, int64_t d, int64_t ldx, int64_t n, double *y_out, int nthreads);
void kqo_factors_from_lu(const double *abc, int64_t nblk, double *G);
void kqo_block_K(const float *factors20, double *K1024);
void kqo_block_K_kron(const float *factors20, double *K1024);
void kqo_block_Kinv(const float *factors20, double *K1024);

/* synth/synth.c */
uint64_t synth_stream_key(uint64_t seed, uint64_t stream);
void synth_uniform(uint64_t key, uint64_t start, int64_t n, double *out);
void synth_normal(uint64_t key, uint64_t start, int64_t n, double *out);
void synth_to_bf16(const double *x, int64_t n, uint16_t *out);
void synth_activation(uint16_t *out, int64_t m, int64_t d, uint64_t kz, const double *tok, const double *colscale,
                      const uint8_t *skew, int nthreads);

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int failures = 0;
#define CHECK(cond)                                                     \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static void run_shape(int64_t m, int64_t d, int64_t lda, int threads) {
    const int64_t nblk = d / 32;
    uint64_t key = synth_stream_key(7 + m + d, 0);
    /* activations: synth draws, exact-size buffers */
    double *z = xmalloc(sizeof(double) * (size_t)(m * lda));
    synth_normal(key, 0, m * lda, z);
    for (int64_t i = 0; i < m * lda; ++i) z[i] *= (i % 13 == 0) ? 80.0 : 1.0;
    uint16_t *A = xmalloc(sizeof(uint16_t) * (size_t)(m * lda));
    synth_to_bf16(z, m * lda, A);
    double *colscale = xmalloc(sizeof(double) * (size_t)d), *tok = xmalloc(sizeof(double) * (size_t)m);
    uint8_t *skew = xmalloc((size_t)d);
    synth_uniform(synth_stream_key(3, 1), 0, d, colscale);
    synth_uniform(synth_stream_key(3, 2), 0, m, tok);
    for (int64_t c = 0; c < d; ++c) skew[c] = (uint8_t)(c % 3 == 0);
    uint16_t *A2 = xmalloc(sizeof(uint16_t) * (size_t)(m * d));
    synth_activation(A2, m, d, key, tok, colscale, skew, threads);
    /* factors: Eq. 6 parameters away from a = 0 */
    double *abc = xmalloc(sizeof(double) * (size_t)(nblk * 15));
    synth_normal(synth_stream_key(5, 5), 0, nblk * 15, abc);
    for (int64_t t = 0; t < nblk * 5; ++t) abc[3 * t] = 0.7 + 0.1 * fabs(abc[3 * t]);
    double *G = xmalloc(sizeof(double) * (size_t)(nblk * 20));
    kqo_factors_from_lu(abc, nblk, G);
    float *fac = xmalloc(sizeof(float) * (size_t)(nblk * 20));
    for (int64_t t = 0; t < nblk * 20; ++t) fac[t] = (float)G[t];
    float *inv = xmalloc(sizeof(float) * (size_t)d);
    for (int64_t c = 0; c < d; ++c) inv[c] = (float)(0.5 + colscale[c]);

    uint8_t *codes = xmalloc((size_t)(m * d / 2)), *scales = xmalloc((size_t)(m * nblk));
    uint8_t *codes2 = xmalloc((size_t)(m * d / 2)), *scales2 = xmalloc((size_t)(m * nblk));
    double *y = xmalloc(sizeof(double) * (size_t)(m * d));
    double *Af = xmalloc(sizeof(double) * (size_t)(m * d));
    float *Ax = xmalloc(sizeof(float) * (size_t)(m * d));
    for (int64_t i = 0; i < m; ++i)
        for (int64_t c = 0; c < d; ++c) {
            Af[i * d + c] = kqo_bf16_to_double(A[i * lda + c]);
            Ax[i * d + c] = (float)Af[i * d + c];
        }

    /* the three quantizer inputs agree on exactly representable values */
    kqo_quantize_bf16(A, m, d, lda, codes, scales, threads);
    kqo_quantize_f64(Af, m, d, d, codes2, scales2, threads);
    CHECK(memcmp(codes, codes2, (size_t)(m * d / 2)) == 0 && memcmp(scales, scales2, (size_t)(m * nblk)) == 0);
    kqo_quantize_f32(Ax, m, d, d, codes2, scales2, threads);
    CHECK(memcmp(codes, codes2, (size_t)(m * d / 2)) == 0);
    CHECK(kqo_transform_quantize(A, m, d, lda, fac, codes, scales, y, threads) == 0);
    CHECK(kqo_transform_quantize(A, m, d, lda, fac, NULL, NULL, y, threads) == 0);
    kqo_smoothquant_quantize(A, m, d, lda, inv, codes, scales, threads);

    double *deq = xmalloc(sizeof(double) * (size_t)(m * d));
    kqo_dequantize(codes, scales, m, d, deq);
    int64_t *rows = xmalloc(sizeof(int64_t) * (size_t)m);
    for (int64_t i = 0; i < m; ++i) rows[i] = m - 1 - i;
    double *O = xmalloc(sizeof(double) * (size_t)(m * m));
    CHECK(kqo_gemm_dequant(codes, scales, codes, scales, m, d, rows, m, O, threads) == 0);

    double *Wf = xmalloc(sizeof(double) * (size_t)(m * d));
    CHECK(kqo_inverse_fold(Ax, m, d, fac, Wf, threads) == 0);
    double K[1024], Kk[1024], Ki[1024];
    kqo_block_K(fac, K);
    kqo_block_K_kron(fac, Kk);
    kqo_block_Kinv(fac, Ki);
    for (int i = 0; i < 1024; ++i) CHECK(fabs(K[i] - Kk[i]) <= 1e-12 * (1.0 + fabs(K[i])));

    for (int64_t n = 32; n <= d; n *= 2) {
        if (d % n) continue;
        CHECK(kqo_hadamard_quantize(A, m, d, lda, n, codes, scales, y, threads) == 0);
        CHECK(kqo_hadamard_f64(Af, m, d, d, n, y, threads) == 0);
    }
    CHECK(kqo_hadamard_quantize(A, m, d, lda, 48, codes, scales, y, threads) == -1);

    free(z); free(A); free(colscale); free(tok); free(skew); free(A2); free(abc); free(G); free(fac); free(inv);
    free(codes); free(scales); free(codes2); free(scales2); free(y); free(Af); free(Ax); free(deq); free(rows);
    free(O); free(Wf);
}

int main(void) {
    run_shape(1, 32, 32, 1);
    run_shape(3, 64, 72, 8);     /* more threads than rows, padded rows */
    run_shape(17, 256, 264, 4);
    run_shape(9, 1152, 1152, 3);
    run_shape(2, 4096, 4104, 2);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle/synth sanitizer driver: ok\n");
    return 0;
}
