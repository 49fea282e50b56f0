/*
 * KroQuant activation quantizer -- CPU ORACLE (test infrastructure only).
 *
 * Plain, slow, obviously-correct reference for what the GPU library computes.
 * It is used by the tests, the smoke check and the bench's CPU-baseline leg,
 * and by nothing on the product path. It shares no code, header or table with
 * the GPU library. Every quantity is formed in float64 from its definition.
 *
 * Sources (KroQuant, arXiv 2607.21446v1; "the paper" below):
 *   Sec. 1, Eq. 1      A -> A T, W -> W T^{-T}; the product A W^T is unchanged.
 *   Sec. 3.1           blockwise quantizer: each row split into blocks of n,
 *                      each block stored as one shared scale plus an n-vector
 *                      of b-bit values.
 *   Sec. 3.1, Eq. 4    T = diag(K^(1), ..., K^(d/32)).
 *   Sec. 3.2, Eq. 5    K = G1 (x) G2 (x) ... (x) G5 (Kronecker product).
 *   Sec. 3.2           (G1 (x) ... (x) G5)^{-1} = G1^{-1} (x) ... (x) G5^{-1}.
 *   Sec. 3.2, Eq. 6    G = [[1,0],[c,1]] . [[a,b],[0,-1/a]].
 *   Sec. 3.5.1, Eq. 12 K[r,c] = prod_{k=1..5} G_k[bit_{5-k}(r), bit_{5-k}(c)].
 *   Sec. 4.1 "Data format" and Appendix D: MXFP4 E2M1 elements, FP8 E8M0
 *                      block scale, block size 32, per the OCP MX spec.
 *   Appendix D.2       SmoothQuant per-channel vector gamma.
 *   Sec. 3.2 "Hadamard initialization", Sec. 1, Sec. 4.4 (Table 2's
 *                      Hadamard-32 row, Table 3's FWHT): the normalized
 *                      Hadamard matrix of order n = 2^k, the k-fold Kronecker
 *                      power of [[1,1],[1,-1]]/sqrt(2), applied to each group
 *                      of n consecutive channels (n = d: full-width transform).
 *
 * Readings taken where the paper is silent (OCP MX v1.0 conventions):
 *   - shared exponent e = floor(log2(max|y|)) - 2 (2 = largest E2M1 exponent),
 *     clamped to [-127, 127]; an all-zero block takes e = -127; the E8M0 byte
 *     is e + 127;
 *   - each element v = y / 2^e is rounded to the nearest E2M1 magnitude
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, so |v| > 6 lands on 6;
 *   - code = sign(y) << 3 | index of the magnitude; the sign bit follows y,
 *     including -0;
 *   - two codes per byte, element 2k in the low nibble of byte k; codes are
 *     [m][d/2] bytes and scales [m][d/32] bytes, both row-major.
 *   - the transformed block y = a . K is quantized directly (no rounding of y
 *     to the input dtype first).
 *   - SmoothQuant multiplies each input by the fp32 inverse scale in one IEEE
 *     fp32 multiply, then quantizes.
 */
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Scalars                                                                   */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes by 3-bit index (1 sign, 2 exponent, 1 mantissa bit). */
static const double E2M1_LEVEL[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double kqo_bf16_to_double(uint16_t bits) {
    union { uint32_t u; float f; } cv;
    cv.u = (uint32_t)bits << 16;
    return (double)cv.f;
}

double kqo_e2m1_value(uint8_t code) {
    double v = E2M1_LEVEL[code & 7];
    return (code & 8) ? -v : v;
}

/* Index of the E2M1 magnitude nearest to v >= 0; on a tie the even index. */
int kqo_e2m1_round_index(double v) {
    int best = 0;
    double bestd = fabs(v - E2M1_LEVEL[0]);
    for (int i = 1; i < 8; ++i) {
        double dd = fabs(v - E2M1_LEVEL[i]);
        if (dd < bestd || (dd == bestd && (i % 2) == 0)) {
            best = i;
            bestd = dd;
        }
    }
    return best;
}

/* Shared exponent of a block whose largest magnitude is amax. */
int kqo_shared_exponent(double amax) {
    if (amax == 0.0) return -127;
    int ex;
    frexp(amax, &ex);          /* amax = f * 2^ex with 0.5 <= f < 1 */
    int e = (ex - 1) - 2;      /* floor(log2 amax) - emax(E2M1) */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Quantize one block of 32 float64 values: 16 code bytes and one scale byte. */
void kqo_quantize_block(const double *y, uint8_t *codes16, uint8_t *scale) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i)
        if (fabs(y[i]) > amax) amax = fabs(y[i]);
    int e = kqo_shared_exponent(amax);
    memset(codes16, 0, 16);
    for (int i = 0; i < 32; ++i) {
        double v = ldexp(fabs(y[i]), -e);
        uint8_t code = (uint8_t)kqo_e2m1_round_index(v);
        if (signbit(y[i])) code |= 8;
        codes16[i / 2] |= (uint8_t)(code << ((i % 2) * 4));
    }
    *scale = (uint8_t)(e + 127);
}

/* ------------------------------------------------------------------------ */
/* Kronecker blocks                                                          */
/* ------------------------------------------------------------------------ */

/* Eq. 12: K[r][c] = prod_k G_k[bit_{5-k}(r)][bit_{5-k}(c)], k = 1..5 (G[0] is G1). */
void kqo_build_K_eq12(const double G[5][2][2], double K[32][32]) {
    for (int r = 0; r < 32; ++r)
        for (int c = 0; c < 32; ++c) {
            double p = 1.0;
            for (int k = 1; k <= 5; ++k) {
                int bit = 5 - k;
                p *= G[k - 1][(r >> bit) & 1][(c >> bit) & 1];
            }
            K[r][c] = p;
        }
}

/* Eq. 5 by repeated Kronecker products: M <- M (x) G_k, starting from G_1. */
void kqo_build_K_kron(const double G[5][2][2], double K[32][32]) {
    double M[32][32], N[32][32];
    int n = 2;
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) M[i][j] = G[0][i][j];
    for (int k = 1; k < 5; ++k) {
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j)
                for (int p = 0; p < 2; ++p)
                    for (int q = 0; q < 2; ++q)
                        N[2 * i + p][2 * j + q] = M[i][j] * G[k][p][q];
        n *= 2;
        memcpy(M, N, sizeof(M));
    }
    memcpy(K, M, sizeof(M));
}

static void widen_factors(const float *f20, double G[5][2][2]) {
    for (int k = 0; k < 5; ++k)
        for (int i = 0; i < 2; ++i)
            for (int j = 0; j < 2; ++j) G[k][i][j] = (double)f20[k * 4 + i * 2 + j];
}

/* 2x2 inverse by adjugate over determinant (Sec. 3.2: the inverse of the
 * Kronecker product is the Kronecker product of the five 2x2 inverses). */
static void inverse_factors(const double G[5][2][2], double Gi[5][2][2]) {
    for (int k = 0; k < 5; ++k) {
        double det = G[k][0][0] * G[k][1][1] - G[k][0][1] * G[k][1][0];
        Gi[k][0][0] = G[k][1][1] / det;
        Gi[k][0][1] = -G[k][0][1] / det;
        Gi[k][1][0] = -G[k][1][0] / det;
        Gi[k][1][1] = G[k][0][0] / det;
    }
}

void kqo_block_K(const float *factors20, double *K1024) {
    double G[5][2][2];
    widen_factors(factors20, G);
    kqo_build_K_eq12(G, (double(*)[32])K1024);
}

void kqo_block_K_kron(const float *factors20, double *K1024) {
    double G[5][2][2];
    widen_factors(factors20, G);
    kqo_build_K_kron(G, (double(*)[32])K1024);
}

void kqo_block_Kinv(const float *factors20, double *K1024) {
    double G[5][2][2], Gi[5][2][2];
    widen_factors(factors20, G);
    inverse_factors(G, Gi);
    kqo_build_K_eq12(Gi, (double(*)[32])K1024);
}

/* Eq. 6: G = [[1,0],[c,1]] . [[a,b],[0,-1/a]] = [[a, b],[c a, c b - 1/a]]. */
void kqo_factors_from_lu(const double *abc, int64_t nblk, double *G) {
    for (int64_t t = 0; t < nblk * 5; ++t) {
        double a = abc[3 * t], b = abc[3 * t + 1], c = abc[3 * t + 2];
        double L[2][2] = {{1.0, 0.0}, {c, 1.0}};
        double U[2][2] = {{a, b}, {0.0, -1.0 / a}};
        for (int i = 0; i < 2; ++i)
            for (int j = 0; j < 2; ++j) G[4 * t + 2 * i + j] = L[i][0] * U[0][j] + L[i][1] * U[1][j];
    }
}

/* ------------------------------------------------------------------------ */
/* Row-parallel driver                                                       */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void *ctx, int64_t r0, int64_t r1);

typedef struct {
    row_fn fn;
    void *ctx;
    int64_t r0, r1;
} row_job;

static void *row_worker(void *p) {
    row_job *j = (row_job *)p;
    j->fn(j->ctx, j->r0, j->r1);
    return NULL;
}

int kqo_default_threads(void) {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int n = CPU_COUNT(&set);
        if (n > 0) return n;
    }
    return 1;
}

static void parallel_rows(int64_t m, int nthreads, row_fn fn, void *ctx) {
    if (nthreads <= 0) nthreads = kqo_default_threads();
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > m) nthreads = (int)(m > 0 ? m : 1);
    if (nthreads == 1) {
        fn(ctx, 0, m);
        return;
    }
    pthread_t th[256];
    row_job jobs[256];
    int ok[256];
    int64_t per = (m + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        int64_t r0 = (int64_t)t * per, r1 = r0 + per < m ? r0 + per : m;
        if (r0 > m) r0 = m;
        jobs[t] = (row_job){fn, ctx, r0, r1};
        ok[t] = pthread_create(&th[t], NULL, row_worker, &jobs[t]) == 0;
        if (!ok[t]) row_worker(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (ok[t]) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Path entry points                                                         */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *A;      /* bf16 bits, [m][lda] */
    const float *X;         /* fp32, [m][lda] */
    const double *Y;        /* fp64, [m][lda] */
    int64_t d, lda;
    const float *factors;   /* [d/32][5][2][2] */
    const float *inv_scale; /* [d] */
    uint8_t *codes;         /* [m][d/2] */
    uint8_t *scales;        /* [m][d/32] */
    double *y_out;          /* [m][d] or NULL */
    const double *Kall;     /* [d/32][32][32] precomputed blocks */
} qctx;

/* Quantize-only on bf16 input: y = a. */
static void rows_quantize_bf16(void *p, int64_t r0, int64_t r1) {
    qctx *c = (qctx *)p;
    double y[32];
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < c->d / 32; ++j) {
            for (int t = 0; t < 32; ++t) y[t] = kqo_bf16_to_double(c->A[i * c->lda + 32 * j + t]);
            kqo_quantize_block(y, c->codes + i * (c->d / 2) + 16 * j, c->scales + i * (c->d / 32) + j);
        }
}

void kqo_quantize_bf16(const uint16_t *A, int64_t m, int64_t d, int64_t lda, uint8_t *codes,
                       uint8_t *scales, int nthreads) {
    qctx c = {.A = A, .d = d, .lda = lda, .codes = codes, .scales = scales};
    parallel_rows(m, nthreads, rows_quantize_bf16, &c);
}

static void rows_quantize_f32(void *p, int64_t r0, int64_t r1) {
    qctx *c = (qctx *)p;
    double y[32];
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < c->d / 32; ++j) {
            for (int t = 0; t < 32; ++t) y[t] = (double)c->X[i * c->lda + 32 * j + t];
            kqo_quantize_block(y, c->codes + i * (c->d / 2) + 16 * j, c->scales + i * (c->d / 32) + j);
        }
}

void kqo_quantize_f32(const float *X, int64_t m, int64_t d, int64_t ldx, uint8_t *codes,
                      uint8_t *scales, int nthreads) {
    qctx c = {.X = X, .d = d, .lda = ldx, .codes = codes, .scales = scales};
    parallel_rows(m, nthreads, rows_quantize_f32, &c);
}

static void rows_quantize_f64(void *p, int64_t r0, int64_t r1) {
    qctx *c = (qctx *)p;
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < c->d / 32; ++j)
            kqo_quantize_block(c->Y + i * c->lda + 32 * j, c->codes + i * (c->d / 2) + 16 * j,
                               c->scales + i * (c->d / 32) + j);
}

void kqo_quantize_f64(const double *Y, int64_t m, int64_t d, int64_t ldy, uint8_t *codes,
                      uint8_t *scales, int nthreads) {
    qctx c = {.Y = Y, .d = d, .lda = ldy, .codes = codes, .scales = scales};
    parallel_rows(m, nthreads, rows_quantize_f64, &c);
}

/* y_c = sum_r a_r K[r][c] (row of A times the block, Eq. 1's A T), r in order. */
static void rows_transform(void *p, int64_t r0, int64_t r1) {
    qctx *c = (qctx *)p;
    double a[32], y[32];
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < c->d / 32; ++j) {
            const double *K = c->Kall + j * 1024;
            for (int t = 0; t < 32; ++t) a[t] = kqo_bf16_to_double(c->A[i * c->lda + 32 * j + t]);
            for (int col = 0; col < 32; ++col) {
                double s = 0.0;
                for (int r = 0; r < 32; ++r) s += a[r] * K[r * 32 + col];
                y[col] = s;
            }
            if (c->y_out)
                for (int t = 0; t < 32; ++t) c->y_out[i * c->d + 32 * j + t] = y[t];
            if (c->codes)
                kqo_quantize_block(y, c->codes + i * (c->d / 2) + 16 * j, c->scales + i * (c->d / 32) + j);
        }
}

static double *all_blocks(const float *factors, int64_t nblk, int inverse) {
    double *K = (double *)malloc(sizeof(double) * 1024 * (size_t)(nblk > 0 ? nblk : 1));
    if (!K) return NULL;
    for (int64_t j = 0; j < nblk; ++j) {
        if (inverse)
            kqo_block_Kinv(factors + 20 * j, K + 1024 * j);
        else
            kqo_block_K(factors + 20 * j, K + 1024 * j);
    }
    return K;
}

/* Fused transform + quantize; any of codes/scales (both) and y_out may be NULL. */
int kqo_transform_quantize(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                           const float *factors, uint8_t *codes, uint8_t *scales, double *y_out,
                           int nthreads) {
    double *K = all_blocks(factors, d / 32, 0);
    if (!K) return -1;
    qctx c = {.A = A, .d = d, .lda = lda, .factors = factors, .codes = codes, .scales = scales,
              .y_out = y_out, .Kall = K};
    parallel_rows(m, nthreads, rows_transform, &c);
    free(K);
    return 0;
}

/* SmoothQuant: y_c = fl32(a_c * inv_scale_c) (one fp32 multiply), then quantize. */
static void rows_smoothquant(void *p, int64_t r0, int64_t r1) {
    qctx *c = (qctx *)p;
    double y[32];
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < c->d / 32; ++j) {
            for (int t = 0; t < 32; ++t) {
                volatile float a = (float)kqo_bf16_to_double(c->A[i * c->lda + 32 * j + t]);
                volatile float s = c->inv_scale[32 * j + t];
                volatile float prod = a * s;
                y[t] = (double)prod;
            }
            kqo_quantize_block(y, c->codes + i * (c->d / 2) + 16 * j, c->scales + i * (c->d / 32) + j);
        }
}

void kqo_smoothquant_quantize(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                              const float *inv_scale, uint8_t *codes, uint8_t *scales,
                              int nthreads) {
    qctx c = {.A = A, .d = d, .lda = lda, .inv_scale = inv_scale, .codes = codes, .scales = scales};
    parallel_rows(m, nthreads, rows_smoothquant, &c);
}

/* Weight fold W' = W T^{-T}: per block w'_c = sum_r w_r (K^{-1})^T[r][c] = sum_r w_r Kinv[c][r]. */
typedef struct {
    const float *W;
    int64_t d;
    double *Wf;
    const double *Kinv;
} fctx;

static void rows_fold(void *p, int64_t r0, int64_t r1) {
    fctx *c = (fctx *)p;
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < c->d / 32; ++j) {
            const double *Ki = c->Kinv + j * 1024;
            const float *w = c->W + i * c->d + 32 * j;
            for (int col = 0; col < 32; ++col) {
                double s = 0.0;
                for (int r = 0; r < 32; ++r) s += (double)w[r] * Ki[col * 32 + r];
                c->Wf[i * c->d + 32 * j + col] = s;
            }
        }
}

int kqo_inverse_fold(const float *W, int64_t o, int64_t d, const float *factors, double *Wf,
                     int nthreads) {
    double *Ki = all_blocks(factors, d / 32, 1);
    if (!Ki) return -1;
    fctx c = {W, d, Wf, Ki};
    parallel_rows(o, nthreads, rows_fold, &c);
    free(Ki);
    return 0;
}

/* Decoded value (-1)^s * level * 2^(scale - 127). */
void kqo_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t m, int64_t d, double *out) {
    for (int64_t i = 0; i < m; ++i)
        for (int64_t c = 0; c < d; ++c) {
            uint8_t byte = codes[i * (d / 2) + c / 2];
            uint8_t code = (c % 2) ? (byte >> 4) : (byte & 15);
            int e = (int)scales[i * (d / 32) + c / 32] - 127;
            out[i * d + c] = ldexp(kqo_e2m1_value(code), e);
        }
}

/* O[r][n] = sum_k deq(A)[rows[r]][k] * deq(W)[n][k] in float64 for selected rows. */
typedef struct {
    const uint8_t *ca, *sa, *cw, *sw;
    int64_t nout, k;
    const int64_t *rows;
    double *O;
    const double *Wdq;
} gctx;

static void rows_gemm(void *p, int64_t r0, int64_t r1) {
    gctx *c = (gctx *)p;
    double *a = (double *)malloc(sizeof(double) * (size_t)c->k);
    if (!a) return;
    for (int64_t r = r0; r < r1; ++r) {
        int64_t i = c->rows[r];
        kqo_dequantize(c->ca + i * (c->k / 2), c->sa + i * (c->k / 32), 1, c->k, a);
        for (int64_t n = 0; n < c->nout; ++n) {
            const double *w = c->Wdq + n * c->k;
            double s = 0.0;
            for (int64_t t = 0; t < c->k; ++t) s += a[t] * w[t];
            c->O[r * c->nout + n] = s;
        }
    }
    free(a);
}

int kqo_gemm_dequant(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                     const uint8_t *scales_w, int64_t nout, int64_t k, const int64_t *rows,
                     int64_t nrows, double *O, int nthreads) {
    double *Wdq = (double *)malloc(sizeof(double) * (size_t)(nout * k > 0 ? nout * k : 1));
    if (!Wdq) return -1;
    kqo_dequantize(codes_w, scales_w, nout, k, Wdq);
    gctx c = {codes_a, scales_a, codes_w, scales_w, nout, k, rows, O, Wdq};
    parallel_rows(nrows, nthreads, rows_gemm, &c);
    free(Wdq);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Block Hadamard (the fixed-rotation baselines)                             */
/* ------------------------------------------------------------------------ */

/* Sylvester form of the k-fold Kronecker power of [[1,1],[1,-1]]:
 * H_n[r][c] = (-1)^popcount(r & c); the normalized matrix divides by sqrt(n).
 * For each row and each group g of n channels,
 *     y[g n + c] = (1 / sqrt(n)) * sum_{r = 0..n-1} x[g n + r] H_n[r][c],
 * summed in float64 with r in order (a dense O(n^2) product per group). */
static void hadamard_group(const double *x, int64_t n, double inv_sqrt_n, double *y) {
    for (int64_t col = 0; col < n; ++col) {
        double s = 0.0;
        for (int64_t r = 0; r < n; ++r) {
            if (__builtin_popcountll((unsigned long long)(r & col)) & 1)
                s -= x[r];
            else
                s += x[r];
        }
        y[col] = s * inv_sqrt_n;
    }
}

typedef struct {
    const uint16_t *A; /* bf16 bits [m][lda], or NULL */
    const double *X;   /* fp64 [m][lda], or NULL */
    int64_t d, lda, n;
    uint8_t *codes, *scales;
    double *y_out;
} hctx;

static void rows_hadamard(void *p, int64_t r0, int64_t r1) {
    hctx *c = (hctx *)p;
    double *x = (double *)malloc(sizeof(double) * (size_t)c->d);
    double *y = (double *)malloc(sizeof(double) * (size_t)c->d);
    if (!x || !y) {
        free(x);
        free(y);
        return;
    }
    const double inv_sqrt_n = 1.0 / sqrt((double)c->n);
    for (int64_t i = r0; i < r1; ++i) {
        for (int64_t t = 0; t < c->d; ++t)
            x[t] = c->A ? kqo_bf16_to_double(c->A[i * c->lda + t]) : c->X[i * c->lda + t];
        for (int64_t g = 0; g < c->d / c->n; ++g) hadamard_group(x + g * c->n, c->n, inv_sqrt_n, y + g * c->n);
        if (c->y_out)
            for (int64_t t = 0; t < c->d; ++t) c->y_out[i * c->d + t] = y[t];
        if (c->codes)
            for (int64_t j = 0; j < c->d / 32; ++j)
                kqo_quantize_block(y + 32 * j, c->codes + i * (c->d / 2) + 16 * j, c->scales + i * (c->d / 32) + j);
    }
    free(x);
    free(y);
}

/* Block-Hadamard transform of bf16 A (group size n, a power of two dividing d),
 * then quantize; codes/scales (both) and y_out may be NULL. Returns -1 on a
 * bad n. */
int kqo_hadamard_quantize(const uint16_t *A, int64_t m, int64_t d, int64_t lda, int64_t n,
                          uint8_t *codes, uint8_t *scales, double *y_out, int nthreads) {
    if (n < 1 || (n & (n - 1)) != 0 || d % n != 0) return -1;
    hctx c = {.A = A, .d = d, .lda = lda, .n = n, .codes = codes, .scales = scales, .y_out = y_out};
    parallel_rows(m, nthreads, rows_hadamard, &c);
    return 0;
}

/* The same transform of float64 rows (no quantization), for checking the
 * transform on inputs that are not bf16. */
int kqo_hadamard_f64(const double *X, int64_t m, int64_t d, int64_t ldx, int64_t n, double *y_out,
                     int nthreads) {
    if (n < 1 || (n & (n - 1)) != 0 || d % n != 0) return -1;
    hctx c = {.X = X, .d = d, .lda = ldx, .n = n, .y_out = y_out};
    parallel_rows(m, nthreads, rows_hadamard, &c);
    return 0;
}
