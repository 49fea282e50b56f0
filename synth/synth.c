/*
 * Bulk draws for the seeded synthetic inputs (see synth/__init__.py).
 *
 * One counter-based generator, SplitMix64 (Steele, Lea and Flood, OOPSLA
 * 2014): output n of the stream keyed by k is mix64(k + (n + 1) * GAMMA).
 * Uniforms use the top 53 bits, normals the Box-Muller cosine branch on
 * uniforms 2n and 2n + 1, and float64 -> bfloat16 rounding is
 * round-to-nearest-even on the float64 significand. Nothing here knows about
 * quantization or transforms; it only draws numbers.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t raw64(uint64_t key, uint64_t n) { return mix64(key + (n + 1) * GAMMA); }

static double unif(uint64_t key, uint64_t n) {
    return (double)(raw64(key, n) >> 11) * 0x1.0p-53;
}

static double gauss(uint64_t key, uint64_t n) {
    double u1 = unif(key, 2 * n), u2 = unif(key, 2 * n + 1);
    return sqrt(-2.0 * log1p(-u1)) * cos(6.283185307179586 * u2);
}

/* float64 -> bf16 bits, round to nearest even; x finite and in bf16 range. */
static uint16_t bf16_rne(double x) {
    int ex;
    double mant = frexp(x, &ex);              /* x = mant * 2^ex, 0.5 <= |mant| < 1 */
    int keep = ex >= -125 ? 8 : ex + 133;     /* bf16 subnormal step is 2^-133 */
    double r = ldexp(nearbyint(ldexp(mant, keep)), ex - keep);
    float f = (float)r;                       /* exact: at most 8 significant bits */
    union { float f; uint32_t u; } cv;
    cv.f = f;
    return (uint16_t)(cv.u >> 16);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) { return raw64(seed, stream); }

void synth_uniform(uint64_t key, uint64_t start, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = unif(key, start + (uint64_t)i);
}

void synth_normal(uint64_t key, uint64_t start, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = gauss(key, start + (uint64_t)i);
}

void synth_to_bf16(const double *x, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(x[i]);
}

typedef struct {
    uint16_t *out;
    int64_t r0, r1, d;
    uint64_t kz;
    const double *tok;      /* [m] token scale or NULL */
    const double *colscale; /* [d] */
    const uint8_t *skew;    /* [d] or NULL */
} act_job;

static void *act_worker(void *p) {
    act_job *j = (act_job *)p;
    for (int64_t i = j->r0; i < j->r1; ++i) {
        double t = j->tok ? j->tok[i] : 1.0;
        for (int64_t c = 0; c < j->d; ++c) {
            double z = gauss(j->kz, (uint64_t)(i * j->d + c));
            if (j->skew && j->skew[c]) z = fabs(z) - 0.2;
            j->out[i * j->d + c] = bf16_rne(t * j->colscale[c] * z);
        }
    }
    return NULL;
}

/* out[i][c] = bf16(tok[i] * colscale[c] * z_ic), z_ic = normal number i*d+c of
 * stream kz (folded to |z| - 0.2 on skew channels). Rows split over threads;
 * the result does not depend on the thread count. */
void synth_activation(uint16_t *out, int64_t m, int64_t d, uint64_t kz, const double *tok,
                      const double *colscale, const uint8_t *skew, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    act_job jobs[256];
    int64_t per = (m + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t r0 = t * per, r1 = r0 + per < m ? r0 + per : m;
        if (r0 >= r1) break;
        jobs[t] = (act_job){out, r0, r1, d, kz, tok, colscale, skew};
        if (pthread_create(&th[t], NULL, act_worker, &jobs[t]) != 0) {
            act_worker(&jobs[t]);
            th[t] = 0;
        }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t)
        if (th[t]) pthread_join(th[t], NULL);
}
