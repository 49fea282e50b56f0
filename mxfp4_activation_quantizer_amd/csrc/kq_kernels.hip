// KroQuant online activation quantizer for MI355X (gfx950): kernels and the
// C ABI declared in include/kq.h.
//
// Method: KroQuant (arXiv 2607.21446v1). Per row of A and per 32-channel block
// j, y = a . K^(j) with K^(j) = G1 (x) G2 (x) G3 (x) G4 (x) G5 (Sec. 3.2 Eq. 5,
// Sec. 3.5.1 Eq. 12), then MXFP4 (Sec. 3.1; Sec. 4.1 "Data format", App. D).
//
// Work mapping (all bf16 kernels): a workgroup of 256 lanes = 64 quads; a quad
// owns one 32-channel block of one row (16 bytes per lane). The 64 quads cover
// CB = 2^cb_log2 consecutive blocks of R = 64 / CB consecutive rows, so every
// row segment a workgroup touches is CB * 64 contiguous bytes. A workgroup
// stays on one column group (its per-block parameters load once into
// registers) and walks `iters` row tiles of one slab. The op is HBM-bound:
// 2 bytes in, 0.5 + 1/32 bytes out per element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"
#include "kq_device.hpp"

namespace kq {

constexpr int kThreads = 256;

enum Mode { kQuantOnly = 0, kSmooth = 1, kKron = 2 };

struct Geom {
    int64_t m, lda, d;
    int nblk, cb_log2, iters, ncg;
};

// Row, block column and lane-in-quad of this lane for row tile `it`.
__device__ __forceinline__ void lane_coords(const Geom &g, int &j, int &sub, int64_t &row0, int &R) {
    const int tid = threadIdx.x;
    const int quad = tid >> 2;
    sub = tid & 3;
    const int cg = blockIdx.x % g.ncg;
    const int slab = blockIdx.x / g.ncg;
    R = 64 >> g.cb_log2;
    j = (cg << g.cb_log2) + (quad & ((1 << g.cb_log2) - 1));
    row0 = (int64_t)slab * R * g.iters + (quad >> g.cb_log2);
}

template <int MODE, bool DEBUG>
__global__ __launch_bounds__(kThreads) void bf16_quant_kernel(
    const uint16_t *__restrict__ A, Geom g, const float *__restrict__ params,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ ydbg) {
    int j, sub, R;
    int64_t row0;
    lane_coords(g, j, sub, row0, R);
    const int64_t c0 = (int64_t)j * 32 + sub * 8;

    KronLane L;
    float sq[8];
    if (MODE == kKron) kron_lane_setup(params + (int64_t)j * 20, sub, L);
    if (MODE == kSmooth) {
        const float4 a = *reinterpret_cast<const float4 *>(params + c0);
        const float4 b = *reinterpret_cast<const float4 *>(params + c0 + 4);
        sq[0] = a.x; sq[1] = a.y; sq[2] = a.z; sq[3] = a.w;
        sq[4] = b.x; sq[5] = b.y; sq[6] = b.z; sq[7] = b.w;
    }

    for (int it = 0; it < g.iters; ++it) {
        const int64_t row = row0 + (int64_t)it * R;
        if (row >= g.m) break;  // uniform within a quad
        const uint4 q = *reinterpret_cast<const uint4 *>(A + row * g.lda + c0);
        float y[8];
        widen8(q, y);
        if (MODE == kSmooth) {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = y[i] * sq[i];
        }
        if (MODE == kKron) kron_apply8(y, L);
        if (DEBUG) {
            float4 *o = reinterpret_cast<float4 *>(ydbg + row * g.d + c0);
            o[0] = make_float4(y[0], y[1], y[2], y[3]);
            o[1] = make_float4(y[4], y[5], y[6], y[7]);
        }
        uint32_t sbyte;
        const uint32_t packed = quantize_quad8(y, sbyte);
        *reinterpret_cast<uint32_t *>(codes + row * (g.d / 2) + (int64_t)j * 16 + sub * 4) = packed;
        if (sub == 0) scales[row * g.nblk + j] = (uint8_t)sbyte;
    }
}

// fp32 input: the same quad layout with two 16-byte loads per lane.
// MODE kQuantOnly quantizes X; MODE kKron writes X . (K^(j))^{-T} (the weight
// fold) to `out` instead of quantizing.
template <int MODE>
__global__ __launch_bounds__(kThreads) void f32_kernel(
    const float *__restrict__ X, Geom g, const float *__restrict__ factors,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ out) {
    int j, sub, R;
    int64_t row0;
    lane_coords(g, j, sub, row0, R);
    const int64_t c0 = (int64_t)j * 32 + sub * 8;

    KronLane L;
    if (MODE == kKron) {
        // Stage factors of (K^{-1})^T = (x) (G_k^{-1})^T with G^{-1} = adj(G) / det(G),
        // so (G^{-1})^T = [[g11, -g10], [-g01, g00]] / det (computed in fp64).
        float h[20];
        const float *f = factors + (int64_t)j * 20;
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            const double g00 = f[4 * k], g01 = f[4 * k + 1], g10 = f[4 * k + 2], g11 = f[4 * k + 3];
            const double det = g00 * g11 - g01 * g10;
            h[4 * k + 0] = (float)(g11 / det);
            h[4 * k + 1] = (float)(-g10 / det);
            h[4 * k + 2] = (float)(-g01 / det);
            h[4 * k + 3] = (float)(g00 / det);
        }
        kron_lane_setup(h, sub, L);
    }

    for (int it = 0; it < g.iters; ++it) {
        const int64_t row = row0 + (int64_t)it * R;
        if (row >= g.m) break;
        const float4 *p = reinterpret_cast<const float4 *>(X + row * g.lda + c0);
        const float4 a = p[0], b = p[1];
        float y[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        if (MODE == kKron) {
            kron_apply8(y, L);
            float4 *o = reinterpret_cast<float4 *>(out + row * g.d + c0);
            o[0] = make_float4(y[0], y[1], y[2], y[3]);
            o[1] = make_float4(y[4], y[5], y[6], y[7]);
        } else {
            uint32_t sbyte;
            const uint32_t packed = quantize_quad8(y, sbyte);
            *reinterpret_cast<uint32_t *>(codes + row * (g.d / 2) + (int64_t)j * 16 + sub * 4) = packed;
            if (sub == 0) scales[row * g.nblk + j] = (uint8_t)sbyte;
        }
    }
}

}  // namespace kq

// ===========================================================================
// Host side: argument checks (no HIP call before they pass) and launches
// ===========================================================================
namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks common to every [m][ld] x d operand.
kq_status check_shape(int64_t m, int64_t d, int64_t ld) {
    if (m < 0 || d < 0 || ld < 0) return KQ_ERR_SHAPE;
    if (d % 32 != 0) return KQ_ERR_SHAPE;
    if (ld < d) return KQ_ERR_SHAPE;
    if (d / 32 > (int64_t)0x7FFFFFFF) return KQ_ERR_SHAPE;
    if (ld > 0 && m > INT64_MAX / 4 / ld) return KQ_ERR_SHAPE;  // byte offsets of fp32 rows fit
    return KQ_OK;
}

int pick_cb_log2(int64_t nblk) {
    for (int l = 4; l > 0; --l)
        if (nblk % (1 << l) == 0) return l;
    return 0;
}

// Grid: one workgroup per (column group, row slab); slabs sized so that the
// launch has about 16 workgroups per CU when the matrix is large enough.
bool make_geom(int64_t m, int64_t d, int64_t ld, kq::Geom &g, unsigned &nwg) {
    g.m = m;
    g.d = d;
    g.lda = ld;
    g.nblk = (int)(d / 32);
    g.cb_log2 = pick_cb_log2(g.nblk);
    g.ncg = g.nblk >> g.cb_log2;
    const int64_t R = 64 >> g.cb_log2;
    const int64_t row_tiles = (m + R - 1) / R;
    const int64_t units = row_tiles * g.ncg;
    const int64_t target = 256 * 16;
    int64_t iters = (units + target - 1) / target;
    if (iters < 1) iters = 1;
    if (iters > (1 << 20)) iters = 1 << 20;
    const int64_t nslab = (row_tiles + iters - 1) / iters;
    const int64_t total = nslab * g.ncg;
    if (total > 0x7FFFFFFF) return false;
    g.iters = (int)iters;
    nwg = (unsigned)total;
    return true;
}

kq_status launched() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return KQ_ERR_HIP;
    }
    return KQ_OK;
}

template <int MODE, bool DEBUG>
kq_status launch_bf16(const uint16_t *A, int64_t m, int64_t d, int64_t lda, const float *params,
                      uint8_t *codes, uint8_t *scales, float *ydbg, kq_stream_t stream) {
    kq::Geom g;
    unsigned nwg;
    if (!make_geom(m, d, lda, g, nwg)) return KQ_ERR_SHAPE;
    hipLaunchKernelGGL((kq::bf16_quant_kernel<MODE, DEBUG>), dim3(nwg), dim3(kq::kThreads), 0,
                       (hipStream_t)stream, A, g, params, codes, scales, ydbg);
    return launched();
}

kq_status check_bf16_io(const uint16_t *A, int64_t lda, const uint8_t *codes, const uint8_t *scales) {
    if (!A || !codes || !scales) return KQ_ERR_NULL;
    if (!aligned(A, 16) || lda % 8 != 0 || !aligned(codes, 16)) return KQ_ERR_ALIGN;
    return KQ_OK;
}

}  // namespace

extern "C" {

kq_status kq_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda, uint8_t *codes,
                            uint8_t *scales, kq_stream_t stream) {
    kq_status s = check_shape(m, d, lda);
    if (s != KQ_OK) return s;
    if (m == 0 || d == 0) return KQ_OK;
    if ((s = check_bf16_io(A, lda, codes, scales)) != KQ_OK) return s;
    return launch_bf16<kq::kQuantOnly, false>(A, m, d, lda, nullptr, codes, scales, nullptr, stream);
}

kq_status kq_transform_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                      const float *factors, uint8_t *codes, uint8_t *scales,
                                      float *y_debug, kq_stream_t stream) {
    kq_status s = check_shape(m, d, lda);
    if (s != KQ_OK) return s;
    if (m == 0 || d == 0) return KQ_OK;
    if ((s = check_bf16_io(A, lda, codes, scales)) != KQ_OK) return s;
    if (!factors) return KQ_ERR_NULL;
    if (!aligned(factors, 16) || (y_debug && !aligned(y_debug, 16))) return KQ_ERR_ALIGN;
    if (y_debug)
        return launch_bf16<kq::kKron, true>(A, m, d, lda, factors, codes, scales, y_debug, stream);
    return launch_bf16<kq::kKron, false>(A, m, d, lda, factors, codes, scales, nullptr, stream);
}

kq_status kq_smoothquant_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                        const float *inv_scale, uint8_t *codes, uint8_t *scales,
                                        kq_stream_t stream) {
    kq_status s = check_shape(m, d, lda);
    if (s != KQ_OK) return s;
    if (m == 0 || d == 0) return KQ_OK;
    if ((s = check_bf16_io(A, lda, codes, scales)) != KQ_OK) return s;
    if (!inv_scale) return KQ_ERR_NULL;
    if (!aligned(inv_scale, 16)) return KQ_ERR_ALIGN;
    return launch_bf16<kq::kSmooth, false>(A, m, d, lda, inv_scale, codes, scales, nullptr, stream);
}

kq_status kq_quantize_mxfp4_f32(const float *X, int64_t m, int64_t d, int64_t ldx, uint8_t *codes,
                                uint8_t *scales, kq_stream_t stream) {
    kq_status s = check_shape(m, d, ldx);
    if (s != KQ_OK) return s;
    if (m == 0 || d == 0) return KQ_OK;
    if (!X || !codes || !scales) return KQ_ERR_NULL;
    if (!aligned(X, 16) || ldx % 4 != 0 || !aligned(codes, 16)) return KQ_ERR_ALIGN;
    kq::Geom g;
    unsigned nwg;
    if (!make_geom(m, d, ldx, g, nwg)) return KQ_ERR_SHAPE;
    hipLaunchKernelGGL((kq::f32_kernel<kq::kQuantOnly>), dim3(nwg), dim3(kq::kThreads), 0,
                       (hipStream_t)stream, X, g, nullptr, codes, scales, nullptr);
    return launched();
}

kq_status kq_inverse_fold_weights(const float *W, int64_t o, int64_t d, const float *factors,
                                  float *W_folded, kq_stream_t stream) {
    kq_status s = check_shape(o, d, d);
    if (s != KQ_OK) return s;
    if (o == 0 || d == 0) return KQ_OK;
    if (!W || !factors || !W_folded) return KQ_ERR_NULL;
    if (!aligned(W, 16) || !aligned(factors, 16) || !aligned(W_folded, 16)) return KQ_ERR_ALIGN;
    kq::Geom g;
    unsigned nwg;
    if (!make_geom(o, d, d, g, nwg)) return KQ_ERR_SHAPE;
    hipLaunchKernelGGL((kq::f32_kernel<kq::kKron>), dim3(nwg), dim3(kq::kThreads), 0,
                       (hipStream_t)stream, W, g, factors, nullptr, nullptr, W_folded);
    return launched();
}

const char *kq_status_string(kq_status s) {
    switch (s) {
        case KQ_OK: return "KQ_OK";
        case KQ_ERR_NULL: return "KQ_ERR_NULL: a required pointer is NULL";
        case KQ_ERR_SHAPE: return "KQ_ERR_SHAPE: bad size (d % 32 != 0, ld < d, negative or too large)";
        case KQ_ERR_ALIGN: return "KQ_ERR_ALIGN: pointer or leading dimension misaligned";
        case KQ_ERR_HIP: return "KQ_ERR_HIP: the HIP runtime rejected the launch";
        case KQ_ERR_UNSUPPORTED: return "KQ_ERR_UNSUPPORTED";
    }
    return "unknown kq_status";
}

int kq_last_hip_error(void) { return g_last_hip_error; }

kq_status kq_factors_from_lu(const double *abc, int64_t nblk, float *factors) {
    if (nblk < 0) return KQ_ERR_SHAPE;
    if (nblk == 0) return KQ_OK;
    if (!abc || !factors) return KQ_ERR_NULL;
    for (int64_t t = 0; t < nblk * 5; ++t)
        if (abc[3 * t] == 0.0) return KQ_ERR_SHAPE;
    for (int64_t t = 0; t < nblk * 5; ++t) {
        const double a = abc[3 * t], b = abc[3 * t + 1], c = abc[3 * t + 2];
        factors[4 * t + 0] = (float)a;
        factors[4 * t + 1] = (float)b;
        factors[4 * t + 2] = (float)(c * a);
        factors[4 * t + 3] = (float)(c * b - 1.0 / a);
    }
    return KQ_OK;
}

}  // extern "C"
