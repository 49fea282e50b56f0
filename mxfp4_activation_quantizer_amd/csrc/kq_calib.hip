// Layer-wise calibration of the Kronecker factors on gfx950 (KroQuant, arXiv
// 2607.21446v1, Sec. 3.3): minimize
//   L = ||Q(A T) Q(W T^{-T})^T - A W^T||^2 / (M o)                  (Eq. 7)
//     + lambda_A ||Q(A T) - A T||^2 / (M d)                          (Eq. 8)
//     + lambda_W ||Q(W T^{-T}) - W T^{-T}||^2 / (o d)                (Eq. 8)
// over the 15 parameters per block (a, b, c per factor, Eq. 6) with Adam and a
// straight-through estimator; lambda from Eq. 10 at the Hadamard start.
//
// Straight-through reading: inside the output product Q passes gradients
// unchanged; inside the operand terms the quantized value is held fixed, so
// dL_A/dX = -2 (Q(X) - X) / (M d) (with the identity there too those terms
// would contribute nothing).
//
// One step is a fixed sequence of launches on caller-provided workspace:
//   factors   theta -> G (Eq. 6) and (G^{-1})^T per block and factor;
//   qdq       X = A T and Y = W T^{-T} (five 2x2 stages per block, quad layout),
//             their MXFP4 quantize-dequantize, and partial sums of the Eq. 8 terms;
//   gemm      E = Q(X) Q(Y)^T - A W^T (A W^T kept from init), partial sums of E^2;
//   losses    the three terms, and lambda when asked (Eq. 10);
//   gemm      E Q(Y) and E^T Q(X);
//   outer     per block j, over row chunks: A_j^T G_X,j and W_j^T G_Y,j with
//             G_X = 2/(M o) E Q(Y) - lambda_A 2/(M d) (Q(X) - X), G_Y likewise;
//   update    per block: dL/dK = A-part - K^{-T} (W-part)^T K^{-T} (Y = W P,
//             P = K^{-T}, dP = -K^{-T} dK^T K^{-T}), dL/dG_k through Eq. 12,
//             dL/d(a, b, c) through Eq. 6, then Adam (Kingma and Ba 2014).
// All reductions run in a fixed order: results are deterministic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kq.h"
#include "kq_device.hpp"
#include "kq_host.hpp"

namespace kq {

// --- theta -> factors -------------------------------------------------------
__global__ __launch_bounds__(256) void calib_factors_kernel(const float *__restrict__ theta, int64_t nfac,
                                                            float *__restrict__ fac,
                                                            float *__restrict__ facit) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nfac) return;
    const float a = theta[3 * t], b = theta[3 * t + 1], c = theta[3 * t + 2];
    const float g00 = a, g01 = b, g10 = c * a, g11 = c * b - 1.0f / a;
    fac[4 * t + 0] = g00;
    fac[4 * t + 1] = g01;
    fac[4 * t + 2] = g10;
    fac[4 * t + 3] = g11;
    // (G^{-1})^T = [[g11, -g10], [-g01, g00]] / det, in fp64
    const double det = (double)g00 * g11 - (double)g01 * g10;
    facit[4 * t + 0] = (float)(g11 / det);
    facit[4 * t + 1] = (float)(-g10 / det);
    facit[4 * t + 2] = (float)(-g01 / det);
    facit[4 * t + 3] = (float)(g00 / det);
}

// --- transform + quantize-dequantize ------------------------------------------
__device__ __forceinline__ float e2m1_value(uint32_t n) {  // magnitude of a 3-bit E2M1 index
    return n < 2 ? 0.5f * (float)n : ldexpf(1.0f + 0.5f * (float)(n & 1), (int)(n >> 1) - 1);
}

// Block reduction of one double per thread (256 threads), fixed order; result in thread 0.
__device__ __forceinline__ double block_sum(double v) {
    __shared__ double red[256];
    red[threadIdx.x] = v;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    return red[0];
}

// One quad per (row, block), grid-stride over all of them. T = in . K (five
// stages with the block's factors), Tq = its MXFP4 quantize-dequantize;
// partial[blockIdx] = sum over this workgroup of (Tq - T)^2.
template <bool BF16>
__global__ __launch_bounds__(256) void calib_qdq_kernel(const void *__restrict__ in, int64_t rows, int64_t d,
                                                        const float *__restrict__ fac,
                                                        float *__restrict__ T, float *__restrict__ Tq,
                                                        double *__restrict__ partial) {
    const int sub = threadIdx.x & 3;
    const int64_t nblk = d / 32, nq = rows * nblk;
    double acc = 0.0;
    for (int64_t q = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2); q < nq; q += (int64_t)gridDim.x * 64) {
        const int64_t row = q / nblk, j = q - row * nblk;
        const int64_t off = row * d + j * 32 + sub * 8;
        float x[8];
        if (BF16) {
            const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(in) + off);
            widen8(w, x);
        } else {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(in) + off);
            const float4 u = p[0], v = p[1];
            x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
        }
        KronLane L;
        kron_lane_setup(fac + j * 20, sub, L);
        kron_apply8(x, L);
        uint32_t sbyte;
        const uint32_t packed = quantize_quad_f32(x, sbyte);
        const float scale = ldexpf(1.0f, (int)sbyte - 127);
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t code = (packed >> (4 * i)) & 15u;
            const float v = e2m1_value(code & 7u) * scale;
            y[i] = (code & 8u) ? -v : v;
            const double e = (double)y[i] - (double)x[i];
            acc += e * e;
        }
        float4 *o = reinterpret_cast<float4 *>(T + off);
        o[0] = make_float4(x[0], x[1], x[2], x[3]);
        o[1] = make_float4(x[4], x[5], x[6], x[7]);
        float4 *oq = reinterpret_cast<float4 *>(Tq + off);
        oq[0] = make_float4(y[0], y[1], y[2], y[3]);
        oq[1] = make_float4(y[4], y[5], y[6], y[7]);
    }
    const double s = block_sum(acc);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// bf16 -> fp32 copy (the calibration keeps A in fp32 once).
__global__ __launch_bounds__(256) void widen_kernel(const uint16_t *__restrict__ A, int64_t n,
                                                    float *__restrict__ out) {
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += (int64_t)gridDim.x * 256 * 8) {
        const uint4 w = *reinterpret_cast<const uint4 *>(A + i);
        float x[8];
        widen8(w, x);
        float4 *o = reinterpret_cast<float4 *>(out + i);
        o[0] = make_float4(x[0], x[1], x[2], x[3]);
        o[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
}

// --- fp32 GEMM: D = alpha op(A) op(B) + beta C ----------------------------------
// On the fp32 matrix instruction v_mfma_f32_32x32x2_f32 (gfx950 runs it at the fp32
// peak without packed vector math). 128 x 128 output tile per workgroup of four
// waves, each wave 64 x 64 = 2 x 2 instruction tiles; k in steps of 16 through LDS,
// double-buffered, both operands staged k-major (As[k][m], Bs[k][n]) so a matrix
// operand (lane l: row or column l % 32 at k row 2 kk + l / 32) is 32 consecutive
// floats; rows are padded to 160 floats, which puts the two k rows a read touches
// in opposite bank halves. The next step's elements go to registers before the
// current step's matrix work and to LDS after it. op(A) is m x k (A row-major m x k,
// or k x m when TA); op(B) is k x n (B row-major k x n, or n x k when TB). Elements
// past m, n or k read as zero. Optional: per-workgroup sum of squares of D (double).
constexpr int kGT = 128;      // output tile
constexpr int kGK = 16;       // k per step
constexpr int kGP = kGT + 32; // LDS row pitch (floats)

typedef float floatx16_t __attribute__((ext_vector_type(16)));

template <bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(256) void gemm_f32_kernel(int64_t m, int64_t n, int64_t k, float alpha,
                                                       const float *__restrict__ A, int64_t lda,
                                                       const float *__restrict__ B, int64_t ldb, float beta,
                                                       const float *__restrict__ C, int64_t ldc,
                                                       float *__restrict__ D, int64_t ldd,
                                                       double *__restrict__ sumsq) {
    __shared__ __attribute__((aligned(16))) float As[2][kGK][kGP];
    __shared__ __attribute__((aligned(16))) float Bs[2][kGK][kGP];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t tiles_n = (n + kGT - 1) / kGT;
    const int64_t m0 = (blockIdx.x / tiles_n) * kGT, n0 = (blockIdx.x % tiles_n) * kGT;
    // staging of one step, 8 elements of each operand per thread:
    //   row-major m x k side: row t % 128, k 8 (t / 128) .. + 7 (a wave writes 64
    //   consecutive rows of one k row of the tile: no bank conflicts);
    //   k-major side: k row t / 16, columns 8 (t % 16) .. + 7
    float ra[8], rb[8];
    // 8 consecutive elements of one row of a row-major matrix, as two 16-byte loads when
    // VEC (16-byte aligned matrix, row stride a multiple of 4) and all 8 are in range
    auto run8 = [&](const float *M, int64_t ld, int64_t row, int64_t rows, int64_t c0, int64_t cols, float v[8]) {
        if (VEC && row < rows && c0 + 7 < cols) {
            const float4 x = *reinterpret_cast<const float4 *>(M + row * ld + c0);
            const float4 y = *reinterpret_cast<const float4 *>(M + row * ld + c0 + 4);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
            v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (row < rows && c0 + e < cols) ? M[row * ld + c0 + e] : 0.0f;
        }
    };
    auto fetch = [&](int64_t k0) {
        if (VEC) {
            if (!TA) run8(A, lda, m0 + (t & 127), m, k0 + 8 * (t >> 7), k, ra);
            else run8(A, lda, k0 + (t >> 4), k, m0 + 8 * (t & 15), m, ra);
            if (!TB) run8(B, ldb, k0 + (t >> 4), k, n0 + 8 * (t & 15), n, rb);
            else run8(B, ldb, n0 + (t & 127), n, k0 + 8 * (t >> 7), k, rb);
            return;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (!TA) {
                const int64_t gm = m0 + (t & 127), gk = k0 + 8 * (t >> 7) + e;
                ra[e] = (gm < m && gk < k) ? A[gm * lda + gk] : 0.0f;
            } else {
                const int64_t gk = k0 + (t >> 4), gm = m0 + 8 * (t & 15) + e;
                ra[e] = (gm < m && gk < k) ? A[gk * lda + gm] : 0.0f;
            }
            if (!TB) {
                const int64_t gk = k0 + (t >> 4), gn = n0 + 8 * (t & 15) + e;
                rb[e] = (gn < n && gk < k) ? B[gk * ldb + gn] : 0.0f;
            } else {
                const int64_t gn = n0 + (t & 127), gk = k0 + 8 * (t >> 7) + e;
                rb[e] = (gn < n && gk < k) ? B[gn * ldb + gk] : 0.0f;
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (!TA) As[buf][8 * (t >> 7) + e][t & 127] = ra[e];
            else As[buf][t >> 4][8 * (t & 15) + e] = ra[e];
            if (!TB) Bs[buf][t >> 4][8 * (t & 15) + e] = rb[e];
            else Bs[buf][8 * (t >> 7) + e][t & 127] = rb[e];
        }
    };
    const int r = lane & 31, hi = lane >> 5;
    const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
    floatx16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    const int64_t steps = (k + kGK - 1) / kGK;
    if (steps > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();
    for (int64_t st = 0; st < steps; ++st) {
        const int cur = (int)(st & 1);
        if (st + 1 < steps) fetch((st + 1) * kGK);
#pragma unroll
        for (int kk = 0; kk < kGK / 2; ++kk) {
            float a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = As[cur][2 * kk + hi][wm + 32 * i + r];
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = Bs[cur][2 * kk + hi][wn + 32 * j + r];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        // the other buffer was last read in step st - 1, before the previous barrier
        if (st + 1 < steps) stash(cur ^ 1);
        __syncthreads();
    }
    // lane (r, hi) holds D[wm + 32 i + 8 (q / 4) + 4 hi + q % 4][wn + 32 j + r] in acc[i][j][q]
    double sq = 0.0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t gn = n0 + wn + 32 * j + r;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int64_t gm = m0 + wm + 32 * i + 8 * (q >> 2) + 4 * hi + (q & 3);
                if (gm >= m || gn >= n) continue;
                float v = alpha * acc[i][j][q];
                if (beta != 0.0f) v = fmaf(beta, C[gm * ldc + gn], v);
                D[gm * ldd + gn] = v;
                sq += (double)v * v;
            }
        }
    if (sumsq) {
        const double s = block_sum(sq);
        if (t == 0) sumsq[blockIdx.x] = s;
    }
}

// --- losses and lambda ------------------------------------------------------------
__global__ __launch_bounds__(256) void calib_losses_kernel(const double *__restrict__ pE, int nE,
                                                           const double *__restrict__ pA, int nA,
                                                           const double *__restrict__ pW, int nW,
                                                           double inv_mo, double inv_md, double inv_od,
                                                           float *__restrict__ losses,
                                                           float *__restrict__ lambdas, int auto_lambda) {
    double e = 0.0, a = 0.0, w = 0.0;
    for (int i = threadIdx.x; i < nE; i += 256) e += pE[i];
    for (int i = threadIdx.x; i < nA; i += 256) a += pA[i];
    for (int i = threadIdx.x; i < nW; i += 256) w += pW[i];
    const double se = block_sum(e);
    __syncthreads();
    const double sa = block_sum(a);
    __syncthreads();
    const double sw = block_sum(w);
    if (threadIdx.x == 0) {
        const double lo = se * inv_mo, la = sa * inv_md, lw = sw * inv_od;
        losses[0] = (float)lo;
        losses[1] = (float)la;
        losses[2] = (float)lw;
        if (auto_lambda) {  // Eq. 10; a term that is zero at the start gets weight 0
            lambdas[0] = la > 0.0 ? (float)(lo / la) : 0.0f;
            lambdas[1] = lw > 0.0 ? (float)(lo / lw) : 0.0f;
        }
    }
}

// --- per-block outer products -----------------------------------------------------
// out[chunk][j][r][c] = sum over rows i of the chunk of L[i][32 j + r] * G[i][32 j + c],
// G = s1 Gp - lambda s2 (Q - T). Grid (nblk, nchunks); thread t owns row r = t / 8 of
// the 32 x 32 result and columns 4 (t % 8) .. +3.
__global__ __launch_bounds__(256) void calib_outer_kernel(const float *__restrict__ Lm, const float *__restrict__ Gp,
                                                          const float *__restrict__ Q, const float *__restrict__ T,
                                                          int64_t rows, int64_t d, int64_t chunk_rows, float s1,
                                                          const float *__restrict__ lam, float s2,
                                                          float *__restrict__ out) {
    __shared__ float Ls[64][33];
    __shared__ float Gs[64][33];
    const int t = threadIdx.x;
    const int64_t j = blockIdx.x, nblk = d / 32, chunk = blockIdx.y;
    const float ls2 = lam[0] * s2;
    const int r = t >> 3, c4 = (t & 7) * 4;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t i_begin = chunk * chunk_rows;
    const int64_t i_end = i_begin + chunk_rows < rows ? i_begin + chunk_rows : rows;
    for (int64_t i0 = i_begin; i0 < i_end; i0 += 64) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = t * 8 + e;  // 0..2047 = 64 rows x 32 channels
            const int ii = idx >> 5, cc = idx & 31;
            const int64_t gi = i0 + ii;
            float lv = 0.0f, gv = 0.0f;
            if (gi < i_end) {
                const int64_t off = gi * d + j * 32 + cc;
                lv = Lm[off];
                gv = s1 * Gp[off] - ls2 * (Q[off] - T[off]);
            }
            Ls[ii][cc] = lv;
            Gs[ii][cc] = gv;
        }
        __syncthreads();
#pragma unroll 8
        for (int ii = 0; ii < 64; ++ii) {
            const float l = Ls[ii][r];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = fmaf(l, Gs[ii][c4 + q], acc[q]);
        }
        __syncthreads();
    }
    float *o = out + (chunk * nblk + j) * 1024 + r * 32 + c4;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = acc[q];
}

// --- per-block gradient through Eq. 12 and Eq. 6, then Adam ----------------------
struct AdamArgs {
    float lr, beta1, beta2, eps, bc1, bc2;  // bc = 1 - beta^t
};

__global__ __launch_bounds__(256) void calib_update_kernel(const float *__restrict__ fac, const float *__restrict__ facit,
                                                           const float *__restrict__ dKA, int nchA,
                                                           const float *__restrict__ dPW, int nchW, int64_t nblk,
                                                           float *__restrict__ theta, float *__restrict__ am,
                                                           float *__restrict__ av, AdamArgs ad,
                                                           float *__restrict__ grad_theta) {
    __shared__ float dK[32][33], dP[32][33], KiT[32][33], Tm[32][33];
    __shared__ float G[20], GiT[20];
    __shared__ float red[256];
    __shared__ float dG[20];
    const int t = threadIdx.x;
    const int64_t j = blockIdx.x;
    if (t < 20) {
        G[t] = fac[j * 20 + t];
        GiT[t] = facit[j * 20 + t];
    }
    __syncthreads();
    const int r = t >> 3, c4 = (t & 7) * 4;
    // chunk sums (fixed order) and (K^{-1})^T = (x)_k (G_k^{-1})^T by Eq. 12
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = c4 + q;
        float sa = 0.0f, sw = 0.0f;
        for (int ch = 0; ch < nchA; ++ch) sa += dKA[(ch * nblk + j) * 1024 + r * 32 + c];
        for (int ch = 0; ch < nchW; ++ch) sw += dPW[(ch * nblk + j) * 1024 + r * 32 + c];
        dK[r][c] = sa;
        dP[r][c] = sw;
        float p = 1.0f;
#pragma unroll
        for (int k = 0; k < 5; ++k) p *= GiT[4 * k + 2 * ((r >> (4 - k)) & 1) + ((c >> (4 - k)) & 1)];
        KiT[r][c] = p;
    }
    __syncthreads();
    // Tm = KiT dP^T
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = c4 + q;
        float s = 0.0f;
        for (int u = 0; u < 32; ++u) s = fmaf(KiT[r][u], dP[c][u], s);
        Tm[r][c] = s;
    }
    __syncthreads();
    // dL/dK = A-part - Tm KiT
    float dk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = c4 + q;
        float s = 0.0f;
        for (int u = 0; u < 32; ++u) s = fmaf(Tm[r][u], KiT[u][c], s);
        dk[q] = dK[r][c] - s;
    }
    // dL/dG_k[p][q] = sum over (r, c) with bits (p, q) at position 4 - k of dK[r][c] prod_{i != k} G_i[..]
    float part[20];
#pragma unroll
    for (int e = 0; e < 20; ++e) part[e] = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = c4 + q;
        float f[5], pre[6], suf[6];
#pragma unroll
        for (int k = 0; k < 5; ++k) f[k] = G[4 * k + 2 * ((r >> (4 - k)) & 1) + ((c >> (4 - k)) & 1)];
        pre[0] = 1.0f;
#pragma unroll
        for (int k = 0; k < 5; ++k) pre[k + 1] = pre[k] * f[k];
        suf[5] = 1.0f;
#pragma unroll
        for (int k = 4; k >= 0; --k) suf[k] = suf[k + 1] * f[k];
#pragma unroll
        for (int k = 0; k < 5; ++k) {  // bucket (p, q) of factor k, selected without indexing registers
            const int pq = 2 * ((r >> (4 - k)) & 1) + ((c >> (4 - k)) & 1);
            const float v = dk[q] * (pre[k] * suf[k + 1]);
#pragma unroll
            for (int e = 0; e < 4; ++e) part[4 * k + e] += pq == e ? v : 0.0f;
        }
    }
    for (int e = 0; e < 20; ++e) {
        red[t] = part[e];
        __syncthreads();
        for (int s = 128; s > 0; s >>= 1) {
            if (t < s) red[t] += red[t + s];
            __syncthreads();
        }
        if (t == 0) dG[e] = red[0];
        __syncthreads();
    }
    // Eq. 6 chain rule and Adam, one thread per parameter. Every thread of a
    // factor reads that factor's (a, b, c) before any of them is overwritten:
    // the new values are written after a barrier all threads reach.
    const bool active = t < 15;
    const int64_t pi = j * 15 + t;
    float updated = 0.0f;
    if (active) {
        const int k = t / 3, which = t % 3;
        const float a = theta[j * 15 + 3 * k], b = theta[j * 15 + 3 * k + 1], c = theta[j * 15 + 3 * k + 2];
        const float g00 = dG[4 * k], g01 = dG[4 * k + 1], g10 = dG[4 * k + 2], g11 = dG[4 * k + 3];
        float g;
        if (which == 0) g = g00 + c * g10 + g11 / (a * a);
        else if (which == 1) g = g01 + c * g11;
        else g = a * g10 + b * g11;
        if (grad_theta) grad_theta[pi] = g;
        const float m = ad.beta1 * am[pi] + (1.0f - ad.beta1) * g;
        const float v = ad.beta2 * av[pi] + (1.0f - ad.beta2) * g * g;
        am[pi] = m;
        av[pi] = v;
        const float mhat = m / ad.bc1, vhat = v / ad.bc2;
        updated = theta[pi] - ad.lr * mhat / (sqrtf(vhat) + ad.eps);
    }
    __syncthreads();
    if (active) theta[pi] = updated;
}

}  // namespace kq
namespace {

using kqhost::aligned;
using kqhost::launched;

// Workspace layout (byte offsets, each 256-aligned) for M activation rows,
// width d and o weight rows.
struct CalibLayout {
    int64_t Af, C0, X, Xq, Y, Yq, E, GX, GY, fac, facit, pA, pW, pE, dKA, dPW, total;
    int64_t qdq_wg_A, qdq_wg_W, gemm_wg_E, nchA, nchW;
};

constexpr int64_t kChunkRows = 256;

int64_t qdq_grid(int64_t rows, int64_t d) {
    const int64_t quads = rows * (d / 32);
    int64_t wg = (quads + 63) / 64;
    return wg < 2048 ? (wg < 1 ? 1 : wg) : 2048;
}

CalibLayout calib_layout(int64_t M, int64_t d, int64_t o) {
    CalibLayout L{};
    const int64_t nblk = d / 32;
    L.qdq_wg_A = qdq_grid(M, d);
    L.qdq_wg_W = qdq_grid(o, d);
    L.gemm_wg_E = ((M + kq::kGT - 1) / kq::kGT) * ((o + kq::kGT - 1) / kq::kGT);
    L.nchA = (M + kChunkRows - 1) / kChunkRows;
    L.nchW = (o + kChunkRows - 1) / kChunkRows;
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = off;
        off += (bytes + 255) / 256 * 256;
        return at;
    };
    L.Af = take(M * d * 4);
    L.C0 = take(M * o * 4);
    L.X = take(M * d * 4);
    L.Xq = take(M * d * 4);
    L.Y = take(o * d * 4);
    L.Yq = take(o * d * 4);
    L.E = take(M * o * 4);
    L.GX = take(M * d * 4);
    L.GY = take(o * d * 4);
    L.fac = take(nblk * 20 * 4);
    L.facit = take(nblk * 20 * 4);
    L.pA = take(L.qdq_wg_A * 8);
    L.pW = take(L.qdq_wg_W * 8);
    L.pE = take(L.gemm_wg_E * 8);
    L.dKA = take(L.nchA * nblk * 1024 * 4);
    L.dPW = take(L.nchW * nblk * 1024 * 4);
    L.total = off;
    return L;
}

kq_status calib_shape(int64_t M, int64_t d, int64_t o) {
    if (M <= 0 || o <= 0 || d <= 0 || d % 32 != 0) return KQ_ERR_SHAPE;
    if (M > ((int64_t)1 << 31) / d || o > ((int64_t)1 << 31) / d || M > ((int64_t)1 << 31) / o)
        return KQ_ERR_UNSUPPORTED;  // every matrix of the step below 2^31 elements
    return KQ_OK;
}

template <bool TA, bool TB>
kq_status launch_gemm(int64_t m, int64_t n, int64_t k, float alpha, const float *A, int64_t lda, const float *B,
                      int64_t ldb, float beta, const float *C, int64_t ldc, float *D, int64_t ldd, double *sumsq,
                      hipStream_t s) {
    const int64_t wg = ((m + kq::kGT - 1) / kq::kGT) * ((n + kq::kGT - 1) / kq::kGT);
    if (wg > 0x7FFFFFFF) return KQ_ERR_SHAPE;
    const bool vec = aligned(A, 16) && aligned(B, 16) && lda % 4 == 0 && ldb % 4 == 0;
    if (vec)
        hipLaunchKernelGGL((kq::gemm_f32_kernel<TA, TB, true>), dim3((unsigned)wg), dim3(256), 0, s, m, n, k, alpha, A,
                           lda, B, ldb, beta, C, ldc, D, ldd, sumsq);
    else
        hipLaunchKernelGGL((kq::gemm_f32_kernel<TA, TB, false>), dim3((unsigned)wg), dim3(256), 0, s, m, n, k, alpha,
                           A, lda, B, ldb, beta, C, ldc, D, ldd, sumsq);
    return launched();
}

// The allocation-free step's workspace: a device array of the library, one copy
// per GPU (each device holds it, at its own address, until the process ends).
// Host code never uses its name as an address: the per-device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];

kq_status scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        kqhost::g_last_hip_error = (int)e;
        return KQ_ERR_HIP;
    }
    if (dev < 0 || dev >= 64) return KQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            kqhost::g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return KQ_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KQ_OK;
}

}  // namespace

extern "C" {

kq_status kq_gemm_f32(int transa, int transb, int64_t m, int64_t n, int64_t k, float alpha, const float *A,
                      int64_t lda, const float *B, int64_t ldb, float beta, const float *C, int64_t ldc, float *D,
                      int64_t ldd, kq_stream_t stream) {
    if (m < 0 || n < 0 || k < 0) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({m, n, k, lda, ldb, ldc, ldd})) return KQ_ERR_UNSUPPORTED;
    if (m == 0 || n == 0) return KQ_OK;
    if (!A || !B || !D || (beta != 0.0f && !C)) return KQ_ERR_NULL;
    if (lda < (transa ? m : k) || ldb < (transb ? k : n) || ldd < n || (beta != 0.0f && ldc < n) || lda < 1 ||
        ldb < 1)
        return KQ_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    if (!transa && !transb) return launch_gemm<false, false>(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, nullptr, s);
    if (!transa && transb) return launch_gemm<false, true>(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, nullptr, s);
    if (transa && !transb) return launch_gemm<true, false>(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, nullptr, s);
    return launch_gemm<true, true>(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, nullptr, s);
}

kq_status kq_calib_workspace_bytes(int64_t M, int64_t d, int64_t o, int64_t *bytes) {
    if (!bytes) return KQ_ERR_NULL;
    const kq_status s = calib_shape(M, d, o);
    if (s != KQ_OK) return s;
    *bytes = calib_layout(M, d, o).total;
    return KQ_OK;
}

kq_status kq_calib_init(const uint16_t *A, int64_t M, int64_t d, const float *W, int64_t o, void *workspace,
                        int64_t workspace_bytes, kq_stream_t stream) {
    kq_status st = calib_shape(M, d, o);
    if (st != KQ_OK) return st;
    if (!A || !W || !workspace) return KQ_ERR_NULL;
    if (!aligned(A, 16) || !aligned(W, 16) || !aligned(workspace, 256)) return KQ_ERR_ALIGN;
    const CalibLayout L = calib_layout(M, d, o);
    if (workspace_bytes < L.total) return KQ_ERR_SHAPE;
    char *ws = static_cast<char *>(workspace);
    float *Af = reinterpret_cast<float *>(ws + L.Af);
    hipStream_t s = (hipStream_t)stream;
    int64_t wg = (M * d / 8 + 255) / 256;
    if (wg > 4096) wg = 4096;
    hipLaunchKernelGGL(kq::widen_kernel, dim3((unsigned)wg), dim3(256), 0, s, A, M * d, Af);
    if ((st = launched()) != KQ_OK) return st;
    // A W^T, the full-precision output the loss compares against
    return launch_gemm<false, true>(M, o, d, 1.0f, Af, d, W, d, 0.0f, nullptr, o, reinterpret_cast<float *>(ws + L.C0),
                                    o, nullptr, s);
}

kq_status kq_calib_step(const float *W, int64_t M, int64_t d, int64_t o, float *theta, float *adam_m, float *adam_v,
                        int64_t t, float lr, float beta1, float beta2, float eps, float *lambdas, int auto_lambda,
                        float *losses, float *grad_theta, void *workspace, int64_t workspace_bytes,
                        kq_stream_t stream) {
    kq_status st = calib_shape(M, d, o);
    if (st != KQ_OK) return st;
    if (!W || !theta || !adam_m || !adam_v || !lambdas || !losses || !workspace) return KQ_ERR_NULL;
    if (!aligned(W, 16) || !aligned(workspace, 256)) return KQ_ERR_ALIGN;
    if (t < 1 || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps >= 0.0f) ||
        !(lr >= 0.0f))
        return KQ_ERR_SHAPE;
    const CalibLayout L = calib_layout(M, d, o);
    if (workspace_bytes < L.total) return KQ_ERR_SHAPE;
    const int64_t nblk = d / 32;
    char *ws = static_cast<char *>(workspace);
    auto F = [&](int64_t off) { return reinterpret_cast<float *>(ws + off); };
    auto Dp = [&](int64_t off) { return reinterpret_cast<double *>(ws + off); };
    hipStream_t s = (hipStream_t)stream;

    hipLaunchKernelGGL(kq::calib_factors_kernel, dim3((unsigned)((nblk * 5 + 255) / 256)), dim3(256), 0, s, theta,
                       nblk * 5, F(L.fac), F(L.facit));
    if ((st = launched()) != KQ_OK) return st;
    hipLaunchKernelGGL((kq::calib_qdq_kernel<false>), dim3((unsigned)L.qdq_wg_A), dim3(256), 0, s,
                       static_cast<const void *>(F(L.Af)), M, d, F(L.fac), F(L.X), F(L.Xq), Dp(L.pA));
    if ((st = launched()) != KQ_OK) return st;
    hipLaunchKernelGGL((kq::calib_qdq_kernel<false>), dim3((unsigned)L.qdq_wg_W), dim3(256), 0, s,
                       static_cast<const void *>(W), o, d, F(L.facit), F(L.Y), F(L.Yq), Dp(L.pW));
    if ((st = launched()) != KQ_OK) return st;
    // E = Q(X) Q(Y)^T - A W^T
    if ((st = launch_gemm<false, true>(M, o, d, 1.0f, F(L.Xq), d, F(L.Yq), d, -1.0f, F(L.C0), o, F(L.E), o, Dp(L.pE),
                                       s)) != KQ_OK)
        return st;
    hipLaunchKernelGGL(kq::calib_losses_kernel, dim3(1), dim3(256), 0, s, Dp(L.pE), (int)L.gemm_wg_E, Dp(L.pA),
                       (int)L.qdq_wg_A, Dp(L.pW), (int)L.qdq_wg_W, 1.0 / ((double)M * o), 1.0 / ((double)M * d),
                       1.0 / ((double)o * d), losses, lambdas, auto_lambda);
    if ((st = launched()) != KQ_OK) return st;
    // E Q(Y) (M x d) and E^T Q(X) (o x d)
    if ((st = launch_gemm<false, false>(M, d, o, 1.0f, F(L.E), o, F(L.Yq), d, 0.0f, nullptr, d, F(L.GX), d, nullptr,
                                        s)) != KQ_OK)
        return st;
    if ((st = launch_gemm<true, false>(o, d, M, 1.0f, F(L.E), o, F(L.Xq), d, 0.0f, nullptr, d, F(L.GY), d, nullptr,
                                       s)) != KQ_OK)
        return st;
    const float sO = (float)(2.0 / ((double)M * o));
    hipLaunchKernelGGL(kq::calib_outer_kernel, dim3((unsigned)nblk, (unsigned)L.nchA), dim3(256), 0, s, F(L.Af),
                       F(L.GX), F(L.Xq), F(L.X), M, d, kChunkRows, sO, lambdas, (float)(2.0 / ((double)M * d)),
                       F(L.dKA));
    if ((st = launched()) != KQ_OK) return st;
    hipLaunchKernelGGL(kq::calib_outer_kernel, dim3((unsigned)nblk, (unsigned)L.nchW), dim3(256), 0, s, W, F(L.GY),
                       F(L.Yq), F(L.Y), o, d, kChunkRows, sO, lambdas + 1, (float)(2.0 / ((double)o * d)), F(L.dPW));
    if ((st = launched()) != KQ_OK) return st;
    kq::AdamArgs ad;
    ad.lr = lr;
    ad.beta1 = beta1;
    ad.beta2 = beta2;
    ad.eps = eps;
    ad.bc1 = (float)(1.0 - pow((double)beta1, (double)t));
    ad.bc2 = (float)(1.0 - pow((double)beta2, (double)t));
    hipLaunchKernelGGL(kq::calib_update_kernel, dim3((unsigned)nblk), dim3(256), 0, s, F(L.fac), F(L.facit), F(L.dKA),
                       (int)L.nchA, F(L.dPW), (int)L.nchW, nblk, theta, adam_m, adam_v, ad, grad_theta);
    return launched();
}

kq_status kq_calib_step_noalloc(const uint16_t *A, const float *W, int64_t M, int64_t d, int64_t o, float *theta,
                                float *adam_m, float *adam_v, int64_t t, float lr, float beta1, float beta2, float eps,
                                float *lambdas, int auto_lambda, float *losses, float *grad_theta,
                                kq_stream_t stream) {
    kq_status st = calib_shape(M, d, o);
    if (st != KQ_OK) return st;
    if (calib_layout(M, d, o).total > kScratchBytes) return KQ_ERR_UNSUPPORTED;
    if (!A || !W || !theta || !adam_m || !adam_v || !lambdas || !losses) return KQ_ERR_NULL;
    if (!aligned(A, 16) || !aligned(W, 16)) return KQ_ERR_ALIGN;
    if (t < 1 || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps >= 0.0f) ||
        !(lr >= 0.0f))
        return KQ_ERR_SHAPE;
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != KQ_OK) return st;
    // every part of the workspace the step reads is written first in this call
    // (A in fp32 and A W^T by the init half, the rest by the step's own kernels),
    // so nothing of an earlier call's contents is used and nothing needs clearing
    if ((st = kq_calib_init(A, M, d, W, o, ws, kScratchBytes, stream)) != KQ_OK) return st;
    return kq_calib_step(W, M, d, o, theta, adam_m, adam_v, t, lr, beta1, beta2, eps, lambdas, auto_lambda, losses,
                         grad_theta, ws, kScratchBytes, stream);
}

}  // extern "C"
