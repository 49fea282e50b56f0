// MXFP4 matrix products on gfx950 scaled FP4 matrix instructions: the W4A4
// GEMM of Eq. 2 (KroQuant, arXiv 2607.21446v1), optionally with the low-rank
// term of Sec. 3.4 Eq. 11 added in its epilogue, and that term's projection of
// the 16-bit activations onto Q(R).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"
#include "kq_device.hpp"
#include "kq_host.hpp"

namespace kq {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Low-rank branch helpers (Eq. 11's A T R^T L^T with MXFP4 L and R)
// ---------------------------------------------------------------------------

// 8 E2M1 codes (element 2i in the low nibble of byte i) with one E8M0 scale,
// decoded exactly to bf16: a level has at most two significant bits and the
// scale is a power of two, so the fp32 product is exact and its top 16 bits
// are the bf16 value.
__device__ __forceinline__ bf16x8_t decode_fp4x8_bf16(uint32_t c8, uint32_t sbyte) {
    const float scale = ldexpf(1.0f, (int)sbyte - 127);
    uint16_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t code = (c8 >> (4 * i)) & 15u, n = code & 7u;
        const float lvl = n < 2 ? 0.5f * (float)n : ldexpf(1.0f + 0.5f * (float)(n & 1), (int)(n >> 1) - 1);
        const float v = (code & 8u) ? -(lvl * scale) : lvl * scale;
        h[i] = (uint16_t)(__float_as_uint(v) >> 16);
    }
    bf16x8_t out;
    __builtin_memcpy(&out, h, 16);
    return out;
}

// fp32 x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in fp32).
__device__ __forceinline__ void split_bf16x8(const float x[8], bf16x8_t &hi, bf16x8_t &lo) {
    uint16_t h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = bf16_rne_bits(x[i]);
        l[i] = bf16_rne_bits(x[i] - __uint_as_float((uint32_t)h[i] << 16));
    }
    __builtin_memcpy(&hi, h, 16);
    __builtin_memcpy(&lo, l, 16);
}

// Z = X Q(R)^T: X bf16 [m][ldx] (the branch's 16-bit activations), R MXFP4
// [r][d] (codes [r][d/2], scales [r][d/32]), Z fp32 [m][r]. A workgroup
// computes 64 rows x 128 columns of Z (each wave 32 x 64 = 2 x 4 MFMA tiles),
// walking d in steps of 32 with v_mfma_f32_16x16x32_bf16: lane l supplies row
// l % 16 and k = 8 (l / 16) .. +7 of X (one 16-byte load) and of the decoded R
// row; it receives rows 4 (l / 16) + t, column l % 16.
struct ProjGeom {
    int64_t m, d, ldx, r, tiles_r;
};

__global__ __launch_bounds__(kThreads) void lowrank_project_kernel(const uint16_t *__restrict__ X, ProjGeom g,
                                                                   const uint8_t *__restrict__ cr,
                                                                   const uint8_t *__restrict__ sr,
                                                                   float *__restrict__ Z) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t tm = blockIdx.x / g.tiles_r, tr = blockIdx.x % g.tiles_r;
    const int64_t row0 = tm * 64 + (wave >> 1) * 32, col0 = tr * 128 + (wave & 1) * 64;
    const int r = lane & 15, grp = lane >> 4;
    floatx4_t acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    for (int64_t k0 = 0; k0 < g.d; k0 += 32) {
        const int64_t k = k0 + 8 * grp;
        bf16x8_t xa[2], rb[4];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int64_t row = row0 + a * 16 + r;
            uint4 q = make_uint4(0, 0, 0, 0);
            if (row < g.m) q = load_stream(reinterpret_cast<const uint4 *>(X + row * g.ldx + k), true);
            xa[a] = as_bf16x8(q);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t n = col0 + b * 16 + r;
            uint32_t c8 = 0, s = 127;
            if (n < g.r) {
                c8 = *reinterpret_cast<const uint32_t *>(cr + n * (g.d / 2) + k / 2);
                s = sr[n * (g.d / 32) + k0 / 32];
            }
            rb[b] = decode_fp4x8_bf16(c8, s);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[a], rb[b], acc[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t col = col0 + b * 16 + r;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int64_t row = row0 + a * 16 + grp * 4 + t;
                if (row < g.m && col < g.r) Z[row * g.r + col] = acc[a][b][t];
            }
        }
}

// ---------------------------------------------------------------------------
// W4A4 GEMM on MXFP4 operands: O[i][j] = sum_k deq(A)[i][k] deq(W)[j][k]
// (Eq. 2's Q(A T) Q(W T^{-T})^T), fp32 accumulation on
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in E2M1. Lane l of a
// wave supplies row l % 16 and the 32 consecutive k of group l / 16 (16 code
// bytes) with that group's E8M0 byte as its scale, which is exactly the MX
// layout of the codes/scales arrays; it receives O rows 4 (l / 16) + t, column
// l % 16.
//
// A workgroup of 4 waves computes a 128 x 128 tile, each wave 64 x 64 (4 x 4
// MFMA tiles), walking k in steps of 128 (64 code bytes and 4 scale bytes per
// row). The A and W tiles of a step are staged through LDS, double-buffered:
// every thread fetches its share of the next step's codes and scales into
// registers before the MFMAs of the current step and stores them to the other
// buffer after, one barrier per step. LDS rows are padded to 80 bytes so the 16
// rows an operand read touches fall in distinct banks. Rows and columns past m
// or n, and k groups past k, read zero codes (scale 2^0) and are not stored;
// k must be a multiple of 32.
// ---------------------------------------------------------------------------
typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct GemmGeom {
    int64_t m, n, k, ldo, tiles_n;
    int64_t r;  // rank of the low-rank term (0: none)
};

constexpr int kGemmTile = 128;

// Staged rows of one operand tile: KS k blocks of 128 (64 code bytes each) per
// stage, padded by 16 bytes so the 16 rows an operand read touches fall in
// distinct banks.
template <int KS>
struct GemmStage {
    static constexpr int kRow = KS * 64 + 16;
    static constexpr int kLoads = KS * 2;  // 16-byte code loads per thread per operand
};

// This thread's share of one operand tile for the stage starting at code byte
// kb0: rows (t >> 2) + 64 h, 16 bytes at column 16 (t & 3) + 64 c of each
// 128-k block c, and, for threads below 128, row t's KS * 4 scale bytes.
template <int KS>
struct TileRegs {
    uint4 code[KS][2];
    uint32_t scl[KS];
};

template <int KS>
__device__ __forceinline__ void fetch_tile(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                           int64_t row_base, int64_t nrows, int64_t kbytes, int64_t kblocks,
                                           int64_t kb0, TileRegs<KS> &R) {
    const int t = threadIdx.x;
    const int r0 = t >> 2, c16 = (t & 3) * 16;
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t row = row_base + r0 + 64 * h, kb = kb0 + 64 * c + c16;
            R.code[c][h] = make_uint4(0, 0, 0, 0);
            if (row < nrows && kb < kbytes)
                R.code[c][h] = *reinterpret_cast<const uint4 *>(codes + row * kbytes + kb);
        }
    if (t < kGemmTile) {
        const int64_t row = row_base + t;
#pragma unroll
        for (int c = 0; c < KS; ++c) {
            const int64_t g0 = kb0 / 16 + 4 * c;  // first 32-k group of this 128-k block
            uint32_t v = 0x7F7F7F7Fu;             // 2^0 for rows and k groups past the ends
            if (row < nrows) {
                if ((kblocks & 3) == 0 && (reinterpret_cast<uintptr_t>(scales) & 3) == 0 && g0 + 4 <= kblocks) {
                    v = *reinterpret_cast<const uint32_t *>(scales + row * kblocks + g0);
                } else {
                    v = 0;
#pragma unroll
                    for (int gi = 0; gi < 4; ++gi)
                        v |= (g0 + gi < kblocks ? (uint32_t)scales[row * kblocks + g0 + gi] : 0x7Fu) << (8 * gi);
                }
            }
            R.scl[c] = v;
        }
    }
}

template <int KS>
__device__ __forceinline__ void stash_tile(uint8_t *codes_lds, uint32_t *scales_lds, const TileRegs<KS> &R) {
    const int t = threadIdx.x;
    const int r0 = t >> 2, c16 = (t & 3) * 16;
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *reinterpret_cast<uint4 *>(codes_lds + (r0 + 64 * h) * GemmStage<KS>::kRow + 64 * c + c16) = R.code[c][h];
    if (t < kGemmTile)
#pragma unroll
        for (int c = 0; c < KS; ++c) scales_lds[c * kGemmTile + t] = R.scl[c];
}

template <int KS, bool LR>
__global__ __launch_bounds__(kThreads) void mxfp4_gemm_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const uint8_t *__restrict__ cw,
    const uint8_t *__restrict__ sw, GemmGeom g, const float *__restrict__ Z, const uint8_t *__restrict__ cl,
    const uint8_t *__restrict__ sl, float *__restrict__ O) {
    constexpr int ROW = GemmStage<KS>::kRow;
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kGemmTile * ROW];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[2][kGemmTile * ROW];
    __shared__ uint32_t as_lds[2][KS * kGemmTile], bs_lds[2][KS * kGemmTile];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t tm = blockIdx.x / g.tiles_n, tn = blockIdx.x % g.tiles_n;
    const int64_t m0 = tm * kGemmTile, n0 = tn * kGemmTile;
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;  // this wave's 64 x 64 within the tile
    const int r = lane & 15, grp = lane >> 4;
    const int64_t kbytes = g.k / 2, kblocks = g.k / 32;
    const int64_t stages = (g.k + 128 * KS - 1) / (128 * KS);

    floatx4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    TileRegs<KS> ra, rb;
    fetch_tile<KS>(ca, sa, m0, g.m, kbytes, kblocks, 0, ra);
    fetch_tile<KS>(cw, sw, n0, g.n, kbytes, kblocks, 0, rb);
    stash_tile<KS>(a_lds[0], as_lds[0], ra);
    stash_tile<KS>(b_lds[0], bs_lds[0], rb);
    __syncthreads();
    for (int64_t s = 0; s < stages; ++s) {
        const int cur = (int)(s & 1);
        if (s + 1 < stages) {
            fetch_tile<KS>(ca, sa, m0, g.m, kbytes, kblocks, (s + 1) * 64 * KS, ra);
            fetch_tile<KS>(cw, sw, n0, g.n, kbytes, kblocks, (s + 1) * 64 * KS, rb);
        }
#pragma unroll
        for (int c = 0; c < KS; ++c) {
            i32x8_t bv[4];
            int bsc[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint4 q =
                    *reinterpret_cast<const uint4 *>(b_lds[cur] + (wc + b * 16 + r) * ROW + 64 * c + grp * 16);
                bv[b] = i32x8_t{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
                bsc[b] = (int)((bs_lds[cur][c * kGemmTile + wc + b * 16 + r] >> (8 * grp)) & 0xFFu);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const uint4 q =
                    *reinterpret_cast<const uint4 *>(a_lds[cur] + (wr + a * 16 + r) * ROW + 64 * c + grp * 16);
                const i32x8_t av = i32x8_t{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
                const int asc = (int)((as_lds[cur][c * kGemmTile + wr + a * 16 + r] >> (8 * grp)) & 0xFFu);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv[b], acc[a][b], 4, 4, 0, asc,
                                                                                 0, bsc[b]);
            }
        }
        if (s + 1 < stages) {
            stash_tile<KS>(a_lds[cur ^ 1], as_lds[cur ^ 1], ra);
            stash_tile<KS>(b_lds[cur ^ 1], bs_lds[cur ^ 1], rb);
        }
        __syncthreads();
    }
    if (LR) {
        // Low-rank term Z Q(L)^T into the same accumulators: Z fp32 [m][r] split
        // as hi + lo bf16 (exact to 2^-16 relative), Q(L) decoded to bf16 (exact),
        // two v_mfma_f32_16x16x32_bf16 per tile pair and 32 k of r.
        for (int64_t kk = 0; kk < g.r; kk += 32) {
            const int64_t k = kk + 8 * grp;
            bf16x8_t lb[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int64_t nrow = n0 + wc + b * 16 + r;
                uint32_t c8 = 0, s = 127;
                if (nrow < g.n) {
                    c8 = *reinterpret_cast<const uint32_t *>(cl + nrow * (g.r / 2) + k / 2);
                    s = sl[nrow * (g.r / 32) + kk / 32];
                }
                lb[b] = decode_fp4x8_bf16(c8, s);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int64_t row = m0 + wr + a * 16 + r;
                float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (row < g.m) {
                    const float4 *p = reinterpret_cast<const float4 *>(Z + row * g.r + k);
                    const float4 u = p[0], v = p[1];
                    z[0] = u.x; z[1] = u.y; z[2] = u.z; z[3] = u.w; z[4] = v.x; z[5] = v.y; z[6] = v.z; z[7] = v.w;
                }
                bf16x8_t zh, zl;
                split_bf16x8(z, zh, zl);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zh, lb[b], acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zl, lb[b], acc[a][b], 0, 0, 0);
                }
            }
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t col = n0 + wc + b * 16 + r;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int64_t row = m0 + wr + a * 16 + grp * 4 + t;
                if (row < g.m && col < g.n) O[row * g.ldo + col] = acc[a][b][t];
            }
        }
}

}  // namespace kq

namespace {
using kqhost::aligned;
using kqhost::launched;
}  // namespace

extern "C" {

kq_status kq_mxfp4_gemm(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                        const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, float *O, int64_t ldo,
                        kq_stream_t stream) {
    if (m < 0 || n < 0 || k < 0 || k % 32 != 0 || ldo < n) return KQ_ERR_SHAPE;
    if (m == 0 || n == 0) return KQ_OK;
    if (!codes_a || !scales_a || !codes_w || !scales_w || !O) return KQ_ERR_NULL;
    if (!aligned(codes_a, 16) || !aligned(codes_w, 16) || (k / 2) % 16 != 0) return KQ_ERR_ALIGN;
    const int64_t tiles_m = (m + kq::kGemmTile - 1) / kq::kGemmTile, tiles_n = (n + kq::kGemmTile - 1) / kq::kGemmTile;
    if (tiles_m * tiles_n > 0x7FFFFFFF || m > INT64_MAX / 4 / (ldo > 0 ? ldo : 1)) return KQ_ERR_SHAPE;
    kq::GemmGeom g{m, n, k, ldo, tiles_n, 0};
    hipLaunchKernelGGL((kq::mxfp4_gemm_kernel<2, false>), dim3((unsigned)(tiles_m * tiles_n)), dim3(kq::kThreads), 0,
                       (hipStream_t)stream, codes_a, scales_a, codes_w, scales_w, g, nullptr, nullptr, nullptr, O);
    return launched();
}

kq_status kq_mxfp4_gemm_lowrank(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                                const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, const float *Z,
                                const uint8_t *codes_l, const uint8_t *scales_l, int64_t r, float *O, int64_t ldo,
                                kq_stream_t stream) {
    if (m < 0 || n < 0 || k < 0 || k % 32 != 0 || ldo < n || r <= 0 || r % 32 != 0) return KQ_ERR_SHAPE;
    if (m == 0 || n == 0) return KQ_OK;
    if (!codes_a || !scales_a || !codes_w || !scales_w || !O || !Z || !codes_l || !scales_l) return KQ_ERR_NULL;
    if (!aligned(codes_a, 16) || !aligned(codes_w, 16) || (k / 2) % 16 != 0 || !aligned(Z, 16) ||
        !aligned(codes_l, 16))
        return KQ_ERR_ALIGN;
    const int64_t tiles_m = (m + kq::kGemmTile - 1) / kq::kGemmTile, tiles_n = (n + kq::kGemmTile - 1) / kq::kGemmTile;
    if (tiles_m * tiles_n > 0x7FFFFFFF || m > INT64_MAX / 4 / (ldo > 0 ? ldo : 1) || m > INT64_MAX / 4 / r)
        return KQ_ERR_SHAPE;
    kq::GemmGeom g{m, n, k, ldo, tiles_n, r};
    hipLaunchKernelGGL((kq::mxfp4_gemm_kernel<2, true>), dim3((unsigned)(tiles_m * tiles_n)), dim3(kq::kThreads), 0,
                       (hipStream_t)stream, codes_a, scales_a, codes_w, scales_w, g, Z, codes_l, scales_l, O);
    return launched();
}

kq_status kq_lowrank_project(const uint16_t *X16, int64_t m, int64_t d, int64_t ldx, const uint8_t *codes_r,
                             const uint8_t *scales_r, int64_t r, float *Z, kq_stream_t stream) {
    if (m < 0 || d < 0 || d % 32 != 0 || ldx < d || r <= 0 || r % 32 != 0) return KQ_ERR_SHAPE;
    if (m == 0 || d == 0) return KQ_OK;
    if (!X16 || !codes_r || !scales_r || !Z) return KQ_ERR_NULL;
    if (!aligned(X16, 16) || ldx % 8 != 0 || !aligned(codes_r, 16) || !aligned(Z, 16)) return KQ_ERR_ALIGN;
    const int64_t tiles_m = (m + 63) / 64, tiles_r = (r + 127) / 128;
    if (tiles_m * tiles_r > 0x7FFFFFFF || m > INT64_MAX / 4 / (ldx > r ? ldx : r)) return KQ_ERR_SHAPE;
    kq::ProjGeom g{m, d, ldx, r, tiles_r};
    hipLaunchKernelGGL(kq::lowrank_project_kernel, dim3((unsigned)(tiles_m * tiles_r)), dim3(kq::kThreads), 0,
                       (hipStream_t)stream, X16, g, codes_r, scales_r, Z);
    return launched();
}

}  // extern "C"
