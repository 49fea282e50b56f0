// The W4A4 product of Eq. 2 (KroQuant, arXiv 2607.21446v1),
//   O = deq(Q(A T)) deq(Q(W T^{-T}))^T,
// on gfx950 scaled FP4 matrix instructions with wide output tiles, in two
// forms: from an MXFP4 activation (codes and scales, as the quantizer writes
// them), and straight from the bf16 activation with the Kronecker transform of
// Sec. 3.2 (Eq. 5, Sec. 3.5.1 Eq. 12) and the MXFP4 quantizer in the
// product's prologue, so the activation's codes never leave the chip.
//
// Tiling. A workgroup (8 waves) computes 128 rows x 512 columns of O; wave w
// owns rows 64 (w >> 2) .. +63 and columns 128 (w & 3) .. +127 as 2 x 4 tiles of
// 32 x 32 (v_mfma_scale_f32_32x32x64_f8f6f4, both operands E2M1 with E8M0
// scales; on gfx950 it issues FP4 at twice the rate of the 16 x 16 x 128 form).
// Operands are swapped (the W fragment first), so lane l supplies row l % 32
// of each fragment and MX block 2 j + l / 32 of k step j, and receives O row
// l % 32, columns 8 q + 4 (l / 32) + 0..3 of the W fragment in accumulator
// registers 4 q .. 4 q + 3 -- the instruction, operand order and k order of
// the packed-scale GEMM, whose results this kernel reproduces bit for bit. k
// advances 128 per stage (two k steps), one MX group of four E8M0 bytes per
// row, double-buffered in LDS with one barrier per stage; the next stage's
// activation loads are in flight while the current stage's matrix instructions
// run. Staged rows are 80 bytes (64 code bytes + 16 pad), so the 16 rows of one
// pass of a fragment read fall in distinct banks.
//
// Why the wide tile: with the transform in the prologue, every workgroup that
// shares an activation row block repeats its transform, n / 512 times here
// (6 at n = 3072), against n / 128 with 128-wide tiles. The transform's VALU
// work per stage (4 chunks of 8 elements per lane) is independent of the tile
// width, while the matrix work per stage grows with it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"
#include "kq_device.hpp"
#include "kq_host.hpp"

namespace kq {

namespace w4 {

constexpr int kThreads = 512;
constexpr int kM = 128, kN = 512;
constexpr int kRow = 80;  // staged bytes per row: 64 code bytes (128 k) + 16 pad

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

struct Geom {
    int64_t m, n, k, lda, ldo;
    int64_t tiles_n;
    int kblocks;  // k / 32
    int stages;   // ceil(k / 128)
};

// Which activation operand the workgroup reads.
enum Prologue { kCodes = 0, kBf16Kron = 1 };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// The stage's share of W held in registers: rows (t >> 2) + 128 h of the tile,
// 16 code bytes at (t & 3) * 16, and row t's four scale bytes.
struct WRegs {
    uint4 code[4];
    uint32_t scl;
};

// The stage's share of the activation: codes (row t >> 2, 16 bytes at
// (t & 3) * 16; row t's scale dword for t < 128), or bf16 (rows (t >> 4) + 32 i,
// 8 channels of block (t >> 2) & 3 at sub-block t & 3).
struct ARegs {
    uint4 q[4];
    uint32_t scl;
};

// Four E8M0 bytes of one row's 128-k group (k groups past the end read 2^0).
__device__ __forceinline__ uint32_t load_scales4(const uint8_t *__restrict__ s, int64_t row, const Geom &g,
                                                 int stage, bool valid) {
    const int g0 = stage * 4;
    if (!valid || g0 >= g.kblocks) return 0x7F7F7F7Fu;
    if ((g.kblocks & 3) == 0) return *reinterpret_cast<const uint32_t *>(s + row * g.kblocks + g0);
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) v |= (g0 + i < g.kblocks ? (uint32_t)s[row * g.kblocks + g0 + i] : 0x7Fu) << (8 * i);
    return v;
}

__device__ __forceinline__ void fetch_w(const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw,
                                        const Geom &g, int64_t n0, int stage, WRegs &R) {
    const int t = threadIdx.x;
    const int64_t kbytes = g.k / 2;
    const int64_t rows = g.n - n0 < kN ? g.n - n0 : kN;
    const auto rs = rsrc(cw + n0 * kbytes, (uint32_t)(rows * kbytes));  // rows past n read zeros
    const int64_t kb = (int64_t)stage * 64 + (t & 3) * 16;
    const bool kin = kb < kbytes;  // a 16-byte piece is entirely in or out (k % 32 == 0)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int64_t row = (t >> 2) + 128 * h;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(row * kbytes + kb), 0, 0);
        R.code[h] = kin ? make_uint4(v[0], v[1], v[2], v[3]) : make_uint4(0, 0, 0, 0);
    }
    R.scl = load_scales4(sw, n0 + t, g, stage, n0 + t < g.n);
}

__device__ __forceinline__ void stash_w(uint8_t *b_lds, uint32_t *bs_lds, const WRegs &R) {
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 4; ++h)
        *reinterpret_cast<uint4 *>(b_lds + ((t >> 2) + 128 * h) * kRow + (t & 3) * 16) = R.code[h];
    bs_lds[t] = R.scl;
}

template <int PRO>
__device__ __forceinline__ void fetch_a(const void *__restrict__ A, const uint8_t *__restrict__ sa, const Geom &g,
                                        int64_t m0, int stage, ARegs &R) {
    const int t = threadIdx.x;
    const int64_t rows = g.m - m0 < kM ? g.m - m0 : kM;
    if (PRO == kCodes) {
        const uint8_t *ca = static_cast<const uint8_t *>(A);
        const int64_t kbytes = g.k / 2;
        const auto rs = rsrc(ca + m0 * kbytes, (uint32_t)(rows * kbytes));
        const int64_t kb = (int64_t)stage * 64 + (t & 3) * 16;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((t >> 2) * kbytes + kb), 0, 0);
        R.q[0] = kb < kbytes ? make_uint4(v[0], v[1], v[2], v[3]) : make_uint4(0, 0, 0, 0);
        if (t < kM) R.scl = load_scales4(sa, m0 + t, g, stage, m0 + t < g.m);
    } else {
        // bf16 rows past m read zeros through the record count; channels of
        // blocks past k are read from the row's tail or the next row and their
        // codes are discarded in the prologue
        const uint16_t *a = static_cast<const uint16_t *>(A);
        const auto rs = rsrc(a + m0 * g.lda, (uint32_t)(rows * g.lda * 2));
        const int64_t col = (int64_t)stage * 128 + ((t >> 2) & 3) * 32 + (t & 3) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = (t >> 4) + 32 * i;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((row * g.lda + col) * 2), 0, 2);
            R.q[i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }
}

// Per-lane coefficients of the stage's four blocks (16 lanes: block b = l >> 2,
// sub-block l & 3), written by wave 0's first 16 lanes; layout and arithmetic
// as the fused quantizer's (shear form when all four blocks admit it, else
// the general 2x2 stages for all four).
struct CoefStage {
    float c[16][17];
    int shear;
};

__device__ __forceinline__ void derive_coefs(const float *__restrict__ factors, const Geom &g, int stage,
                                             CoefStage &C) {
    const int l = threadIdx.x;  // called by threads 0..15 only
    const int blk = stage * 4 + (l >> 2), sub = l & 3;
    const bool active = blk < g.kblocks;
    const bool b4 = (sub >> 1) & 1, b3 = sub & 1;
    float *dst = C.c[l];
    float f[20];
    if (active) {
        load_factors20(factors + (int64_t)blk * 20, f);
    } else {
#pragma unroll
        for (int i = 0; i < 20; ++i) f[i] = 0.f;
    }
    // shear-form coefficients, written as they are computed
    const float lim = 0x1.0p20f;
    bool ok = true;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const float p = f[4 * k + 1] * __builtin_amdgcn_rcpf(f[4 * k + 3]);
        const float q = f[4 * k + 2] * __builtin_amdgcn_rcpf(f[4 * k]);
        ok = (int)ok & (int)(fabsf(p) <= lim) & (int)(fabsf(q) <= lim);  // false for inf and NaN
        if (k == 0) dst[0] = b4 ? p : q;
        else if (k == 1) dst[1] = b3 ? p : q;
        else {
            dst[2 * k - 2] = p;
            dst[2 * k - 1] = q;
        }
    }
    const float d12 = (b4 ? f[3] : f[0]) * (b3 ? f[7] : f[4]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        dst[8 + i] = ((d12 * f[8 + 3 * ((i >> 2) & 1)]) * f[12 + 3 * ((i >> 1) & 1)]) * f[16 + 3 * (i & 1)];
    const bool all = __builtin_amdgcn_ballot_w64(active && !ok) == 0;  // over the 16 deriving lanes
    if (!all) {  // some block of the stage has no shear form: general stages for all four
        dst[0] = b4 ? f[3] : f[0];
        dst[1] = b4 ? f[1] : f[2];
        dst[2] = b3 ? f[7] : f[4];
        dst[3] = b3 ? f[5] : f[6];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dst[4 + i] = f[8 + i];
            dst[8 + i] = f[12 + i];
            dst[12 + i] = f[16 + i];
        }
    }
    if (l == 0) C.shear = all;
}

template <bool SHEAR>
__device__ __forceinline__ void apply_stage(float y[8], const float c[16]) {
    if (SHEAR) {
        fmac_partner_xor2(y, c[0]);
        fmac_partner_xor1(y, c[1]);
        shear_stage<4>(y, c[2], c[3]);
        shear_stage<2>(y, c[4], c[5]);
        shear_stage<1>(y, c[6], c[7]);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = y[i] * c[8 + i];
    } else {
        KronLane L;
        L.s1 = c[0]; L.o1 = c[1]; L.s2 = c[2]; L.o2 = c[3];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            L.g3[i] = c[4 + i];
            L.g4[i] = c[8 + i];
            L.g5[i] = c[12 + i];
        }
        kron_apply8(y, L);
    }
}

// Activation operand of one stage into LDS: codes as loaded, or the bf16
// chunks transformed and quantized (quad layout: four lanes per row and
// block), codes of blocks past k zeroed.
template <int PRO>
__device__ __forceinline__ void stash_a(uint8_t *a_lds, uint32_t *as_lds, const ARegs &R, const CoefStage &C,
                                        const Geom &g, int stage) {
    const int t = threadIdx.x;
    if (PRO == kCodes) {
        *reinterpret_cast<uint4 *>(a_lds + (t >> 2) * kRow + (t & 3) * 16) = R.q[0];
        if (t < kM) as_lds[t] = R.scl;
        return;
    }
    const int b = (t >> 2) & 3, sub = t & 3;
    float c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = C.c[b * 4 + sub][i];
    const bool kin = stage * 4 + b < g.kblocks;
    const bool shear = __builtin_amdgcn_readfirstlane(C.shear);
    uint8_t *as8 = reinterpret_cast<uint8_t *>(as_lds);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (t >> 4) + 32 * i;
        float y[8];
        widen8(R.q[i], y);
        if (shear) apply_stage<true>(y, c);
        else apply_stage<false>(y, c);
        uint32_t sbyte;
        uint32_t packed = quantize_quad_f32(y, sbyte);
        if (!kin) {
            packed = 0u;
            sbyte = 0x7Fu;
        }
        *reinterpret_cast<uint32_t *>(a_lds + row * kRow + b * 16 + sub * 4) = packed;
        if (sub == 0) as8[row * 4 + b] = (uint8_t)sbyte;
    }
}

template <int PRO>
__global__ __launch_bounds__(kThreads) void w4a4_kernel(const void *__restrict__ A, const uint8_t *__restrict__ sa,
                                                        const float *__restrict__ factors,
                                                        const uint8_t *__restrict__ cw,
                                                        const uint8_t *__restrict__ sw, Geom g,
                                                        float *__restrict__ O) {
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kM * kRow];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[2][kN * kRow];
    __shared__ uint32_t as_lds[2][kM], bs_lds[2][kN];
    __shared__ CoefStage coef[PRO == kBf16Kron ? 2 : 1];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t tm = blockIdx.x / g.tiles_n, tn = blockIdx.x % g.tiles_n;
    const int64_t m0 = tm * kM, n0 = tn * kN;
    const int wm = (wave >> 2) * 64, wn = (wave & 3) * 128;
    const int r = lane & 31, hi = lane >> 5;

    floatx16_t acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

    ARegs ra;
    WRegs rw;
    // stage 0 operands; coefficients of stages 0 and 1
    fetch_a<PRO>(A, sa, g, m0, 0, ra);
    fetch_w(cw, sw, g, n0, 0, rw);
    if (PRO == kBf16Kron) {
        if (t < 16) derive_coefs(factors, g, 0, coef[0]);
        __syncthreads();
        if (t < 16 && g.stages > 1) derive_coefs(factors, g, 1, coef[1]);
    }
    stash_a<PRO>(a_lds[0], as_lds[0], ra, coef[0], g, 0);
    stash_w(b_lds[0], bs_lds[0], rw);
    __syncthreads();

    // Per stage: the activation's next loads go out first (they come from HBM),
    // then this stage's matrix instructions, then the next W loads (mostly L2
    // hits, their latency covered by the coefficient derivation and the
    // transform), so the W registers are not live across the matrix loop.
    for (int s = 0; s < g.stages; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < g.stages;
        if (more) fetch_a<PRO>(A, sa, g, m0, s + 1, ra);

        // k step j of the stage (64 k): lane (r, hi) supplies row r of each
        // fragment and MX block 2 j + hi (16 code bytes); its scale dword is
        // rearranged so that byte j holds that block's scale (the instruction's
        // byte select is uniform across lanes)
        auto lane_scales = [&](uint32_t d) {
            return hi ? ((d >> 8) & 0xFFu) | ((d >> 16) & 0xFF00u) : (d & 0xFFu) | ((d >> 8) & 0xFF00u);
        };
        int asc[2], bsc[4];
#pragma unroll
        for (int a = 0; a < 2; ++a) asc[a] = (int)lane_scales(as_lds[cur][wm + 32 * a + r]);
#pragma unroll
        for (int b = 0; b < 4; ++b) bsc[b] = (int)lane_scales(bs_lds[cur][wn + 32 * b + r]);
        auto frag = [&](const uint8_t *base, int row, int j) {
            const uint4 q = *reinterpret_cast<const uint4 *>(base + row * kRow + (2 * j + hi) * 16);
            return i32x8_t{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        };
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            i32x8_t av[2], bv[4];
#pragma unroll
            for (int a = 0; a < 2; ++a) av[a] = frag(a_lds[cur], wm + 32 * a + r, j);
#pragma unroll
            for (int b = 0; b < 4; ++b) bv[b] = frag(b_lds[cur], wn + 32 * b + r, j);
            // swapped operands (W fragment first), so a lane receives output row r
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    if (j == 0)
                        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv[b], av[a], acc[a][b], 4, 4, 0,
                                                                                    bsc[b], 0, asc[a]);
                    else
                        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv[b], av[a], acc[a][b], 4, 4, 1,
                                                                                    bsc[b], 1, asc[a]);
                }
        }
        if (more) fetch_w(cw, sw, g, n0, s + 1, rw);
        // coefficients two stages ahead go to the buffer stage s's were in
        if (PRO == kBf16Kron && t < 16 && s + 2 < g.stages) derive_coefs(factors, g, s + 2, coef[cur]);
        if (more) {
            stash_a<PRO>(a_lds[cur ^ 1], as_lds[cur ^ 1], ra, coef[PRO == kBf16Kron ? cur ^ 1 : 0], g, s + 1);
            stash_w(b_lds[cur ^ 1], bs_lds[cur ^ 1], rw);
        }
        __syncthreads();
    }

    // lane (r, hi): O row wm + 32 a + r, columns wn + 32 b + 8 q + 4 hi + 0..3
    const bool vec = (reinterpret_cast<uintptr_t>(O) & 15) == 0 && g.ldo % 4 == 0;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int64_t row = m0 + wm + 32 * a + r;
        if (row >= g.m) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t col = n0 + wn + 32 * b + 8 * q + 4 * hi;
                float *o = O + row * g.ldo + col;
                if (vec && col + 3 < g.n) {
                    *reinterpret_cast<floatx4_t *>(o) =
                        floatx4_t{acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < g.n) o[e] = acc[a][b][4 * q + e];
                }
            }
    }
}

}  // namespace w4
}  // namespace kq

namespace {

using kqhost::aligned;
using kqhost::launched;

bool make_w4geom(int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldo, kq::w4::Geom &g, unsigned &nwg) {
    g.m = m;
    g.n = n;
    g.k = k;
    g.lda = lda;
    g.ldo = ldo;
    g.kblocks = (int)(k / 32);
    g.stages = (int)((k + 127) / 128);
    const int64_t tiles_m = (m + kq::w4::kM - 1) / kq::w4::kM;
    g.tiles_n = (n + kq::w4::kN - 1) / kq::w4::kN;
    // buffer records and offsets are 32-bit: one tile's rows of each operand must fit
    if ((int64_t)kq::w4::kM * (lda > k / 2 ? lda : k / 2) * 2 >= ((int64_t)1 << 31)) return false;
    if ((int64_t)kq::w4::kN * (k / 2) >= ((int64_t)1 << 31)) return false;
    if (tiles_m * g.tiles_n > 0x7FFFFFFF || k / 32 > 0x7FFFFFFF) return false;
    nwg = (unsigned)(tiles_m * g.tiles_n);
    return true;
}

kq_status check_w(const uint8_t *codes_w, const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, const float *O,
                  int64_t ldo) {
    if (m < 0 || n < 0 || k < 0 || k % 32 != 0 || ldo < n) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({m, n, k, ldo})) return KQ_ERR_UNSUPPORTED;
    if (m > 0 && n > 0 && (!codes_w || !scales_w || !O)) return KQ_ERR_NULL;
    if (!aligned(codes_w, 16)) return KQ_ERR_ALIGN;
    if ((k / 32) % 4 == 0 && !aligned(scales_w, 4)) return KQ_ERR_ALIGN;
    return KQ_OK;
}

}  // namespace

extern "C" {

kq_status kq_mxfp4_gemm_wide(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                             const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, float *O, int64_t ldo,
                             kq_stream_t stream) {
    kq_status s = check_w(codes_w, scales_w, m, n, k, O, ldo);
    if (s != KQ_OK) return s;
    if (m == 0 || n == 0) return KQ_OK;
    if (!codes_a || !scales_a) return KQ_ERR_NULL;
    if (!aligned(codes_a, 16) || ((k / 32) % 4 == 0 && !aligned(scales_a, 4))) return KQ_ERR_ALIGN;
    kq::w4::Geom g;
    unsigned nwg;
    if (!make_w4geom(m, n, k, k / 2, ldo, g, nwg)) return KQ_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((kq::w4::w4a4_kernel<kq::w4::kCodes>), dim3(nwg), dim3(kq::w4::kThreads), 0,
                       (hipStream_t)stream, codes_a, scales_a, nullptr, codes_w, scales_w, g, O);
    return launched();
}

kq_status kq_transform_quantize_mxfp4_gemm(const uint16_t *A, int64_t m, int64_t k, int64_t lda,
                                           const float *factors, const uint8_t *codes_w, const uint8_t *scales_w,
                                           int64_t n, float *O, int64_t ldo, kq_stream_t stream) {
    kq_status s = check_w(codes_w, scales_w, m, n, k, O, ldo);
    if (s != KQ_OK) return s;
    if (lda < k) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({lda})) return KQ_ERR_UNSUPPORTED;
    if (m == 0 || n == 0) return KQ_OK;
    if (!A || !factors) return KQ_ERR_NULL;
    if (!aligned(A, 16) || lda % 8 != 0 || !aligned(factors, 16)) return KQ_ERR_ALIGN;
    kq::w4::Geom g;
    unsigned nwg;
    if (!make_w4geom(m, n, k, lda, ldo, g, nwg)) return KQ_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((kq::w4::w4a4_kernel<kq::w4::kBf16Kron>), dim3(nwg), dim3(kq::w4::kThreads), 0,
                       (hipStream_t)stream, A, nullptr, factors, codes_w, scales_w, g, O);
    return launched();
}

}  // extern "C"
