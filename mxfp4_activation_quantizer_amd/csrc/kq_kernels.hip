// KroQuant online activation quantizer for MI355X (gfx950): kernels and the
// C ABI declared in include/kq.h.
//
// Method: KroQuant (arXiv 2607.21446v1). Per row of A and per 32-channel block
// j, y = a . K^(j) with K^(j) = G1 (x) G2 (x) G3 (x) G4 (x) G5 (Sec. 3.2 Eq. 5,
// Sec. 3.5.1 Eq. 12), then MXFP4 (Sec. 3.1; Sec. 4.1 "Data format", App. D).
//
// Work mapping of the bf16 kernels here (SmoothQuant and the fused transform;
// quantize-only and the Hadamard baselines use the flat tiles of kq_flat.hip):
// row-wave strips. A quad of lanes owns one 32-channel block of one row (16
// bytes per lane), a wave 16 consecutive blocks (one 1 KB segment) of one row,
// and a workgroup NW waves on NW consecutive rows of the same segment, walking
// `iters` such row groups. Rows are therefore wave-uniform: every address is a
// per-row scalar base (a buffer resource) plus a per-lane offset that never
// changes, so the vector ALU spends nothing on addressing. The op is HBM-bound
// in principle (2 bytes in, 0.5 + 1/32 bytes out per element), but the
// transform's arithmetic is close to the VALU budget, which is why the loop
// carries nothing else.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"
#include "kq_device.hpp"
#include "kq_host.hpp"

namespace kq {

constexpr int kThreads = 256;


// Grid-stride mapping of the fp32 kernels (fold, fp32 quantize): blocks are
// numbered row-major (b = row * nblk + j); workgroup w, quad q starts at block
// 64 w + q and advances by the whole grid (64 gridDim.x blocks, a multiple of
// nblk, so j stays fixed) per sweep, i.e. by rstep = 64 gridDim.x / nblk rows.
// A quad keeps one block column for its whole life, so per-block parameters
// load once.
struct Geom {
    int64_t m, lda, d, rstep;
    int nblk, iters;
};

__device__ __forceinline__ void flat_coords(const Geom &g, int &j, int &sub, int64_t &row0) {
    sub = threadIdx.x & 3;
    const int64_t b0 = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
    j = (int)(b0 % g.nblk);
    row0 = b0 / g.nblk;
}

// What a row-wave kernel writes besides codes and scales: nothing, the fp32
// transform result (check mode), or that result rounded to bf16 (the 16-bit
// activation a low-rank branch consumes).
enum YOut { kYNone = 0, kYF32 = 1, kYBF16 = 2 };

// Row-wave strips (see the file header). Workgroup b takes segment b % nseg
// (blocks 16 seg .. 16 seg + 15) and rows NW U (b / nseg) + w + NW u for its
// waves w and u < U: each wave issues its U row loads at once and handles
// them as one group. The last segment of a row may be partial (nblk % 16 !=
// 0): each buffer resource's record count is the valid bytes from the segment
// start to the end of the row's d channels, so lanes past the last block read
// zeros and their stores are dropped by the hardware range check.
struct RGeom {
    int64_t m, lda, d;  // elements
    int nblk, nseg;
};

// Buffer resource over `bytes` bytes from `base` (raw addressing, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// The per-row output pointers of a wave, advanced by NW rows after each store.
struct RowOut {
    char *codes, *scales, *y;
    int64_t codes_step, scales_step, y_step;
    uint32_t codes_bytes, scales_bytes, y_bytes;
};

// Per-lane byte offsets of a row's stores, computed once (kept in registers
// rather than recomputed per row).
struct LaneOff {
    uint32_t y32, y16, code, scale;
    bool scale_lane;  // lane 0 of its quad
};

// widen8 as one asm statement (the same eight shifts and masks): reading the
// load's registers makes the compiler wait for that load right there, and the
// dependence on `after` (a previous row's result) keeps the statement, and so
// the wait, after that row's work.
__device__ __forceinline__ void widen8_ordered(const uint4 &q, float x[8], uint32_t after) {
    asm volatile(
        "v_lshlrev_b32 %0, 16, %8\n\t"
        "v_and_b32 %1, 0xffff0000, %8\n\t"
        "v_lshlrev_b32 %2, 16, %9\n\t"
        "v_and_b32 %3, 0xffff0000, %9\n\t"
        "v_lshlrev_b32 %4, 16, %10\n\t"
        "v_and_b32 %5, 0xffff0000, %10\n\t"
        "v_lshlrev_b32 %6, 16, %11\n\t"
        "v_and_b32 %7, 0xffff0000, %11"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
        : "v"(q.x), "v"(q.y), "v"(q.z), "v"(q.w), "v"(after));
}

// One row's results as a lane holds them until the stores: codes dword, scale
// byte and, as YOUT asks, y (fp32) or y rounded to bf16 (four packed dwords).
template <int YOUT>
struct RowRes {
    uint32_t packed, sbyte;
    uint32_t y[YOUT == kYF32 ? 8 : (YOUT == kYBF16 ? 4 : 1)];
};

// Quantize the quad-held fp32 block (and keep y as YOUT asks).
template <int YOUT>
__device__ __forceinline__ void finish_row(const float y[8], RowRes<YOUT> &r) {
    if (YOUT == kYF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) r.y[i] = __float_as_uint(y[i]);
    } else if (YOUT == kYBF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.y[i] = (uint32_t)bf16_rne_bits(y[2 * i]) | ((uint32_t)bf16_rne_bits(y[2 * i + 1]) << 16);
    }
    r.packed = quantize_quad_f32(y, r.sbyte);
}

// Store one row's results and advance the output pointers by NW rows.
template <int YOUT>
__device__ __forceinline__ void store_row(const RowRes<YOUT> &r, RowOut &o, const LaneOff &lo) {
    if (YOUT == kYF32) {
        const auto d = buf_rsrc(o.y, o.y_bytes);
        __builtin_amdgcn_raw_buffer_store_b128((u32x4_t){r.y[0], r.y[1], r.y[2], r.y[3]}, d, lo.y32, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128((u32x4_t){r.y[4], r.y[5], r.y[6], r.y[7]}, d, lo.y32 + 16, 0, 0);
    } else if (YOUT == kYBF16) {
        __builtin_amdgcn_raw_buffer_store_b128((u32x4_t){r.y[0], r.y[1], r.y[2], r.y[3]}, buf_rsrc(o.y, o.y_bytes),
                                               lo.y16, 0, 0);
    }
    __builtin_amdgcn_raw_buffer_store_b32(r.packed, buf_rsrc(o.codes, o.codes_bytes), lo.code, 0, 0);
    // one lane per quad stores the block's scale byte (four lanes storing the
    // same byte measured slower)
    if (lo.scale_lane)
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)r.sbyte, buf_rsrc(o.scales, o.scales_bytes), lo.scale, 0, 0);
    o.codes += o.codes_step;
    o.scales += o.scales_step;
    o.y += o.y_step;
}

// The block's 16 per-lane coefficients, written to LDS by wave 0.
//
// Shear form. Each factor splits exactly as G = S D with S = [[1, p], [q, 1]],
// p = G01 / G11, q = G10 / G00, D = diag(G00, G11), and by the mixed-product
// rule K = (S1 (x) ... (x) S5)(D1 (x) ... (x) D5): five unit-diagonal shear
// stages, (x0, x1) -> (x0 + q x1, x1 + p x0), one fma per element each, then
// one multiply per channel by the product of its five diagonal entries. Every
// intermediate is the direct butterfly's intermediate divided by a
// per-channel constant, so rounding errors stay relative to the same
// quantities. The ratios use the hardware reciprocal (about 1 ulp): they are
// coefficients of an exact refactoring, so a last-bit difference only moves y
// by rounding. A block admits the form when every |p|, |q| <= 2^20 (a zero or
// tiny diagonal entry, a swap say, gives an infinite, NaN or huge ratio).
// Lane coefficients: c1 (G1, channel bit 4 = bit 1 of sub: this lane's
// partner weight, q for bit 0 and p for bit 1), c2 (G2, bit 3), p3, q3, p4,
// q4, p5, q5, then the 8 per-channel diagonal products.
//
// General form (any block of the segment without the shear form): the 2x2
// stages y = x_self G[b][b] + x_partner G[1-b][b] (KronLane layout: s1, o1,
// s2, o2, then G3, G4, G5 as 4 entries each).
//
// Every lane-dependent choice is an explicit select: a lane-dependent index
// into the factor array would become a chain of compares and selects.
struct SetupLane {
    float p[5], q[5];
    bool shear;
};

__device__ __forceinline__ void setup_ratios(const float f[20], SetupLane &S) {
    const float lim = 0x1.0p20f;
    S.shear = true;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        S.p[k] = f[4 * k + 1] * __builtin_amdgcn_rcpf(f[4 * k + 3]);
        S.q[k] = f[4 * k + 2] * __builtin_amdgcn_rcpf(f[4 * k]);
        S.shear = S.shear && fabsf(S.p[k]) <= lim && fabsf(S.q[k]) <= lim;  // false for inf and NaN
    }
}

__device__ __forceinline__ void write_shear_coefs(const float f[20], const SetupLane &S, int sub, float *dst) {
    const bool b4 = (sub >> 1) & 1, b3 = sub & 1;
    dst[0] = b4 ? S.p[0] : S.q[0];
    dst[1] = b3 ? S.p[1] : S.q[1];
#pragma unroll
    for (int k = 2; k < 5; ++k) {
        dst[2 * k - 2] = S.p[k];
        dst[2 * k - 1] = S.q[k];
    }
    // diagonal product of channel (b4, b3, i2, i1, i0): ((d12 G3[i2][i2]) G4[i1][i1]) G5[i0][i0]
    const float d12 = (b4 ? f[3] : f[0]) * (b3 ? f[7] : f[4]);
    float t3[2], t4[4];
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) t3[i2] = d12 * f[8 + 3 * i2];
#pragma unroll
    for (int i = 0; i < 4; ++i) t4[i] = t3[i >> 1] * f[12 + 3 * (i & 1)];
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[8 + i] = t4[i >> 1] * f[16 + 3 * (i & 1)];
}

__device__ __forceinline__ void write_general_coefs(const float f[20], int sub, float *dst) {
    const bool b4 = (sub >> 1) & 1, b3 = sub & 1;
    dst[0] = b4 ? f[3] : f[0];  // G1[b4][b4]
    dst[1] = b4 ? f[1] : f[2];  // G1[1-b4][b4]
    dst[2] = b3 ? f[7] : f[4];  // G2[b3][b3]
    dst[3] = b3 ? f[5] : f[6];  // G2[1-b3][b3]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dst[4 + i] = f[8 + i];
        dst[8 + i] = f[12 + i];
        dst[12 + i] = f[16 + i];
    }
}

template <bool SHEAR>
__device__ __forceinline__ void apply_coefs(float y[8], const float c[16]) {
    if (SHEAR) {
        fmac_partner_xor2(y, c[0]);  // G1: channel bit 4 = bit 1 of sub
        fmac_partner_xor1(y, c[1]);  // G2: channel bit 3 = bit 0 of sub
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

// bf16 input, row-wave strips: SmoothQuant (T = diag(inv_scale)) or the
// Kronecker transform. Each wave's U row loads are issued at once; for the
// transform they are in flight while wave 0 derives the segment's
// coefficients (factor loads, reciprocals, LDS writes, barrier).
// PK: scales written in the packed-GEMM layout [d/256][m][8] (even blocks of
// a 256-channel stage first) instead of [m][d/32]; d % 256 == 0.
template <int MODE, int YOUT, int NW, int U, bool PK = false>
__global__ __launch_bounds__(NW * 64) void rowwave_kernel(const uint16_t *__restrict__ A, RGeom g,
                                                          const float *__restrict__ params,
                                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                          void *__restrict__ yout) {
    static_assert(MODE == kSmooth || MODE == kKron, "quantize-only runs on the flat kernel");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane & 3;
    const int seg = (int)(blockIdx.x % (unsigned)g.nseg);
    const int64_t row0 = (int64_t)(blockIdx.x / (unsigned)g.nseg) * NW * U + wave;
    const int j = seg * 16 + (lane >> 2);
    const bool active = j < g.nblk;
    const int64_t c_seg = (int64_t)seg * 512;  // first channel of the segment
    // rows of this wave: row0 + NW u for u < nr
    const int64_t left = row0 < g.m ? (g.m - row0 + NW - 1) / NW : 0;
    const int nr = (int)(left < U ? left : U);

    const char *a_row = reinterpret_cast<const char *>(A + row0 * g.lda + c_seg);
    const int64_t a_step = (int64_t)NW * g.lda * 2;
    const uint32_t a_bytes = (uint32_t)((g.d - c_seg) * 2);
    const uint32_t a_off = (uint32_t)lane * 16;
    LaneOff lo{(uint32_t)lane * 32, (uint32_t)lane * 16, (uint32_t)lane * 4, (uint32_t)lane >> 2, (lane & 3) == 0};
    if constexpr (PK) {
        // packed scale byte of block j: stage j / 8, row, byte 4 (j & 1) + (j & 7) / 2;
        // a lane past the last block gets an offset past the record count
        lo.scale = active ? (uint32_t)((j >> 3) * g.m * 8 + 4 * (j & 1) + ((j & 7) >> 1)) : 0xFFFFFFF0u;
    }
    asm volatile("" : "+v"(lo.y32), "+v"(lo.code), "+v"(lo.scale));  // opaque: not rematerialized per row
    RowOut o;
    if constexpr (PK) {
        // base at the row's 8-byte piece of stage 0; every valid offset of every
        // row of the wave stays below m d / 32 - 8 row0
        const int64_t left_bytes = g.m * g.nblk - row0 * 8;
        o.codes = reinterpret_cast<char *>(codes + row0 * (g.d / 2) + c_seg / 2);
        o.scales = reinterpret_cast<char *>(scales + row0 * 8);
        o.codes_step = (int64_t)NW * (g.d / 2);
        o.scales_step = (int64_t)NW * 8;
        o.codes_bytes = (uint32_t)((g.d - c_seg) / 2);
        o.scales_bytes = (uint32_t)(left_bytes > 0 ? left_bytes : 0);
    } else {
        o.codes = reinterpret_cast<char *>(codes + row0 * (g.d / 2) + c_seg / 2);
        o.scales = reinterpret_cast<char *>(scales + row0 * g.nblk + seg * 16);
        o.codes_step = (int64_t)NW * (g.d / 2);
        o.scales_step = (int64_t)NW * g.nblk;
        o.codes_bytes = (uint32_t)((g.d - c_seg) / 2);
        o.scales_bytes = (uint32_t)(g.nblk - seg * 16);
    }
    const int ysize = YOUT == kYF32 ? 4 : 2;
    o.y = YOUT == kYNone ? nullptr : static_cast<char *>(yout) + (row0 * g.d + c_seg) * ysize;
    o.y_step = (int64_t)NW * g.d * ysize;
    o.y_bytes = (uint32_t)((g.d - c_seg) * ysize);

    // Every load is issued; a row past the wave's last one gets a buffer of
    // zero records, so it reads zeros without touching memory (and the
    // compiler's wait counts stay exact).
    uint4 q[U];
    auto load_rows = [&]() {
        const char *p = a_row;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(p, u < nr ? a_bytes : 0u), a_off, 0, 2);
            q[u] = make_uint4(v[0], v[1], v[2], v[3]);
            p += a_step;
        }
    };
    // Each row is transformed and quantized as soon as its load is back, and
    // every store waits until all rows are done: stores count in the same
    // vector-memory counter as loads, so a wait for a later row's load issued
    // after earlier rows' stores would also wait for those stores to be
    // acknowledged. Row u is widened by widen8_ordered, which reads the load's
    // registers (so the compiler waits for exactly that load there) and takes
    // row u-1's codes dword as an operand (so neither the widening nor its wait
    // is hoisted above row u-1's work, nor merged across the two forms of the
    // transform). Rows past the wave's last one hold zeros; they are computed
    // (no branch) but not stored.
    auto rows = [&](auto per_row) {
        RowRes<YOUT> res[U];
        uint32_t chain = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float y[8];
            widen8_ordered(q[u], y, chain);
            per_row(y);
            finish_row<YOUT>(y, res[u]);
            chain = res[u].packed;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u >= nr) break;
            store_row<YOUT>(res[u], o, lo);
        }
    };
    if (MODE == kSmooth) {
        float sq[8];
        const float4 lo = active ? *reinterpret_cast<const float4 *>(params + j * 32 + sub * 8) : make_float4(0, 0, 0, 0);
        const float4 hi = active ? *reinterpret_cast<const float4 *>(params + j * 32 + sub * 8 + 4) : make_float4(0, 0, 0, 0);
        sq[0] = lo.x; sq[1] = lo.y; sq[2] = lo.z; sq[3] = lo.w;
        sq[4] = hi.x; sq[5] = hi.y; sq[6] = hi.z; sq[7] = hi.w;
        load_rows();
        rows([&](float y[8]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = y[i] * sq[i];
        });
        return;
    }

    // Kronecker transform: wave 0 (one lane per block and channel group)
    // derives the coefficients; a ballot picks one form for the workgroup, so
    // the branch below is uniform and the rows carry no divergence. Wave 0
    // issues its factor loads before its row loads, so waiting for the
    // factors leaves the rows in flight.
    __shared__ float coef[64][17];
    __shared__ int all_shear;
    float f[20];
    if (wave == 0 && active) load_factors20(params + (int64_t)j * 20, f);
    load_rows();
    if (wave == 0) {
        SetupLane S;
        if (active) setup_ratios(f, S);
        const bool all = __builtin_amdgcn_ballot_w64(active && !S.shear) == 0;
        if (!active) {
#pragma unroll
            for (int i = 0; i < 16; ++i) coef[lane][i] = 0.f;
        } else if (all) {
            write_shear_coefs(f, S, sub, coef[lane]);
        } else {
            write_general_coefs(f, sub, coef[lane]);
        }
        if (lane == 0) all_shear = all;
    }
    __syncthreads();
    float c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = coef[lane][i];
    if (__builtin_amdgcn_readfirstlane(all_shear)) {
        rows([&](float y[8]) { apply_coefs<true>(y, c); });
    } else {
        rows([&](float y[8]) { apply_coefs<false>(y, c); });
    }
}

// MFMA form of the fused kernel. Each wave owns NB consecutive blocks and walks
// `iters` tiles of 16 tokens of one slab; a workgroup is 4 such waves with
// consecutive wave ids (neighbouring column groups).
struct MGeom {
    int64_t m, lda, d, nwaves;
    int nblk, ncg, iters;
};

template <int NB, bool DEBUG, int U, bool NT>
__global__ __launch_bounds__(kThreads) void kron_mfma_kernel(
    const uint16_t *__restrict__ A, MGeom g, const float *__restrict__ factors,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ ydbg) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wid >= g.nwaves) return;  // whole waves only
    const int cgw = (int)(wid % g.ncg);
    const int64_t tile0 = (wid / g.ncg) * g.iters;
    const int grp = lane >> 4;

    KSplit S[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ksplit_setup(factors + (int64_t)(cgw * NB + nb) * 20, lane, S[nb]);

    auto load_tiles = [&](int it, uint4 (&q)[U][NB]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t tok = (tile0 + it + u) * 16 + (lane & 15);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int64_t off = tok * g.lda + (int64_t)(cgw * NB + nb) * 32 + grp * 8;
                q[u][nb] = tok < g.m ? load_stream(reinterpret_cast<const uint4 *>(A + off), NT)
                                     : make_uint4(0, 0, 0, 0);
            }
        }
    };

    for (int it = 0; it < g.iters; it += U) {
        if ((tile0 + it) * 16 >= g.m) break;  // uniform within the wave
        uint4 q[U][NB];
        load_tiles(it, q);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t tok = (tile0 + it + u) * 16 + (lane & 15);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int jb = cgw * NB + nb;
                float y[8];
                kron_mfma8(S[nb], q[u][nb], y);  // all 64 lanes take part
                const float amax = max_xor16_xor32(absmax8(y));
                const uint32_t sbyte = e8m0_byte(amax);
                const uint32_t packed = cvt8_f32(y, cvt_scale(sbyte));
                if (tok < g.m) {
                    if (DEBUG) {
                        float4 *o = reinterpret_cast<float4 *>(ydbg + tok * g.d + (int64_t)jb * 32 + grp * 8);
                        o[0] = make_float4(y[0], y[1], y[2], y[3]);
                        o[1] = make_float4(y[4], y[5], y[6], y[7]);
                    }
                    *reinterpret_cast<uint32_t *>(codes + tok * (g.d / 2) + (int64_t)jb * 16 + grp * 4) = packed;
                    if (grp == 0) scales[tok * g.nblk + jb] = (uint8_t)sbyte;
                }
            }
        }
    }
}

// MFMA form with LDS staging. A workgroup (4 waves) owns a strip of 16
// consecutive blocks and walks `iters` tiles of 16 tokens. Each tile (16 rows x
// 1 KB of bf16) is loaded with fully coalesced 16-byte loads (one 1 KB row per
// 64 lanes) into LDS, double-buffered so the next tile's loads are in flight
// while this one is transformed; wave w then reads the MFMA operand of its
// blocks 4w .. 4w+3 (token l % 16, channels 8 (l / 16) .. +7) from LDS. LDS rows
// are padded by 16 bytes, so the 16 lanes of a read phase hit distinct banks.
struct LGeom {
    int64_t m, lda, d;
    int nblk, nstrip, iters;
};

template <bool DEBUG>
__global__ __launch_bounds__(kThreads, 3) void kron_mfma_lds_kernel(
    const uint16_t *__restrict__ A, LGeom g, const float *__restrict__ factors,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ ydbg) {
    __shared__ uint4 xs[2][16][65];
    // codes and scale bytes of a tile, row-major (16 tokens x 16 blocks; a code row is padded to
    // 68 dwords, so the 64 lanes of one write land in 64 different banks), written to HBM after
    // the next barrier as whole 256-byte code rows and 16-byte scale rows
    __shared__ __attribute__((aligned(16))) uint32_t cs[2][16][68];
    __shared__ uint8_t ss[2][16][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4;
    const int strip = (int)(blockIdx.x % (unsigned)g.nstrip);
    const int64_t tile0 = (int64_t)(blockIdx.x / (unsigned)g.nstrip) * g.iters;
    const int jb0 = strip * 16 + wave * 4;

    KSplit S[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ksplit_setup(factors + (int64_t)(jb0 + q) * 20, lane, S[q]);

    // tile t: thread tid moves rows 4 r + tid / 64 (r < 4), 16-byte column tid % 64
    const uint16_t *Astrip = A + (int64_t)strip * 512 + (tid & 63) * 8;
    auto load_tile = [&](int64_t t, uint4 (&v)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t tok = t * 16 + 4 * r + (tid >> 6);
            v[r] = tok < g.m ? load_stream(reinterpret_cast<const uint4 *>(Astrip + tok * g.lda), true)
                             : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&](int buf, const uint4 (&v)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[buf][4 * r + (tid >> 6)][tid & 63] = v[r];
    };

    // tile t from buffer b to HBM: thread tid moves 16 code bytes of token 16 t + tid / 16
    // (columns 16 (tid % 16) ..) and that token's scale byte of block tid % 16 of the strip
    auto flush = [&](int64_t t, int b) {
        const int r = tid >> 4, c = tid & 15;
        const int64_t tok = t * 16 + r;
        if (tok < g.m) {
            *reinterpret_cast<uint4 *>(codes + tok * (g.d / 2) + (int64_t)strip * 256 + 16 * c) =
                *reinterpret_cast<const uint4 *>(&cs[b][r][4 * c]);
            scales[tok * g.nblk + strip * 16 + c] = ss[b][r][c];
        }
    };

    uint4 v[4];
    if (tile0 * 16 >= g.m) return;  // uniform within the workgroup
    load_tile(tile0, v);
    store_tile(0, v);
    __syncthreads();
    int it = 0;
    for (; it < g.iters; ++it) {
        const int64_t t = tile0 + it;
        if (t * 16 >= g.m) break;  // uniform within the workgroup
        const bool more = it + 1 < g.iters && (t + 1) * 16 < g.m;
        if (more) load_tile(t + 1, v);
        const int buf = it & 1;
        // the previous tile's codes, written before the last barrier; buffer buf ^ 1 is written
        // again only after the next barrier
        if (it > 0) flush(t - 1, buf ^ 1);
        const int64_t tok = t * 16 + (lane & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int jb = jb0 + q;
            const uint4 x = xs[buf][lane & 15][(wave * 4 + q) * 4 + grp];
            float y[8];
            kron_mfma8(S[q], x, y);  // all 64 lanes take part
            const float amax = max_xor16_xor32(absmax8(y));
            const uint32_t sbyte = e8m0_byte(amax);
            const uint32_t packed = cvt8_f32(y, cvt_scale(sbyte));
            if (DEBUG && tok < g.m) {
                float4 *o = reinterpret_cast<float4 *>(ydbg + tok * g.d + (int64_t)jb * 32 + grp * 8);
                o[0] = make_float4(y[0], y[1], y[2], y[3]);
                o[1] = make_float4(y[4], y[5], y[6], y[7]);
            }
            cs[buf][lane & 15][(wave * 4 + q) * 4 + grp] = packed;
            if (grp == 0) ss[buf][lane & 15][wave * 4 + q] = (uint8_t)sbyte;
        }
        if (more) store_tile(buf ^ 1, v);
        __syncthreads();
    }
    // it >= 1 here: tile tile0 exists (checked above) and the loop ran it
    flush(tile0 + it - 1, (it - 1) & 1);
}

// fp32 input, quad layout: quantize (MODE kQuantOnly) or, with MODE kKron,
// write X . (K^(j))^{-T} (the weight fold) to `out` instead of quantizing.
template <int MODE>
__global__ __launch_bounds__(kThreads) void f32_kernel(
    const float *__restrict__ X, Geom g, const float *__restrict__ factors,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ out) {
    int j, sub;
    int64_t row0;
    flat_coords(g, j, sub, row0);
    const int64_t R = g.rstep;
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
            const uint32_t packed = quantize_quad_f32(y, sbyte);
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

using kqhost::aligned;
using kqhost::check_bf16_io;
using kqhost::check_shape;
using kqhost::launched;

int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// Grid-stride geometry: about `target_wg` workgroups (fewer if the matrix is small), a multiple
// of nblk / gcd(64, nblk) so that 64 * gridDim.x is a multiple of nblk.
// `iters` (sweeps per workgroup) is rounded up to a multiple of `unroll`.
bool make_geom_flat(int64_t m, int64_t d, int64_t ld, int unroll, int64_t target_wg, kq::Geom &g,
                    unsigned &nwg) {
    g.m = m;
    g.d = d;
    g.lda = ld;
    g.nblk = (int)(d / 32);
    const int64_t k0 = g.nblk / gcd64(64, g.nblk);
    const int64_t need = (m * g.nblk + 63) / 64;
    int64_t w = need < target_wg ? need : target_wg;
    w = (w + k0 - 1) / k0 * k0;
    if (w > 0x7FFFFFFF) return false;
    g.rstep = w * 64 / g.nblk;
    int64_t iters = (m + g.rstep - 1) / g.rstep;
    iters = (iters + unroll - 1) / unroll * unroll;
    if (iters > 0x7FFFFFFF) return false;
    g.iters = (int)iters;
    nwg = (unsigned)w;
    return true;
}

// MFMA form: waves own NB blocks and `iters` 16-token tiles (a multiple of the unroll).
bool make_mgeom(int64_t m, int64_t d, int64_t lda, int nb, int unroll, kq::MGeom &g, unsigned &nwg,
                int64_t target_waves = 0) {
    g.m = m;
    g.d = d;
    g.lda = lda;
    g.nblk = (int)(d / 32);
    g.ncg = g.nblk / nb;
    const int64_t tiles = (m + 15) / 16;
    const int64_t units = tiles * g.ncg;
    // default: about one resident round of waves, occupancy 4 (NB = 2) or 6 (NB = 1) per SIMD
    if (target_waves <= 0) target_waves = 256 * 4 * (nb == 2 ? 4 : 6);
    int64_t iters = (units + target_waves - 1) / target_waves;
    if (iters < 1) iters = 1;
    if (iters > (1 << 20)) iters = 1 << 20;
    iters = (iters + unroll - 1) / unroll * unroll;
    const int64_t nslab = (tiles + iters - 1) / iters;
    g.nwaves = nslab * g.ncg;
    const int64_t wg = (g.nwaves + 3) / 4;
    if (wg > 0x7FFFFFFF) return false;
    g.iters = (int)iters;
    nwg = (unsigned)wg;
    return true;
}

// Row-wave geometry: 16-block segments (the last one partial when nblk % 16 !=
// 0), workgroups of NW waves with U rows each (NW U consecutive rows).
bool make_rgeom(int64_t m, int64_t d, int64_t lda, int nw, int u, kq::RGeom &g, unsigned &nwg) {
    // buffer records and offsets are 32-bit: a row's bytes (fp32 y in check
    // mode: 4 d) must fit
    if (d > ((int64_t)1 << 29)) return false;
    g.m = m;
    g.d = d;
    g.lda = lda;
    g.nblk = (int)(d / 32);
    g.nseg = (g.nblk + 15) / 16;
    const int64_t slabs = (m + (int64_t)nw * u - 1) / ((int64_t)nw * u);
    const int64_t total = slabs * g.nseg;
    if (total > 0x7FFFFFFF) return false;
    nwg = (unsigned)total;
    return true;
}

// Launch shapes, chosen by sweeping waves per workgroup (4, 8, 16), rows per
// load group (2, 3, 4, 8) and row groups per workgroup (2 ... 16) on the
// 18432 x 3072 and 18432 x 12288 shapes: the transform takes 4 waves that
// each load 4 rows at once and finish (a workgroup covers 16 blocks x 16
// rows; longer-lived workgroups were slower although they amortize the setup);
// SmoothQuant, with no setup, takes 8 waves of 4 rows.
template <int MODE, int YOUT, bool PK = false>
kq_status launch_rowwave(const uint16_t *A, int64_t m, int64_t d, int64_t lda, const float *params,
                         uint8_t *codes, uint8_t *scales, void *yout, kq_stream_t stream) {
    constexpr int NW = MODE == kq::kKron ? 4 : 8;
    constexpr int U = 4;
    kq::RGeom g;
    unsigned nwg;
    if (!make_rgeom(m, d, lda, NW, U, g, nwg)) return KQ_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((kq::rowwave_kernel<MODE, YOUT, NW, U, PK>), dim3(nwg), dim3(NW * 64), 0,
                       (hipStream_t)stream, A, g, params, codes, scales, yout);
    return launched();
}

template <int NB, bool DEBUG>
kq_status launch_mfma(const uint16_t *A, int64_t m, int64_t d, int64_t lda, const float *factors,
                      uint8_t *codes, uint8_t *scales, float *ydbg, kq_stream_t stream) {
    kq::MGeom g;
    unsigned nwg;
    if (!make_mgeom(m, d, lda, NB, 2, g, nwg)) return KQ_ERR_SHAPE;
    hipLaunchKernelGGL((kq::kron_mfma_kernel<NB, DEBUG, 2, false>), dim3(nwg), dim3(kq::kThreads), 0,
                       (hipStream_t)stream, A, g, factors, codes, scales, ydbg);
    return launched();
}

// Compute units of the current device (cached per device; 256 on MI355X).
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Tiles per workgroup of the LDS-staged MFMA form. Three workgroups fit a CU (168
// registers per lane, 42.5 KB of LDS); a workgroup's factor setup costs about two
// tiles. Among 4 .. 12 tiles that still give every resident slot a workgroup, the
// fewest rounds x (tiles + 2), where a last round of under 1/16 of the slots counts
// nothing (those few workgroups run at the bandwidth of an idle chip); small inputs
// take the most workgroups. Measured against a fixed 6 (events, interleaved):
// 18432 x 3072 9 tiles 31.3 against 33.7 us, 18432 x 12288 12 tiles 104.2 against
// 105.2, 4096 x 12288 8 tiles 28.8 against 30.6; 8192 x 4608 lost 10% with 4 tiles
// (1152 workgroups) against 6 (774: one round and 6 more).
int64_t lds_form_iters(int64_t tiles, int64_t nstrip) {
    const int64_t slots = 3 * (int64_t)device_cus(), tol = slots / 16;
    int64_t best = 0, best_cost = 0;
    for (int64_t it = 4; it <= 12; ++it) {
        const int64_t wgs = (tiles + it - 1) / it * nstrip;
        if (wgs < slots) break;  // fewer workgroups for every larger count
        const int64_t rounds = (wgs - tol + slots - 1) / slots;
        const int64_t cost = (rounds < 1 ? 1 : rounds) * (it + 2);
        if (best == 0 || cost < best_cost) {
            best = it;
            best_cost = cost;
        }
    }
    if (best) return best;
    const int64_t it = tiles * nstrip / slots;  // largest count that still fills the slots, if any
    return it < 1 ? 1 : (it > 4 ? 4 : it);
}

// LDS-staged MFMA form: strips of 16 blocks (nblk % 16 == 0), `iters` tiles of
// 16 tokens per workgroup (0: chosen by lds_form_iters).
bool make_lgeom(int64_t m, int64_t d, int64_t lda, int64_t iters_per_wg, kq::LGeom &g, unsigned &nwg) {
    g.m = m;
    g.d = d;
    g.lda = lda;
    g.nblk = (int)(d / 32);
    if (g.nblk % 16 != 0) return false;
    g.nstrip = g.nblk / 16;
    const int64_t tiles = (m + 15) / 16;
    if (iters_per_wg == 0 && tiles > 0) iters_per_wg = lds_form_iters(tiles, g.nstrip);
    int64_t iters = iters_per_wg < 1 ? 1 : iters_per_wg;
    if (iters > tiles) iters = tiles;
    const int64_t nslab = (tiles + iters - 1) / iters;
    const int64_t total = nslab * g.nstrip;
    if (total > 0x7FFFFFFF || iters > 0x7FFFFFFF) return false;
    g.iters = (int)iters;
    nwg = (unsigned)total;
    return true;
}

template <bool DEBUG>
kq_status launch_mfma_lds(const uint16_t *A, int64_t m, int64_t d, int64_t lda, const float *factors,
                          uint8_t *codes, uint8_t *scales, float *ydbg, kq_stream_t stream) {
    kq::LGeom g;
    unsigned nwg;
    if (!make_lgeom(m, d, lda, 0, g, nwg)) return KQ_ERR_SHAPE;
    hipLaunchKernelGGL((kq::kron_mfma_lds_kernel<DEBUG>), dim3(nwg), dim3(kq::kThreads), 0,
                       (hipStream_t)stream, A, g, factors, codes, scales, ydbg);
    return launched();
}

// The form of the transform a fused call runs (kq_transform_form): five
// in-register 2x2 stages in shear form (the default), or the materialized 32x32
// block on MFMA with operands loaded directly or through LDS-staged row-major
// tiles (that one needs d a multiple of 512, else the butterfly runs).
template <bool DEBUG>
kq_status launch_fused(const uint16_t *A, int64_t m, int64_t d, int64_t lda, const float *factors,
                       uint8_t *codes, uint8_t *scales, float *ydbg, int form, kq_stream_t stream) {
    if (form == KQ_FORM_MFMA_LDS && (d / 32) % 16 == 0)
        return launch_mfma_lds<DEBUG>(A, m, d, lda, factors, codes, scales, ydbg, stream);
    if (form != KQ_FORM_MFMA)
        return launch_rowwave<kq::kKron, DEBUG ? kq::kYF32 : kq::kYNone>(A, m, d, lda, factors, codes, scales, ydbg,
                                                                          stream);
    if ((d / 32) % 2 == 0)
        return launch_mfma<2, DEBUG>(A, m, d, lda, factors, codes, scales, ydbg, stream);
    return launch_mfma<1, DEBUG>(A, m, d, lda, factors, codes, scales, ydbg, stream);
}

}  // namespace

extern "C" {

kq_status kq_transform_quantize_mxfp4_form(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                           const float *factors, uint8_t *codes, uint8_t *scales,
                                           float *y_debug, int form, kq_stream_t stream) {
    if (form != KQ_FORM_BUTTERFLY && form != KQ_FORM_MFMA && form != KQ_FORM_MFMA_LDS) return KQ_ERR_UNSUPPORTED;
    kq_status s = check_shape(m, d, lda);
    if (s != KQ_OK) return s;
    if (m == 0 || d == 0) return KQ_OK;
    if ((s = check_bf16_io(A, lda, codes, scales)) != KQ_OK) return s;
    if (!factors) return KQ_ERR_NULL;
    if (!aligned(factors, 16) || (y_debug && !aligned(y_debug, 16))) return KQ_ERR_ALIGN;
    if (y_debug) return launch_fused<true>(A, m, d, lda, factors, codes, scales, y_debug, form, stream);
    return launch_fused<false>(A, m, d, lda, factors, codes, scales, nullptr, form, stream);
}

kq_status kq_transform_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                      const float *factors, uint8_t *codes, uint8_t *scales,
                                      float *y_debug, kq_stream_t stream) {
    return kq_transform_quantize_mxfp4_form(A, m, d, lda, factors, codes, scales, y_debug, KQ_FORM_BUTTERFLY,
                                            stream);
}

kq_status kq_transform_quantize_mxfp4_y16(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                          const float *factors, uint8_t *codes, uint8_t *scales, uint16_t *y16,
                                          kq_stream_t stream) {
    kq_status s = check_shape(m, d, lda);
    if (s != KQ_OK) return s;
    if (m == 0 || d == 0) return KQ_OK;
    if ((s = check_bf16_io(A, lda, codes, scales)) != KQ_OK) return s;
    if (!factors || !y16) return KQ_ERR_NULL;
    if (!aligned(factors, 16) || !aligned(y16, 16)) return KQ_ERR_ALIGN;
    return launch_rowwave<kq::kKron, kq::kYBF16>(A, m, d, lda, factors, codes, scales, y16, stream);
}

kq_status kq_transform_quantize_mxfp4_packed(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                             const float *factors, uint8_t *codes, uint8_t *packed_scales,
                                             uint16_t *y16, kq_stream_t stream) {
    kq_status s = check_shape(m, d, lda);
    if (s != KQ_OK) return s;
    if (d % 256 != 0) return KQ_ERR_SHAPE;
    if (m == 0 || d == 0) return KQ_OK;
    if ((s = check_bf16_io(A, lda, codes, packed_scales)) != KQ_OK) return s;
    if (!factors) return KQ_ERR_NULL;
    if (!aligned(factors, 16) || (y16 && !aligned(y16, 16))) return KQ_ERR_ALIGN;
    // packed offsets span the whole scale array in one 32-bit record count
    if (m > (((int64_t)1 << 31) - 16) / (d / 32)) return KQ_ERR_UNSUPPORTED;
    if (y16)
        return launch_rowwave<kq::kKron, kq::kYBF16, true>(A, m, d, lda, factors, codes, packed_scales, y16, stream);
    return launch_rowwave<kq::kKron, kq::kYNone, true>(A, m, d, lda, factors, codes, packed_scales, nullptr, stream);
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
    return launch_rowwave<kq::kSmooth, kq::kYNone>(A, m, d, lda, inv_scale, codes, scales, nullptr, stream);
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
    if (!make_geom_flat(m, d, ldx, 1, 256 * 8, g, nwg)) return KQ_ERR_SHAPE;
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
    if (!make_geom_flat(o, d, d, 1, 256 * 8, g, nwg)) return KQ_ERR_SHAPE;
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

int kq_last_hip_error(void) { return kqhost::g_last_hip_error; }

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
