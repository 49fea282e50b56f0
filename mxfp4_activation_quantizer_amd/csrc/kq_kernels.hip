// KroQuant online activation quantizer for MI355X (gfx950): kernels and the
// C ABI declared in include/kq.h.
//
// Method: KroQuant (arXiv 2607.21446v1). Per row of A and per 32-channel block
// j, y = a . K^(j) with K^(j) = G1 (x) G2 (x) G3 (x) G4 (x) G5 (Sec. 3.2 Eq. 5,
// Sec. 3.5.1 Eq. 12), then MXFP4 (Sec. 3.1; Sec. 4.1 "Data format", App. D).
//
// Work mapping (the strip kernels here: SmoothQuant and the fused transform;
// quantize-only and the Hadamard baselines use the flat tiles of kq_flat.hip):
// a workgroup of 256 lanes = 64 quads; a quad
// owns one 32-channel block of one row (16 bytes per lane). The 64 quads cover
// CB = 2^cb_log2 consecutive blocks of R = 64 / CB consecutive rows, so every
// row segment a workgroup touches is CB * 64 contiguous bytes. A workgroup
// stays on one column group (its per-block parameters load once into
// registers) and walks `iters` row tiles of one slab. The op is HBM-bound:
// 2 bytes in, 0.5 + 1/32 bytes out per element.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "kq.h"
#include "kq_device.hpp"
#include "kq_host.hpp"

namespace kq {

constexpr int kThreads = 256;


// Workgroup -> work mapping of the quad kernels (a workgroup is 64 quads, a
// quad owns one 32-channel block of one row at a time).
//  kStrip: the 64 quads cover CB = 2^cb_log2 consecutive blocks of R = 64 / CB
//          consecutive rows; workgroup w takes column group w % ncg and row
//          slab w / ncg and walks `iters` row tiles of that slab (rstep = R).
//  kFlat:  blocks are numbered row-major (b = row * nblk + j); workgroup w,
//          quad q starts at block 64 w + q and advances by the whole grid
//          (64 gridDim.x blocks, a multiple of nblk, so j stays fixed) per
//          sweep, i.e. by rstep = 64 gridDim.x / nblk rows.
// In both, a quad keeps one block column for its whole life, so per-block
// parameters load once.
enum Map { kStrip = 0, kFlat = 1 };

struct Geom {
    int64_t m, lda, d, rstep;
    int nblk, iters, cb_log2, ncg;
};

template <int MAP>
__device__ __forceinline__ void lane_coords(const Geom &g, int &j, int &sub, int64_t &row0) {
    sub = threadIdx.x & 3;
    const int quad = threadIdx.x >> 2;
    if (MAP == kFlat) {
        const int64_t b0 = (int64_t)blockIdx.x * 64 + quad;
        j = (int)(b0 % g.nblk);
        row0 = b0 / g.nblk;
    } else {
        const int cg = (int)(blockIdx.x % (unsigned)g.ncg);
        const int64_t slab = blockIdx.x / (unsigned)g.ncg;
        j = (cg << g.cb_log2) + (quad & ((1 << g.cb_log2) - 1));
        row0 = slab * g.rstep * g.iters + (quad >> g.cb_log2);
    }
}

// Loads of this quad's rows row0 + (it + u) rstep, u < U (zeros past m).
template <int U, bool NT>
__device__ __forceinline__ void load_rows(const Geom &g, const uint16_t *__restrict__ A, int64_t row0,
                                          int64_t c0, int it, uint4 q[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t row = row0 + (int64_t)(it + u) * g.rstep;
        q[u] = row < g.m ? load_stream(reinterpret_cast<const uint4 *>(A + row * g.lda + c0), NT)
                         : make_uint4(0, 0, 0, 0);
    }
}

// Walks this quad's rows row0 + k rstep (k < iters), U rows' loads at a time,
// and calls body(q, row) for each row below m. `q` holds the first group's
// loads already when `preloaded` (issued before the per-block setup, so their
// latency overlaps it). The row test is uniform within a quad, so DPP inside
// `body` sees all four lanes. (Issuing the next group's loads before
// processing this one, with or without raised wave priority, measured slower
// on the FLUX shapes: it costs registers and occupancy.)
template <int U, bool NT, typename Body>
__device__ __forceinline__ void for_rows(const Geom &g, const uint16_t *__restrict__ A, int64_t row0,
                                         int64_t c0, uint4 q[U], bool preloaded, Body body) {
    const int64_t R = g.rstep;
    for (int it = 0; it < g.iters; it += U) {
        if (row0 + (int64_t)it * R >= g.m) break;
        if (it > 0 || !preloaded) load_rows<U, NT>(g, A, row0, c0, it, q);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = row0 + (int64_t)(it + u) * R;
            if (row >= g.m) break;
            body(q[u], row);
        }
    }
}

// What a quad kernel writes besides codes and scales: nothing, the fp32
// transform result (check mode), or that result rounded to bf16 (the 16-bit
// activation a low-rank branch consumes).
enum YOut { kYNone = 0, kYF32 = 1, kYBF16 = 2 };

// Quantize fp32 values of a quad-held block and store codes and scale, and y
// as YOUT asks (fp32 or bf16 [m][d]).
template <int YOUT>
__device__ __forceinline__ void finish_f32(const float y[8], const Geom &g, int64_t row, int j, int sub,
                                           int64_t c0, uint8_t *__restrict__ codes,
                                           uint8_t *__restrict__ scales, void *__restrict__ yout) {
    if (YOUT == kYF32) {
        float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(yout) + row * g.d + c0);
        o[0] = make_float4(y[0], y[1], y[2], y[3]);
        o[1] = make_float4(y[4], y[5], y[6], y[7]);
    } else if (YOUT == kYBF16) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (uint32_t)bf16_rne_bits(y[2 * i]) | ((uint32_t)bf16_rne_bits(y[2 * i + 1]) << 16);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(yout) + row * g.d + c0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    uint32_t sbyte;
    const uint32_t packed = quantize_quad_f32(y, sbyte);
    *reinterpret_cast<uint32_t *>(codes + row * (g.d / 2) + (int64_t)j * 16 + sub * 4) = packed;
    if (sub == 0) scales[row * g.nblk + j] = (uint8_t)sbyte;
}

// bf16 input, quad layout: SmoothQuant (T = diag(inv_scale)) or the Kronecker
// transform (shear form, or the general stages for blocks that do not admit
// it). Quantize-only runs on the flat tiles of kq_flat.hip.
template <int MODE, int YOUT, int U, bool NT, int MAP, bool PRE>
__global__ __launch_bounds__(kThreads) void bf16_quad_kernel(
    const uint16_t *__restrict__ A, Geom g, const float *__restrict__ params,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, void *__restrict__ ydbg) {
    static_assert(MODE == kSmooth || MODE == kKron, "quantize-only runs on the flat kernel");
    int j, sub;
    int64_t row0;
    lane_coords<MAP>(g, j, sub, row0);
    const int64_t c0 = (int64_t)j * 32 + sub * 8;
    uint4 q[U];

    if (MODE == kSmooth) {
        float sq[8];
        const float4 a = *reinterpret_cast<const float4 *>(params + c0);
        const float4 b = *reinterpret_cast<const float4 *>(params + c0 + 4);
        sq[0] = a.x; sq[1] = a.y; sq[2] = a.z; sq[3] = a.w;
        sq[4] = b.x; sq[5] = b.y; sq[6] = b.z; sq[7] = b.w;
        for_rows<U, NT>(g, A, row0, c0, q, false, [&](const uint4 &x, int64_t row) {
            float y[8];
            widen8(x, y);
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = y[i] * sq[i];
            finish_f32<YOUT>(y, g, row, j, sub, c0, codes, scales, ydbg);
        });
    } else {
        // Per-block setup is shared through LDS when the workgroup's first row
        // of quads holds all its blocks (strip mapping): those quads (wave 0
        // for CB = 16) derive the shear coefficients, everyone reads them back.
        // With PRE the first rows' loads are in flight during the setup.
        ShearLane S;
        if (MAP == kStrip) {
            __shared__ ShearLane lds[64];
            const int quad = threadIdx.x >> 2;
            const bool setter = (quad >> g.cb_log2) == 0;
            float f[20];
            if (setter) load_factors20(params + (int64_t)j * 20, f);
            if (PRE && row0 < g.m) load_rows<U, NT>(g, A, row0, c0, 0, q);
            if (setter) shear_lane_setup(f, sub, lds[threadIdx.x]);
            __syncthreads();
            S = lds[((quad & ((1 << g.cb_log2) - 1)) << 2) | sub];
        } else {
            float f[20];
            load_factors20(params + (int64_t)j * 20, f);
            if (PRE && row0 < g.m) load_rows<U, NT>(g, A, row0, c0, 0, q);
            shear_lane_setup(f, sub, S);
        }
        if (S.ok) {  // one block per quad: uniform within the quad
            for_rows<U, NT>(g, A, row0, c0, q, PRE, [&](const uint4 &x, int64_t row) {
                float y[8];
                widen8(x, y);
                shear_apply8(y, S);
                finish_f32<YOUT>(y, g, row, j, sub, c0, codes, scales, ydbg);
            });
        } else {
            float f[20];
            load_factors20(params + (int64_t)j * 20, f);
            KronLane L;
            kron_lane_setup(f, sub, L);
            for_rows<U, NT>(g, A, row0, c0, q, PRE, [&](const uint4 &x, int64_t row) {
                float y[8];
                widen8(x, y);
                kron_apply8(y, L);
                finish_f32<YOUT>(y, g, row, j, sub, c0, codes, scales, ydbg);
            });
        }
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
__global__ __launch_bounds__(kThreads) void kron_mfma_lds_kernel(
    const uint16_t *__restrict__ A, LGeom g, const float *__restrict__ factors,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ ydbg) {
    __shared__ uint4 xs[2][16][65];
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

    uint4 v[4];
    if (tile0 * 16 >= g.m) return;  // uniform within the workgroup
    load_tile(tile0, v);
    store_tile(0, v);
    __syncthreads();
    for (int it = 0; it < g.iters; ++it) {
        const int64_t t = tile0 + it;
        if (t * 16 >= g.m) break;  // uniform within the workgroup
        const bool more = it + 1 < g.iters && (t + 1) * 16 < g.m;
        if (more) load_tile(t + 1, v);
        const int buf = it & 1;
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
        if (more) store_tile(buf ^ 1, v);
        __syncthreads();
    }
}

// fp32 input, quad layout: quantize (MODE kQuantOnly) or, with MODE kKron,
// write X . (K^(j))^{-T} (the weight fold) to `out` instead of quantizing.
template <int MODE>
__global__ __launch_bounds__(kThreads) void f32_kernel(
    const float *__restrict__ X, Geom g, const float *__restrict__ factors,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ out) {
    int j, sub;
    int64_t row0;
    lane_coords<kFlat>(g, j, sub, row0);
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

int pick_cb_log2(int64_t nblk, int max_log2) {
    for (int l = max_log2; l > 0; --l)
        if (nblk % (1 << l) == 0) return l;
    return 0;
}

// kFlat: about `target_wg` workgroups (fewer if the matrix is small), a multiple
// of nblk / gcd(64, nblk) so that 64 * gridDim.x is a multiple of nblk.
// `iters` (sweeps per workgroup) is rounded up to a multiple of `unroll`.
bool make_geom_flat(int64_t m, int64_t d, int64_t ld, int unroll, int64_t target_wg, kq::Geom &g,
                    unsigned &nwg) {
    g.m = m;
    g.d = d;
    g.lda = ld;
    g.nblk = (int)(d / 32);
    g.cb_log2 = 0;
    g.ncg = 1;
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

// kStrip: column groups of CB blocks (the largest power of two <= 2^max_cb_log2
// dividing nblk), row tiles of R = 64 / CB rows, `iters_per_wg` row tiles per
// workgroup (rounded up to a multiple of `unroll`).
bool make_geom_strip(int64_t m, int64_t d, int64_t ld, int unroll, int64_t iters_per_wg, kq::Geom &g,
                     unsigned &nwg, int max_cb_log2 = 4) {
    g.m = m;
    g.d = d;
    g.lda = ld;
    g.nblk = (int)(d / 32);
    g.cb_log2 = pick_cb_log2(g.nblk, max_cb_log2);
    g.ncg = g.nblk >> g.cb_log2;
    g.rstep = 64 >> g.cb_log2;
    const int64_t row_tiles = (m + g.rstep - 1) / g.rstep;
    int64_t iters = iters_per_wg < 1 ? 1 : iters_per_wg;
    iters = (iters + unroll - 1) / unroll * unroll;
    if (iters > row_tiles) iters = (row_tiles + unroll - 1) / unroll * unroll;
    const int64_t nslab = (row_tiles + iters - 1) / iters;
    const int64_t total = nslab * g.ncg;
    if (total > 0x7FFFFFFF || iters > 0x7FFFFFFF) return false;
    g.iters = (int)iters;
    nwg = (unsigned)total;
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

// Launch shape of the bf16 quad kernels: column strips of 16 blocks, row tiles
// of 4 rows, non-temporal loads. Workgroups are kept short, which the HBM
// system rewards: SmoothQuant walks 2 row tiles (both loads in flight), the
// transform 8 row tiles, 4 at a time (its per-block setup is amortized over
// more rows, and the first 4 rows' loads are issued before the setup). Chosen
// by sweeping tile counts, unroll depth, prefetching and the strip, flat and
// column-per-wave mappings on the 18432 x 3072 and 18432 x 12288 shapes.
template <int MODE, int YOUT>
kq_status launch_quad(const uint16_t *A, int64_t m, int64_t d, int64_t lda, const float *params,
                      uint8_t *codes, uint8_t *scales, void *ydbg, kq_stream_t stream) {
    kq::Geom g;
    unsigned nwg;
    if (MODE == kq::kKron) {
        // 8 row tiles per workgroup, 4 rows' loads at a time; when that leaves
        // fewer than 1024 workgroups (4 per CU), 2 row tiles of 2 rows instead:
        // small inputs need the parallelism more than the amortized setup.
        if (!make_geom_strip(m, d, lda, 4, 8, g, nwg)) return KQ_ERR_SHAPE;
        if (nwg >= 1024) {
            hipLaunchKernelGGL((kq::bf16_quad_kernel<MODE, YOUT, 4, true, kq::kStrip, true>), dim3(nwg),
                               dim3(kq::kThreads), 0, (hipStream_t)stream, A, g, params, codes, scales, ydbg);
            return launched();
        }
        if (!make_geom_strip(m, d, lda, 2, 2, g, nwg)) return KQ_ERR_SHAPE;
        hipLaunchKernelGGL((kq::bf16_quad_kernel<MODE, YOUT, 2, true, kq::kStrip, true>), dim3(nwg),
                           dim3(kq::kThreads), 0, (hipStream_t)stream, A, g, params, codes, scales, ydbg);
        return launched();
    }
    if (!make_geom_strip(m, d, lda, 2, 2, g, nwg)) return KQ_ERR_SHAPE;
    hipLaunchKernelGGL((kq::bf16_quad_kernel<MODE, YOUT, 2, true, kq::kStrip, false>), dim3(nwg),
                       dim3(kq::kThreads), 0, (hipStream_t)stream, A, g, params, codes, scales, ydbg);
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

// LDS-staged MFMA form: strips of 16 blocks (nblk % 16 == 0), `iters` tiles of
// 16 tokens per workgroup.
bool make_lgeom(int64_t m, int64_t d, int64_t lda, int64_t iters_per_wg, kq::LGeom &g, unsigned &nwg) {
    g.m = m;
    g.d = d;
    g.lda = lda;
    g.nblk = (int)(d / 32);
    if (g.nblk % 16 != 0) return false;
    g.nstrip = g.nblk / 16;
    const int64_t tiles = (m + 15) / 16;
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
    if (!make_lgeom(m, d, lda, 8, g, nwg)) return KQ_ERR_SHAPE;
    hipLaunchKernelGGL((kq::kron_mfma_lds_kernel<DEBUG>), dim3(nwg), dim3(kq::kThreads), 0,
                       (hipStream_t)stream, A, g, factors, codes, scales, ydbg);
    return launched();
}

// Which form of the transform the fused entry point runs (KQ_TRANSFORM_FORM,
// read at every call): "butterfly" = five in-register 2x2 stages in shear
// form (default); "mfma" = the materialized 32x32 block on MFMA, operands
// loaded directly; "mfma_lds" = the same through LDS-staged row-major tiles
// (needs d a multiple of 512, else the butterfly runs).
enum Form { kFormButterfly, kFormMfma, kFormMfmaLds };
Form transform_form() {
    const char *v = getenv("KQ_TRANSFORM_FORM");
    if (v && strcmp(v, "mfma") == 0) return kFormMfma;
    if (v && strcmp(v, "mfma_lds") == 0) return kFormMfmaLds;
    return kFormButterfly;
}

template <bool DEBUG>
kq_status launch_fused(const uint16_t *A, int64_t m, int64_t d, int64_t lda, const float *factors,
                       uint8_t *codes, uint8_t *scales, float *ydbg, kq_stream_t stream) {
    const Form f = transform_form();
    if (f == kFormMfmaLds && (d / 32) % 16 == 0)
        return launch_mfma_lds<DEBUG>(A, m, d, lda, factors, codes, scales, ydbg, stream);
    if (f != kFormMfma)
        return launch_quad<kq::kKron, DEBUG ? kq::kYF32 : kq::kYNone>(A, m, d, lda, factors, codes, scales, ydbg,
                                                                       stream);
    if ((d / 32) % 2 == 0)
        return launch_mfma<2, DEBUG>(A, m, d, lda, factors, codes, scales, ydbg, stream);
    return launch_mfma<1, DEBUG>(A, m, d, lda, factors, codes, scales, ydbg, stream);
}

}  // namespace

extern "C" {

kq_status kq_transform_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                      const float *factors, uint8_t *codes, uint8_t *scales,
                                      float *y_debug, kq_stream_t stream) {
    kq_status s = check_shape(m, d, lda);
    if (s != KQ_OK) return s;
    if (m == 0 || d == 0) return KQ_OK;
    if ((s = check_bf16_io(A, lda, codes, scales)) != KQ_OK) return s;
    if (!factors) return KQ_ERR_NULL;
    if (!aligned(factors, 16) || (y_debug && !aligned(y_debug, 16))) return KQ_ERR_ALIGN;
    if (y_debug) return launch_fused<true>(A, m, d, lda, factors, codes, scales, y_debug, stream);
    return launch_fused<false>(A, m, d, lda, factors, codes, scales, nullptr, stream);
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
    return launch_quad<kq::kKron, kq::kYBF16>(A, m, d, lda, factors, codes, scales, y16, stream);
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
    return launch_quad<kq::kSmooth, kq::kYNone>(A, m, d, lda, inv_scale, codes, scales, nullptr, stream);
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
