// Flat-tile kernels on gfx950: quantize-only MXFP4, and the block-Hadamard
// transform + MXFP4 (the fixed-rotation baselines of KroQuant, arXiv
// 2607.21446v1 -- Sec. 1 and Table 2: Hadamard at block size 32; Sec. 4.4 /
// Table 3: the fast Walsh-Hadamard transform over the full power-of-two
// width).
//
// Flat tiles. The matrix is walked as its flattened rows (element E = row d +
// col, which is also the element's index in the contiguous [m][d] outputs).
// A wave owns a tile of WT = 512 R elements: lane t holds R chunks of 8
// consecutive elements, chunk j at tile offset 512 j + 8 t (16-byte loads; a
// wave-wide load covers 1 KB and the R loads of a wave 512 R contiguous
// elements, all issued at once). Offset bits 0-2 are in-register, bits 3-8
// the lane bits, bits 9.. the chunk index; each quad holds one 32-element
// block. With nothing per column to fetch, quantize-only streams best this way
// (one load phase per wave, workgroups covering 16 KB of contiguous input).
//
// Block Hadamard: for every row and every group of n consecutive channels
// (n = 2^LOGN, 32 <= n <= 16384) y = x . H_n / sqrt(n), H_n the Sylvester
// matrix (Sec. 3.2 "Hadamard initialization": the k-fold Kronecker power of
// [[1,1],[1,-1]]/sqrt(2)), computed in fp32 and quantized to MXFP4 exactly as
// the fused Kronecker kernel does. Group row q = row (d / n) + group holds
// channels c < n, E = q n + c.
//
// Butterflies in signed form. A stage on channel bit b maps each pair
// (x0, x1) that differs in bit b to (x0 + x1, x1 - x0): [[1,1],[1,-1]]
// followed by negating the second output. Each element then becomes its own
// value plus +-1 times its partner's -- one add, or one fmac with the partner
// read through DPP -- and by the Kronecker mixed-product rule the negations
// collect into (-1)^popcount(c) for output channel c, which the final
// multiply by +-1/sqrt(n) removes.
//
// Where each channel bit's stage runs:
//   0-2          in-register pairs;
//   3, 4         DPP quad permutes (lane xor 1, xor 2);
//   5            ds_swizzle (lane xor 4 inside 32 lanes);
//   6            DPP row rotate by 8 (lane xor 8 inside 16 lanes);
//   7, 8         v_permlane16_swap / v_permlane32_swap trade lane bit 4 / 5
//                for chunk bit 0, then in-register pairs;
//   9 .. 8+log2R chunk pairs in registers (before the swaps);
//   12, 13       n = 8192 / 16384 spans 2 / 4 waves: one LDS exchange trades
//                those wave bits for chunk bits, then in-register pairs.
// The swaps and the exchange change which elements a chunk holds, never the
// shape: each lane still has 8 consecutive channels per chunk and each quad
// one 32-channel block, so the quad quantizer applies and only the store
// addresses follow the new assignment.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"
#include "kq_device.hpp"
#include "kq_host.hpp"

namespace kq {

struct HGeom {
    int64_t total;     // elements of all group rows: m * d
    int64_t lda;       // row stride of A (elements)
    uint32_t G;        // groups per row, d / n
    int contig;        // lda == d: element E is at A + E
    float inv_sqrt_n;  // fl32(1 / sqrt(n))
};

// (x0, x1) -> (x0 + x1, x1 - x0)
__device__ __forceinline__ void hpair(float &a, float &b) {
    const float s = a + b;
    b = b - a;
    a = s;
}

template <int S>
__device__ __forceinline__ void hstage8(float x[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (!(i & S)) hpair(x[i], x[i + S]);
}

// x[i] += c * x[i] of lane ^ 8 (a row rotate by 8 is the xor-8 permutation).
__device__ __forceinline__ void fmac_partner_xor8(float x[8], float c) { KQ_FMAC_DPP8("row_ror:8"); }

// x[i] += c * x[i] of lane ^ 4: ds_swizzle in bit-mask mode (and 0x1F, or 0, xor 4).
__device__ __forceinline__ void fmac_partner_xor4(float x[8], float c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float p = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x[i]), 0x101F));
        x[i] = fmaf(p, c, x[i]);
    }
}

// Row swap: afterwards a holds what was (chunk bit 0, lane bit 4) = (lane bit 4, 0)
// and b what was (lane bit 4, 1), i.e. lane bit 4 and the a/b choice trade places.
__device__ __forceinline__ void swap16(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// The same for lane bit 5 (half-wave swap).
__device__ __forceinline__ void swap32(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

template <int LOGN>
struct HShape {
    static constexpr int LOGR = LOGN <= 11 ? 2 : 3;  // chunks per lane: 4 or 8
    static constexpr int R = 1 << LOGR;
    static constexpr int LOGWT = 9 + LOGR;           // wave tile: 2048 or 4096 elements
    static constexpr int LOGP = LOGN > LOGWT ? LOGN - LOGWT : 0;  // log2 waves per group row
};

template <int LOGN, bool DEBUG>
__global__ __launch_bounds__(256) void hadamard_kernel(const uint16_t *__restrict__ A, HGeom g,
                                                       uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales,
                                                       float *__restrict__ ydbg) {
    using H = HShape<LOGN>;
    constexpr int R = H::R;
    constexpr int64_t WT = (int64_t)1 << H::LOGWT;
    constexpr int64_t NMASK = ((int64_t)1 << LOGN) - 1;
    // the wave index is the same in every lane; saying so keeps the tile
    // arithmetic on the scalar unit
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tbase = ((int64_t)blockIdx.x * 4 + wave) * WT;

    float x[R][8];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t E = tbase + 512 * j + 8 * lane;
        uint4 q = make_uint4(0, 0, 0, 0);
        if (E < g.total) {
            const uint16_t *p;
            if (g.contig) {
                p = A + E;
            } else {
                const uint32_t gq = (uint32_t)(E >> LOGN);
                const uint32_t row = gq / g.G;
                p = A + (int64_t)row * g.lda + ((int64_t)(gq - row * g.G) << LOGN) + (E & NMASK);
            }
            q = load_stream(reinterpret_cast<const uint4 *>(p), true);
        }
        widen8(q, x[j]);
    }

    // channel bits 0-2, then the chunk bits that are channel bits (9 ..)
#pragma unroll
    for (int j = 0; j < R; ++j) {
        hstage8<1>(x[j]);
        hstage8<2>(x[j]);
        hstage8<4>(x[j]);
    }
#pragma unroll
    for (int jb = 0; jb < H::LOGR; ++jb) {
        if (9 + jb >= LOGN) break;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (j & (1 << jb)) continue;
#pragma unroll
            for (int i = 0; i < 8; ++i) hpair(x[j][i], x[j | (1 << jb)][i]);
        }
    }

    // channel bits 3-6: partner lanes
    {
        const float c1 = (lane & 1) ? -1.0f : 1.0f, c2 = (lane & 2) ? -1.0f : 1.0f;
        const float c4 = (lane & 4) ? -1.0f : 1.0f, c8 = (lane & 8) ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            fmac_partner_xor1(x[j], c1);
            fmac_partner_xor2(x[j], c2);
            if (LOGN > 5) fmac_partner_xor4(x[j], c4);
            if (LOGN > 6) fmac_partner_xor8(x[j], c8);
        }
    }
    // channel bits 7 and 8: into chunk bit 0, then in-register
    if (LOGN > 7) {
#pragma unroll
        for (int j = 0; j < R; j += 2)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                swap16(x[j][i], x[j + 1][i]);
                hpair(x[j][i], x[j + 1][i]);
            }
    }
    if (LOGN > 8) {
#pragma unroll
        for (int j = 0; j < R; j += 2)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                swap32(x[j][i], x[j + 1][i]);
                hpair(x[j][i], x[j + 1][i]);
            }
    }

    // channel bits 12 (and 13): the waves of a group row trade them for chunk
    // bits through LDS, in two rounds (chunk bit 0 = 0, then 1; 32 KB).
    if constexpr (H::LOGP > 0) {
        __shared__ float xs[4][4][8][64];  // [wave][slot][i][lane]: lane-contiguous, conflict-free
#pragma unroll
        for (int r = 0; r < 2; ++r) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 8; ++i) xs[wave][s][i][lane] = x[r + 2 * s][i];
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                int srcw, slot;
                if (H::LOGP == 2) {  // new chunk bits 1-2 = source wave; new wave = old chunk bits 1-2
                    srcw = s;
                    slot = wave;
                } else {             // new chunk bit 2 = source wave of the pair; new wave = old chunk bit 2
                    srcw = (wave & ~1) | (s >> 1);
                    slot = (s & 1) | ((wave & 1) << 1);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) x[r + 2 * s][i] = xs[srcw][slot][i][lane];
            }
            __syncthreads();
        }
#pragma unroll
        for (int jb = 3 - H::LOGP; jb < 3; ++jb)
#pragma unroll
            for (int j = 0; j < R; ++j) {
                if (j & (1 << jb)) continue;
#pragma unroll
                for (int i = 0; i < 8; ++i) hpair(x[j][i], x[j | (1 << jb)][i]);
            }
    }

    // Where each chunk's elements sit (undo the exchange, then the swaps),
    // the sign (-1)^popcount(c) and 1/sqrt(n), quantize, store.
    int64_t sbase = tbase;
    if (H::LOGP == 1) sbase = ((int64_t)blockIdx.x * 4 + (wave & ~1)) * WT;
    if (H::LOGP == 2) sbase = (int64_t)blockIdx.x * 4 * WT;
    const int sub = lane & 3;
#pragma unroll
    for (int jj = 0; jj < R; ++jj) {
        int j_b = jj, p_b = 0, l_b = lane;
        if (H::LOGP == 1) {
            j_b = (jj & 3) | ((wave & 1) << 2);
            p_b = (jj >> 2) & 1;
        } else if (H::LOGP == 2) {
            j_b = (jj & 1) | (wave << 1);
            p_b = (jj >> 1) & 3;
        }
        if (LOGN > 8) {
            const int c0 = j_b & 1;
            j_b = (j_b & ~1) | ((l_b >> 5) & 1);
            l_b = (l_b & ~32) | (c0 << 5);
        }
        if (LOGN > 7) {
            const int c0 = j_b & 1;
            j_b = (j_b & ~1) | ((l_b >> 4) & 1);
            l_b = (l_b & ~16) | (c0 << 4);
        }
        const int64_t E = sbase + (int64_t)p_b * WT + 512 * j_b + 8 * l_b;
        const float sp = (__popcll((uint64_t)(E & NMASK)) & 1) ? -g.inv_sqrt_n : g.inv_sqrt_n;
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = x[jj][i] * ((__builtin_popcount(i) & 1) ? -sp : sp);
        uint32_t sbyte;
        const uint32_t packed = quantize_quad_f32(y, sbyte);
        if (E < g.total) {
            if (DEBUG) {
                float4 *o = reinterpret_cast<float4 *>(ydbg + E);
                o[0] = make_float4(y[0], y[1], y[2], y[3]);
                o[1] = make_float4(y[4], y[5], y[6], y[7]);
            }
            *reinterpret_cast<uint32_t *>(codes + (E >> 1)) = packed;
            if (sub == 0) scales[E >> 5] = (uint8_t)sbyte;
        }
    }
}

// Quantize-only on flat tiles (R = 4). Rows may be padded (lda > d): then the
// row of a chunk is its 32-block index divided by d / 32.
__global__ __launch_bounds__(256) void flat_quantize_kernel(const uint16_t *__restrict__ A, HGeom g,
                                                            uint8_t *__restrict__ codes,
                                                            uint8_t *__restrict__ scales) {
    constexpr int R = 4;
    constexpr int64_t WT = 512 * R;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tbase = ((int64_t)blockIdx.x * 4 + wave) * WT;
    uint4 q[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t E = tbase + 512 * j + 8 * lane;
        q[j] = make_uint4(0, 0, 0, 0);
        if (E < g.total) {
            const uint16_t *p;
            if (g.contig) {
                p = A + E;
            } else {
                const uint32_t blk = (uint32_t)(E >> 5);
                const uint32_t row = blk / g.G;
                p = A + (int64_t)row * g.lda + ((int64_t)(blk - row * g.G) << 5) + (E & 31);
            }
            q[j] = load_stream(reinterpret_cast<const uint4 *>(p), true);
        }
    }
    const int sub = lane & 3;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t E = tbase + 512 * j + 8 * lane;
        uint32_t sbyte;
        const uint32_t packed = quantize_quad_bf16(q[j], sbyte);
        if (E < g.total) {
            *reinterpret_cast<uint32_t *>(codes + (E >> 1)) = packed;
            if (sub == 0) scales[E >> 5] = (uint8_t)sbyte;
        }
    }
}

}  // namespace kq

namespace {

template <int LOGN, bool DEBUG>
kq_status launch_hadamard(const uint16_t *A, const kq::HGeom &g, uint8_t *codes, uint8_t *scales,
                          float *ydbg, kq_stream_t stream) {
    constexpr int64_t WT = (int64_t)1 << kq::HShape<LOGN>::LOGWT;
    const int64_t tiles = (g.total + WT - 1) / WT;
    const int64_t nwg = (tiles + 3) / 4;
    if (nwg > 0x7FFFFFFF) return KQ_ERR_SHAPE;
    hipLaunchKernelGGL((kq::hadamard_kernel<LOGN, DEBUG>), dim3((unsigned)nwg), dim3(256), 0,
                       (hipStream_t)stream, A, g, codes, scales, ydbg);
    return kqhost::launched();
}

template <bool DEBUG>
kq_status dispatch_hadamard(int logn, const uint16_t *A, const kq::HGeom &g, uint8_t *codes,
                            uint8_t *scales, float *ydbg, kq_stream_t stream) {
    switch (logn) {
        case 5: return launch_hadamard<5, DEBUG>(A, g, codes, scales, ydbg, stream);
        case 6: return launch_hadamard<6, DEBUG>(A, g, codes, scales, ydbg, stream);
        case 7: return launch_hadamard<7, DEBUG>(A, g, codes, scales, ydbg, stream);
        case 8: return launch_hadamard<8, DEBUG>(A, g, codes, scales, ydbg, stream);
        case 9: return launch_hadamard<9, DEBUG>(A, g, codes, scales, ydbg, stream);
        case 10: return launch_hadamard<10, DEBUG>(A, g, codes, scales, ydbg, stream);
        case 11: return launch_hadamard<11, DEBUG>(A, g, codes, scales, ydbg, stream);
        case 12: return launch_hadamard<12, DEBUG>(A, g, codes, scales, ydbg, stream);
        case 13: return launch_hadamard<13, DEBUG>(A, g, codes, scales, ydbg, stream);
        case 14: return launch_hadamard<14, DEBUG>(A, g, codes, scales, ydbg, stream);
    }
    return KQ_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

kq_status kq_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda, uint8_t *codes,
                            uint8_t *scales, kq_stream_t stream) {
    kq_status s = kqhost::check_shape(m, d, lda);
    if (s != KQ_OK) return s;
    if (m == 0 || d == 0) return KQ_OK;
    if ((s = kqhost::check_bf16_io(A, lda, codes, scales)) != KQ_OK) return s;
    if (m > (int64_t)0xFFFFFFFF / (d / 32)) return KQ_ERR_UNSUPPORTED;  // block index in 32 bits
    kq::HGeom g;
    g.total = m * d;
    g.lda = lda;
    g.G = (uint32_t)(d / 32);
    g.contig = lda == d;
    g.inv_sqrt_n = 1.0f;
    const int64_t nwg = ((g.total + 2047) / 2048 + 3) / 4;
    if (nwg > 0x7FFFFFFF) return KQ_ERR_SHAPE;
    hipLaunchKernelGGL(kq::flat_quantize_kernel, dim3((unsigned)nwg), dim3(256), 0, (hipStream_t)stream, A, g,
                       codes, scales);
    return kqhost::launched();
}

kq_status kq_hadamard_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda, int64_t n,
                                     uint8_t *codes, uint8_t *scales, float *y_debug,
                                     kq_stream_t stream) {
    kq_status s = kqhost::check_shape(m, d, lda);
    if (s != KQ_OK) return s;
    if (n < 32 || (n & (n - 1)) != 0) return KQ_ERR_SHAPE;
    if (n > 16384) return KQ_ERR_UNSUPPORTED;
    if (d % n != 0) return KQ_ERR_SHAPE;
    if (m == 0 || d == 0) return KQ_OK;
    if ((s = kqhost::check_bf16_io(A, lda, codes, scales)) != KQ_OK) return s;
    if (y_debug && !kqhost::aligned(y_debug, 16)) return KQ_ERR_ALIGN;
    if (m > (int64_t)0xFFFFFFFF / (d / n)) return KQ_ERR_UNSUPPORTED;  // group rows index in 32 bits
    int logn = 0;
    while (((int64_t)1 << logn) < n) ++logn;
    kq::HGeom g;
    g.total = m * d;
    g.lda = lda;
    g.G = (uint32_t)(d / n);
    g.contig = lda == d;
    g.inv_sqrt_n = (float)(1.0 / __builtin_sqrt((double)n));
    if (y_debug) return dispatch_hadamard<true>(logn, A, g, codes, scales, y_debug, stream);
    return dispatch_hadamard<false>(logn, A, g, codes, scales, nullptr, stream);
}

}  // extern "C"
