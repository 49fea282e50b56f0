// MXFP4 matrix products on gfx950 scaled FP4 matrix instructions: the W4A4
// GEMM of Eq. 2 (KroQuant, arXiv 2607.21446v1), optionally with the low-rank
// term of Sec. 3.4 Eq. 11 added in its epilogue, and that term's projection of
// the 16-bit activations onto Q(R).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"
#include "kq_cvt.hpp"
#include "kq_device.hpp"
#include "kq_host.hpp"

namespace kq {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Low-rank branch helpers (Eq. 11's A T R^T L^T with MXFP4 L and R)
// ---------------------------------------------------------------------------

// MXFP4 -> bf16, exact (see decode_fp4x8_bf16_cvt): one thread per 8 codes.
__global__ __launch_bounds__(kThreads) void dequantize_bf16_kernel(const uint32_t *__restrict__ codes,
                                                                   const uint8_t *__restrict__ scales, int64_t n8,
                                                                   bf16x8_t *__restrict__ out) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x)
        out[i] = decode_fp4x8_bf16_cvt(codes[i], scales[i / 4]);
}

// Z = X Q(R)^T: X bf16 [m][ldx] (the branch's 16-bit activations), R MXFP4
// [r][d] (codes [r][d/2], scales [r][d/32]), Z fp32 [m][r]. A workgroup
// computes 64 rows x 128 columns of Z, each wave 16 rows x 128 columns (8 MFMA
// tiles), walking d in steps of 128 with v_mfma_f32_16x16x32_bf16 (four k
// sub-steps of 32 per step): lane l supplies row l % 16 and k = 8 (l / 16) .. +7
// of each sub-step of X (four 16-byte loads, fetched one step ahead) and of the
// decoded R column; it receives rows 4 (l / 16) + t, column l % 16. The
// workgroup decodes each step's 128 x 128 slice of R once into LDS (thread t:
// column t / 2, 64 k), double-buffered, one barrier per step; staged columns are
// padded by 16 bytes so operand reads hit distinct banks. d must be a multiple
// of 32; a step past d reads zero codes.
struct ProjGeom {
    int64_t m, d, ldx, r, tiles_r;
};

constexpr int kProjAhead = 3;  // steps of X in flight per wave

// Z = X R16^T with R in bf16 [r][d] (or MXFP4, decoded by the producers; RMX
// below): per output element the 16 x 16 x 32 bf16 matrix instruction over 32 k
// at a time in ascending k, with the work split by wave. A workgroup covers 80 rows of
// X (18432 rows make 231 workgroups, one round on 256 CUs; 64-row tiles left a
// second round of 32): waves 0-4 own 16 rows each and stream them, kProjAhead
// steps ahead in registers, so their memory waits are for their own X loads
// alone; waves 5 and 6 move each step's 128 x 128 slice of R (L2-resident)
// straight into LDS, 16 loads of 1 KB each, two steps ahead of the one being
// read. LDS holds three slices of 32 KB, columns of 256 bytes with their 16-byte
// chunks permuted (chunk q of column c at slot q ^ (c % 16)), so the 16 columns
// a matrix read touches fall in distinct banks and one direct-to-LDS load (4
// columns, 1 KB) stays contiguous. Measured on 18432 x 3072, r = 128: 39 us,
// against 91 us with one producer wave, one step ahead and 64-row tiles.
// Timing variants (outputs wrong, same launch): without the R and X loads 23
// us, without R 29 us, without X 24 us; with a third R slot and four X steps
// in flight, or with consumer waves of two 16-row groups (R fragments read once
// for 32 rows), unchanged or slower. The remaining floor is the in-CU work: the
// 16 x 16 x 32 instruction issues at half the rate of the 32 x 32 x 16 form on
// gfx950 (1.3 against 2.45 PFLOP/s measured), and two of the five consumer
// waves share a SIMD. A 32 x 32 x 16 form with 32-row waves and 128-row tiles
// ran at 83 us: its X loads cover 32 rows x 32 bytes per instruction, and the
// X stream alone cost 47 us there.
constexpr int kProjWaves = 5;                    // consumer waves, 16 rows each
constexpr int kProjRows = 16 * kProjWaves;       // rows of X per workgroup
constexpr int kProjProducers = 2;                // waves moving R into LDS
constexpr int kProjSlots = 3;                    // R slices in LDS
constexpr int kProjLoads = 32 / kProjProducers;  // 1 KB loads per producer per step
static_assert(kProjSlots == kProjAhead, "the consumers' slot index is their ring position");
__device__ __forceinline__ void proj_dma16(__amdgpu_buffer_rsrc_t d, uint32_t lds, uint32_t voff) {
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "s"(lds), "v"(voff), "s"(d)
        : "memory");
}

// SPLIT: Z leaves as its bf16 split, zh = bf16(z) and zl = bf16(z - zh) (both
// rounded to nearest even by the hardware convert; z - zh is exact in fp32),
// the operands the packed GEMM's low-rank term multiplies, in place of fp32 z.
//
// RMX: R arrives in MXFP4 (codes [r][d/2] at r16's place, scales [r][d/32] at
// sr) and the producers decode it: producer lane c (0 .. 127, one column of the
// tile) loads its column's 64 code bytes and 4 scale bytes of a step two steps
// ahead into registers, and writes the step after the current one into its LDS
// slot as bf16 (the same values as kq_dequantize_mxfp4_bf16, the same layout as
// the bf16 loads), a quarter of the bf16 form's bytes from L2. Consumers as above:
// bit-identical Z.
template <bool SPLIT, bool RMX = false>
__global__ __launch_bounds__(64 * (kProjWaves + kProjProducers)) void lowrank_project_r16_kernel(
    const uint16_t *__restrict__ X, ProjGeom g, const uint16_t *__restrict__ r16, float *__restrict__ Z,
    uint16_t *__restrict__ Zh, uint16_t *__restrict__ Zl, const uint8_t *__restrict__ sr = nullptr) {
    __shared__ __attribute__((aligned(16))) uint8_t rl[kProjSlots][128 * 256];
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t tm = blockIdx.x / g.tiles_r, tr = blockIdx.x % g.tiles_r;
    const int64_t col0 = tr * 128;
    const int64_t steps = (g.d + 127) / 128;
    // a step past d loads zeros (X and R): its products add exact zeros
    const int64_t steps_up = (steps + kProjAhead - 1) / kProjAhead * kProjAhead;
    const uint32_t lds0 = (uint32_t)(uintptr_t)&rl[0][0];
    constexpr int kAhead = kProjSlots - 1;  // R steps in flight beyond the one being read

    if (RMX && wave >= kProjWaves) {
        const int c = 64 * (wave - kProjWaves) + lane;  // the lane's column of the tile
        const int64_t rows_r = g.r - col0 < 128 ? g.r - col0 : 128;
        const uint8_t *cr = reinterpret_cast<const uint8_t *>(r16);
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(cr + col0 * (g.d / 2)), (short)0, (int)(rows_r * (g.d / 2)), 0x00020000);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(sr + col0 * (g.d / 32)), (short)0, (int)(rows_r * (g.d / 32)), 0x00020000);
        struct RStep {
            uint4 q[4];
            uint32_t sc[4];
        };
        // step st's four 32-k groups of column c; a group past d reads zeros (offset
        // beyond every record count), so it decodes to exact zeros
        auto fetch = [&](int64_t st, RStep &R) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int64_t k = st * 128 + 32 * h;
                const bool in = k < g.d;
                const uint32_t co = in ? (uint32_t)(c * (g.d / 2) + k / 2) : 0x80000000u;
                const uint32_t so = in ? (uint32_t)(c * (g.d / 32) + k / 32) : 0x80000000u;
                const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 0);
                R.q[h] = make_uint4(v[0], v[1], v[2], v[3]);
                R.sc[h] = __builtin_amdgcn_raw_buffer_load_b8(rs, so, 0, 0);
            }
        };
        // chunk q (8 values of k, 16 bytes) of column c at slot q ^ (c % 16)
        auto stash = [&](int64_t st, const RStep &R) {
            uint8_t *col = &rl[st % kProjSlots][0] + c * 256;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t w4[4] = {R.q[h].x, R.q[h].y, R.q[h].z, R.q[h].w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<bf16x8_t *>(col + 16 * ((4 * h + i) ^ (c & 15))) =
                        decode_fp4x8_bf16_cvt(w4[i], R.sc[h]);
            }
        };
        // step st + 1 is written during step st (its slot held step st - 2, read before
        // the barrier that opened step st - 1), with its loads issued two steps earlier
        RStep ring[2];
        fetch(0, ring[0]);
        if (1 < steps_up) fetch(1, ring[1]);
        stash(0, ring[0]);
        if (2 < steps_up) fetch(2, ring[0]);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int64_t st0 = 0; st0 < steps_up; st0 += 2) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int64_t st = st0 + p;
                if (st < steps_up) {
                    if (st + 1 < steps_up) {
                        stash(st + 1, ring[(p + 1) & 1]);
                        if (st + 3 < steps_up) fetch(st + 3, ring[(p + 1) & 1]);
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                }
            }
        }
        return;
    }
    if (wave >= kProjWaves) {
        // producer pi: loads j = kProjLoads pi .. of each step; load j covers columns 4 j .. 4 j + 3
        const int pi = wave - kProjWaves;
        const int64_t rows_r = g.r - col0 < 128 ? g.r - col0 : 128;
        const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(r16 + col0 * g.d), (short)0, (int)(rows_r * g.d * 2), 0x00020000);
        const int p = lane & 15;
        auto issue = [&](int64_t st) {
            const uint32_t buf = lds0 + (uint32_t)((st % kProjSlots) * 128 * 256);
#pragma unroll
            for (int jj = 0; jj < kProjLoads; ++jj) {
                const int j = kProjLoads * pi + jj;
                const int c = 4 * j + (lane >> 4);
                const int q = p ^ (c & 15);
                const int64_t k = st * 128 + 8 * q;
                const uint32_t o = k < g.d ? (uint32_t)((c * g.d + k) * 2) : 0x80000000u;
                proj_dma16(rh, buf + 1024 * j, o);
            }
        };
        // wait for the oldest step in flight while the `younger` steps issued after
        // it (kProjLoads loads each) stay in flight, then the step's barrier
        auto wait_then_barrier = [&](int64_t younger) {
            if (younger >= 2) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kProjLoads) : "memory");
            else if (younger == 1) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kProjLoads) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        };
        static_assert(kAhead >= 1 && kAhead <= 3 && 2 * kProjLoads <= 63,
                      "wait_then_barrier covers at most two younger steps");
        for (int s = 0; s < kAhead; ++s)
            if (s < steps_up) issue(s);
        // the first step's slice must have landed; the later ones may still be in flight
        wait_then_barrier((kAhead < steps_up ? kAhead : steps_up) - 1);
        for (int64_t st = 0; st < steps_up; ++st) {
            // the slot of step st + kAhead held step st - 1, read before the last barrier
            if (st + kAhead < steps_up) issue(st + kAhead);
            wait_then_barrier((st + kAhead < steps_up ? st + kAhead : steps_up - 1) - (st + 1));
        }
        return;
    }

    // consumers: 16 rows each, all 128 columns of the tile (8 MFMA tiles)
    const int grp = lane >> 4;
    const int64_t rows_x = g.m - tm * kProjRows < kProjRows ? g.m - tm * kProjRows : kProjRows;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(X + tm * kProjRows * g.ldx), (short)0, (int)(rows_x * g.ldx * 2), 0x00020000);
    const uint32_t xoff = (uint32_t)(((wave * 16 + (lane & 15)) * g.ldx + 8 * grp) * 2);
    auto fetch_x = [&](int64_t k0, uint4 q[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t k = k0 + 32 * u + 8 * grp;
            const uint32_t xo = k < g.d ? xoff + (uint32_t)((k0 + 32 * u) * 2) : 0x80000000u;
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 2);
            q[u] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    floatx4_t acc[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    uint4 xq[kProjAhead][4];
#pragma unroll
    for (int p = 0; p < kProjAhead; ++p) fetch_x((int64_t)p * 128, xq[p]);
    asm volatile("s_barrier" ::: "memory");
    const int cl = lane & 15;
    for (int64_t st0 = 0; st0 < steps_up; st0 += kProjAhead) {
#pragma unroll
        for (int p = 0; p < kProjAhead; ++p) {
            const int64_t st = st0 + p;
            const uint8_t *buf = rl[p];  // slot st % kProjSlots
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bf16x8_t xa = as_bf16x8(xq[p][u]);
                const int q = 4 * u + grp;
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const bf16x8_t rb =
                        *reinterpret_cast<const bf16x8_t *>(buf + (b * 16 + cl) * 256 + 16 * (q ^ cl));
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, rb, acc[b], 0, 0, 0);
                }
            }
            fetch_x((st + kProjAhead) * 128, xq[p]);
            // done reading this slot (the producer refills it after the barrier)
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    }
    const int64_t orow0 = tm * kProjRows + wave * 16 + grp * 4;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int64_t col = col0 + b * 16 + cl;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int64_t orow = orow0 + tt;
            if (orow < g.m && col < g.r) {
                if (SPLIT) {
                    const __bf16 h = (__bf16)acc[b][tt];
                    const __bf16 l = (__bf16)(acc[b][tt] - (float)h);
                    Zh[orow * g.r + col] = __builtin_bit_cast(uint16_t, h);
                    Zl[orow * g.r + col] = __builtin_bit_cast(uint16_t, l);
                } else {
                    Z[orow * g.r + col] = acc[b][tt];
                }
            }
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
        // Low-rank term Z Q(L)^T into the same accumulators, 64 of r at a time:
        // the workgroup stages the tile's Z rows split as hi + lo bf16 (exact to
        // 2^-16 relative) in the free A buffers and its decoded L rows (exact in
        // bf16) in a B buffer, all loads issued at once (thread t: row or column
        // t / 2, 32 of r), then each wave runs two v_mfma_f32_16x16x32_bf16 per
        // tile pair and 32 of r from LDS. Rows 144 bytes apart, as above.
        static_assert(GemmStage<KS>::kRow >= 144, "staged rows must hold 64 bf16");
        constexpr int SR = GemmStage<KS>::kRow;
        uint8_t *zh_lds = a_lds[0], *zl_lds = a_lds[1], *l_lds = b_lds[0];
        const int t = threadIdx.x, sr_ = t >> 1, sh = t & 1;
        for (int64_t r0 = 0; r0 < g.r; r0 += 64) {
            const int64_t rc = r0 + 32 * sh;  // this thread's 32 of r
            float4 zv[8];
            const int64_t zrow = m0 + sr_;
#pragma unroll
            for (int q = 0; q < 8; ++q) zv[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (zrow < g.m && rc < g.r) {
                const float4 *p = reinterpret_cast<const float4 *>(Z + zrow * g.r + rc);
#pragma unroll
                for (int q = 0; q < 8; ++q) zv[q] = p[q];
            }
            const int64_t lrow = n0 + sr_;
            uint4 lc = make_uint4(0, 0, 0, 0);
            uint32_t ls = 127;
            if (lrow < g.n && rc < g.r) {
                lc = *reinterpret_cast<const uint4 *>(cl + lrow * (g.r / 2) + rc / 2);
                ls = sl[lrow * (g.r / 32) + rc / 32];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float z8[8] = {zv[2 * q].x, zv[2 * q].y, zv[2 * q].z, zv[2 * q].w,
                                     zv[2 * q + 1].x, zv[2 * q + 1].y, zv[2 * q + 1].z, zv[2 * q + 1].w};
                bf16x8_t h, l;
                split_bf16x8_cvt(z8, h, l);
                *reinterpret_cast<bf16x8_t *>(zh_lds + sr_ * SR + 64 * sh + 16 * q) = h;
                *reinterpret_cast<bf16x8_t *>(zl_lds + sr_ * SR + 64 * sh + 16 * q) = l;
            }
            const uint32_t lw[4] = {lc.x, lc.y, lc.z, lc.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<bf16x8_t *>(l_lds + sr_ * SR + 64 * sh + 16 * q) = decode_fp4x8_bf16_cvt(lw[q], ls);
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8_t lb[4];
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    lb[b] = *reinterpret_cast<const bf16x8_t *>(l_lds + (wc + b * 16 + r) * SR + 64 * kk + 16 * grp);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int off = (wr + a * 16 + r) * SR + 64 * kk + 16 * grp;
                    const bf16x8_t zh = *reinterpret_cast<const bf16x8_t *>(zh_lds + off);
                    const bf16x8_t zl = *reinterpret_cast<const bf16x8_t *>(zl_lds + off);
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zh, lb[b], acc[a][b], 0, 0, 0);
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zl, lb[b], acc[a][b], 0, 0, 0);
                    }
                }
            }
            __syncthreads();
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

namespace kqhost {
kq_status gemm256_mx(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w, const uint8_t *scales_w,
                     int64_t m, int64_t n, int64_t k, float *O, int64_t ldo, kq_stream_t stream);
kq_status gemm256_mx_lowrank(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                             const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, const float *Z,
                             const uint8_t *codes_l, const uint8_t *scales_l, int64_t r, float *O, int64_t ldo,
                             kq_stream_t stream);
}  // namespace kqhost

namespace {

// RMX: R16 holds R's MXFP4 codes [r][d/2] (16-byte aligned) and SR its scales [r][d/32].
template <bool SPLIT, bool RMX = false>
kq_status project_r16(const uint16_t *X16, int64_t m, int64_t d, int64_t ldx, const uint16_t *R16, int64_t r, float *Z,
                      uint16_t *Zh, uint16_t *Zl, kq_stream_t stream, const uint8_t *SR = nullptr) {
    if (m < 0 || d < 0 || d % 32 != 0 || ldx < d || r <= 0 || r % 32 != 0) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({m, d, ldx, r})) return KQ_ERR_UNSUPPORTED;
    if (m == 0 || d == 0) return KQ_OK;
    if (!X16 || !R16 || (RMX && !SR) || (SPLIT ? (!Zh || !Zl) : !Z)) return KQ_ERR_NULL;
    if (!aligned(X16, 16) || ldx % 8 != 0 || !aligned(R16, 16) || (!SPLIT && !aligned(Z, 16)) ||
        (SPLIT && (!aligned(Zh, 16) || !aligned(Zl, 16))))
        return KQ_ERR_ALIGN;
    const int64_t tiles_m = (m + kq::kProjRows - 1) / kq::kProjRows, tiles_r = (r + 127) / 128;
    if (tiles_m * tiles_r > 0x7FFFFFFF || m > INT64_MAX / 4 / (ldx > r ? ldx : r)) return KQ_ERR_SHAPE;
    // 32-bit buffer records: 80 rows of X, 128 rows of R (bf16, or MXFP4 codes)
    if ((int64_t)kq::kProjRows * ldx * 2 >= ((int64_t)1 << 31) ||
        (int64_t)128 * (RMX ? d / 2 : d * 2) >= ((int64_t)1 << 31))
        return KQ_ERR_UNSUPPORTED;
    kq::ProjGeom g{m, d, ldx, r, tiles_r};
    hipLaunchKernelGGL((kq::lowrank_project_r16_kernel<SPLIT, RMX>), dim3((unsigned)(tiles_m * tiles_r)),
                       dim3(64 * (kq::kProjWaves + kq::kProjProducers)), 0, (hipStream_t)stream, X16, g, R16, Z, Zh,
                       Zl, SR);
    return launched();
}

}  // namespace

extern "C" {

kq_status kq_mxfp4_gemm(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                        const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, float *O, int64_t ldo,
                        kq_stream_t stream) {
    if (m < 0 || n < 0 || k < 0 || k % 32 != 0 || ldo < n) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({m, n, k, ldo})) return KQ_ERR_UNSUPPORTED;
    if (m == 0 || n == 0) return KQ_OK;
    if (!codes_a || !scales_a || !codes_w || !scales_w || !O) return KQ_ERR_NULL;
    if (!aligned(codes_a, 16) || !aligned(codes_w, 16) || (k / 2) % 16 != 0) return KQ_ERR_ALIGN;
    // k a multiple of 256: the 256 x 256-tile kernel reading the MX-layout scales
    // (the same instruction and k order as the packed-scale product); when it takes
    // the shape, it runs
    if (k > 0 && k % 256 == 0 && aligned(scales_a, 4) && aligned(scales_w, 4) && aligned(O, 4)) {
        const kq_status st = kqhost::gemm256_mx(codes_a, scales_a, codes_w, scales_w, m, n, k, O, ldo, stream);
        if (st != KQ_ERR_UNSUPPORTED) return st;
    }
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
    if (!kqhost::sizes_fit({m, n, k, ldo, r})) return KQ_ERR_UNSUPPORTED;
    if (m == 0 || n == 0) return KQ_OK;
    if (!codes_a || !scales_a || !codes_w || !scales_w || !O || !Z || !codes_l || !scales_l) return KQ_ERR_NULL;
    if (!aligned(codes_a, 16) || !aligned(codes_w, 16) || (k / 2) % 16 != 0 || !aligned(Z, 16) ||
        !aligned(codes_l, 16))
        return KQ_ERR_ALIGN;
    // k a multiple of 256: the 256 x 256-tile kernel with the term in its epilogue,
    // reading the MX-layout scales (as kq_mxfp4_gemm)
    if (k > 0 && k % 256 == 0 && aligned(scales_a, 4) && aligned(scales_w, 4) && aligned(O, 4)) {
        const kq_status st = kqhost::gemm256_mx_lowrank(codes_a, scales_a, codes_w, scales_w, m, n, k, Z, codes_l,
                                                        scales_l, r, O, ldo, stream);
        if (st != KQ_ERR_UNSUPPORTED) return st;
    }
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
    if (!kqhost::sizes_fit({m, d, ldx, r})) return KQ_ERR_UNSUPPORTED;
    if (m == 0 || d == 0) return KQ_OK;
    if (!X16 || !codes_r || !scales_r || !Z) return KQ_ERR_NULL;
    if (!aligned(X16, 16) || ldx % 8 != 0 || !aligned(codes_r, 16) || !aligned(Z, 16)) return KQ_ERR_ALIGN;
    return project_r16<false, true>(X16, m, d, ldx, reinterpret_cast<const uint16_t *>(codes_r), r, Z, nullptr,
                                    nullptr, stream, scales_r);
}

kq_status kq_lowrank_project_bf16(const uint16_t *X16, int64_t m, int64_t d, int64_t ldx, const uint16_t *R16,
                                  int64_t r, float *Z, kq_stream_t stream) {
    return project_r16<false>(X16, m, d, ldx, R16, r, Z, nullptr, nullptr, stream);
}

kq_status kq_lowrank_project_bf16_split(const uint16_t *X16, int64_t m, int64_t d, int64_t ldx, const uint16_t *R16,
                                        int64_t r, uint16_t *Zh, uint16_t *Zl, kq_stream_t stream) {
    return project_r16<true>(X16, m, d, ldx, R16, r, nullptr, Zh, Zl, stream);
}

kq_status kq_lowrank_project_split(const uint16_t *X16, int64_t m, int64_t d, int64_t ldx, const uint8_t *codes_r,
                                   const uint8_t *scales_r, int64_t r, uint16_t *Zh, uint16_t *Zl,
                                   kq_stream_t stream) {
    return project_r16<true, true>(X16, m, d, ldx, reinterpret_cast<const uint16_t *>(codes_r), r, nullptr, Zh, Zl,
                                   stream, scales_r);
}

kq_status kq_dequantize_mxfp4_bf16(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t k,
                                   uint16_t *out, kq_stream_t stream) {
    if (rows < 0 || k < 0 || k % 32 != 0) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({rows, k})) return KQ_ERR_UNSUPPORTED;
    if (rows == 0 || k == 0) return KQ_OK;
    if (!codes || !scales || !out) return KQ_ERR_NULL;
    if (!aligned(codes, 4) || !aligned(out, 16)) return KQ_ERR_ALIGN;
    if (rows > INT64_MAX / k) return KQ_ERR_SHAPE;
    const int64_t n8 = rows * (k / 8), blocks = (n8 + kq::kThreads - 1) / kq::kThreads;
    hipLaunchKernelGGL(kq::dequantize_bf16_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)),
                       dim3(kq::kThreads), 0, (hipStream_t)stream, reinterpret_cast<const uint32_t *>(codes), scales,
                       n8, reinterpret_cast<kq::bf16x8_t *>(out));
    return launched();
}

}  // extern "C"
