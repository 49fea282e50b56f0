// The W4A4 GEMM of Eq. 2 (KroQuant, arXiv 2607.21446v1),
//   O = deq(Q(A T)) deq(Q(W T^{-T}))^T,
// on 256 x 256 output tiles with gfx950's 32 x 32 x 64 scaled FP4 matrix
// instruction, plus the scale re-layout it reads.
//
// Why this shape. On gfx950 the 16 x 16 x 128 scaled instruction issues at the
// FP8 rate whatever the operand format, while the 32 x 32 x 64 form runs FP4
// at twice that (measured: 4.35 vs 8.69 PFLOP/s of independent instructions).
// A 256 x 256 tile per workgroup (four waves, 128 x 128 each, 256 accumulator
// registers per lane) is the largest the register file holds, and it sets the
// operand bytes per flop: the product is bound by how fast L2 and HBM feed the
// CUs (about 30 TB/s for L2 hits, 6.5 TB/s once a working set leaves L2), so
// every choice below is about moving fewer and fuller cache lines:
//  - a stage covers 256 k, i.e. 128 code bytes (one full cache line) per row;
//  - operands go straight from memory into LDS (buffer loads with the LDS bit),
//    two stages double-buffered (2 x 68 KB), the next stage's 17 loads per wave
//    issued one after each of the current stage's first 17 matrix instructions
//    (packed tighter, the texture unit's queue stalls the matrix issue; spread
//    over three k steps, they arrive late), and waited for 3/4 of the way
//    through the stage's last k step;
//  - scales are read in a GEMM-ready layout (kq_pack_mxfp4_scales): the 8 scale
//    bytes of one 256-k stage of consecutive rows are consecutive, so a stage's
//    scales for 256 rows are one 2 KB run instead of 256 scattered lines, and
//    they are ordered even blocks first, so the scale a lane needs at step j
//    is byte j of the dword of its block parity: the instruction's byte select
//    picks it, with no per-lane shift. The same kernel also reads the MX layout
//    [rows][k/32] as the quantizer writes it (NS): four 4-byte-per-lane loads per
//    wave and stage gather the rows' eight bytes, and one byte permute builds
//    the parity dword (about 15% slower at 18432 x 3072 x 3072: the scattered
//    scale lines);
//  - tiles are numbered so that each XCD (workgroups are dealt to the eight XCDs
//    round robin) gets a contiguous run, walked in bands of 4 row tiles, which
//    keeps the operand rows a run shares in that XCD's L2; one launch covers
//    whole tiles and half tiles in the order of kq_tileorder.hpp;
//  - the output leaves through LDS: each store instruction writes 4 whole rows
//    of 256 bytes (8 full cache lines) rather than 32 rows x 32 bytes, which
//    the store path serves several times faster (the fp32 epilogue of a tile,
//    256 KB per CU, had taken as long as 4 of its 12 k stages at k = 3072).
//
// LDS layout of a stage: A codes [256 rows][128 bytes], W codes likewise, A
// scales [256 rows][8 bytes], W scales likewise. Code rows are stored with
// their eight 16-byte chunks permuted (chunk c of row r at slot c ^ swz8(r));
// a matrix read (32 rows of one chunk) then hits 32 distinct bank groups.
//
// Matrix layout (swapped operands, so a lane owns output rows): the
// instruction's A operand is a W fragment and its B operand an A fragment;
// lane l supplies row l % 32 of each and k group 2 j + l / 32 of step j (one MX
// block: 16 code bytes, one scale byte), and receives O row l % 32 of its
// fragment, columns 8 q + 4 (l / 32) + 0..3 of the W fragment in accumulator
// registers 4 q .. 4 q + 3, so it stores 16 contiguous bytes per q.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kq.h"
#include "kq_cvt.hpp"
#include "kq_device.hpp"
#include "kq_host.hpp"
#include "kq_tileorder.hpp"

namespace kq {
namespace g256 {

constexpr int kThreads = 256;
constexpr int kTile = 256;                      // output rows per tile; columns TN = 256 or 128
constexpr int kGroupM = 4;                      // row tiles per band of the tile order
constexpr int kLoadSteps = 2;                   // k steps of a stage that carry the next stage's loads
constexpr int kNonTemporal = 2;                 // cache-policy operand of a buffer access: nt

// LDS layout of a stage for TN output columns: A codes [256][128], W codes [TN][128],
// A scales [256][8], W scales [TN][8] (68 KB for TN = 256, 51 KB for TN = 128)
template <int TN>
struct Lay {
    static constexpr int kOffW = kTile * 128;
    static constexpr int kOffSA = kOffW + TN * 128;
    static constexpr int kOffSW = kOffSA + kTile * 8;
    static constexpr int kStage = kOffSW + TN * 8;
    static constexpr int NB = TN / 64;   // 32-column W fragments per wave
    static constexpr int LW = TN / 32;   // W code loads (8 rows each) per wave per stage
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

struct Geom {
    int64_t m, n, ldo;
    int kbytes;  // k / 2
    int stages;  // k / 256
    int tiles_m, tiles_n, nwg;
    int rows16;   // O 16-byte aligned and ldo esz % 16 == 0: output rows staged through LDS
    int r;        // rank of the low-rank term (LR kernels)
    TileOrder order;  // which tile, or half tile, each workgroup computes
};

__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Raw buffer descriptor in SGPRs: base, 32-bit record count (bytes); loads at
// or past the count return zero.
__device__ __forceinline__ i32x4_t sdesc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t d;
    d.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    d.z = __builtin_amdgcn_readfirstlane((int)bytes);
    d.w = 0x00020000;
    return d;
}

// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land at
// lds + 16 l. M0 carries the LDS address and is restored afterwards; the
// compiler does not track these loads, so completion is waited for explicitly
// (vmcnt) before a barrier.
__device__ __forceinline__ void dma16(const i32x4_t &d, uint32_t lds, uint32_t voff, uint32_t soff) {
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "s"(lds), "v"(voff), "s"(d), "s"(soff)
        : "memory");
}

// 4 bytes per lane from the buffer straight into LDS: lane l's bytes land at lds + 4 l.
__device__ __forceinline__ void dma4(const i32x4_t &d, uint32_t lds, uint32_t voff) {
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "s"(lds), "v"(voff), "s"(d)
        : "memory");
}

__device__ __forceinline__ void wait_loads_and_lds_then_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int NB>
struct Frag {
    i32x8_t a[4], b[NB];
};

// a stage's scale dwords of the lane's rows (the same dword serves all four steps)
template <int NB>
struct Scl {
    uint32_t sa[4], sb[NB];
};

typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// LR: after the product, the low-rank term Z deq(L)^T of Sec. 3.4 Eq. 11 is
// added into the same accumulators (Z fp32 [m][r] split as hi + lo bf16, exact
// to 2^-16 relative; deq(L) exact in bf16), 64 of r at a time through LDS, on
// v_mfma_f32_32x32x16_bf16 with the same swapped operands and 32 x 32 layout.
//
// TN = 128 is the half-width form (with or without the low-rank term): half h of
// a tile, its 128 columns at 128 h, each output element accumulated by the same
// instructions in the same k order as in the full tile.
//
// B16: O is written in bf16 (each fp32 sum rounded to nearest even) instead of fp32.
//
// One tile (run-order number u; half h of it when TN = 128) of one workgroup;
// smem holds 2 stages of the full-width layout plus 1 KB.
template <bool LR, int TN, bool B16, bool LRS = false, bool NS = false>
__device__ __forceinline__ void gemm256_tile(const uint8_t *__restrict__ ca, const uint8_t *__restrict__ psa,
                                             const uint8_t *__restrict__ cw, const uint8_t *__restrict__ psw,
                                             const Geom g, const void *__restrict__ lr0,
                                             const void *__restrict__ lr1, const void *__restrict__ lr2,
                                             void *__restrict__ O, int u, int h, uint8_t *smem) {
    static_assert(TN == 256 || TN == 128, "tile width");
    using L = Lay<TN>;
    constexpr int NB = L::NB, LW = L::LW;
    // stage buffers at kStage of the full-width layout (the spare 1 KB after two
    // of them takes the dummy scale load of wave 3 at TN = 128)
    constexpr int kStage = Lay<256>::kStage;
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);

    // run-order tile u: bands of kGroupM row tiles, column-major inside a band
    const int band = u / (kGroupM * g.tiles_n), within = u % (kGroupM * g.tiles_n);
    const int gm = min(kGroupM, g.tiles_m - band * kGroupM);
    const int tm = band * kGroupM + within % gm, tn = within / gm;
    const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile + (TN == 256 ? 0 : 128 * h);
    const int rows_a = (int)min<int64_t>(kTile, g.m - m0), rows_w = (int)min<int64_t>(TN, g.n - n0);
    if (rows_w <= 0) return;  // the right half of a tile narrower than 129 columns (whole workgroup)

    // codes: rows past m or n are past the record count and read zero
    const i32x4_t dca = sdesc(ca + m0 * g.kbytes, (uint32_t)(rows_a * g.kbytes));
    const i32x4_t dcw = sdesc(cw + n0 * g.kbytes, (uint32_t)(rows_w * g.kbytes));
    // packed scales: stage s of row i at 8 (s rows + i), the whole offset in the
    // range-checked vector offset (the scalar offset is not checked), so every
    // read stays inside the packed array: a padding row past m or n reads a
    // later stage's bytes (harmless: its codes are zero and its outputs are
    // never stored), or zero on the last stage
    const i32x4_t dsa = sdesc(psa, (uint32_t)(g.stages * 8 * g.m));
    const i32x4_t dsw = sdesc(psw, (uint32_t)(g.stages * 8 * g.n));
    // (NS) scales in the MX layout [rows][k / 32]: row i's eight bytes of stage s at
    // (k / 32) i + 8 s, blocks in order; same record counts (k / 32 = 8 stages)
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // code load j of wave w: A rows 64 w + 8 j + (lane >> 3) (j < 8), W rows
    // (TN / 4) w + 8 j + (lane >> 3) (j < LW); slot lane & 7
    uint32_t cvoff[8], cvoffw[LW];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = 64 * w + 8 * j + (lane >> 3);
        cvoff[j] = (uint32_t)(row * g.kbytes) + 16u * (uint32_t)((lane & 7) ^ swz8(row & 15));
    }
#pragma unroll
    for (int j = 0; j < LW; ++j) {
        const int row = (TN / 4) * w + 8 * j + (lane >> 3);
        cvoffw[j] = (uint32_t)(row * g.kbytes) + 16u * (uint32_t)((lane & 7) ^ swz8(row & 15));
    }
    // loads of stage s: i in 0..7 A codes, 8..8 + LW - 1 W codes
    auto issue_code = [&](int s, int i) {
        const uint32_t st = lds0 + (uint32_t)((s & 1) * kStage);
        const uint32_t kb = 128u * (uint32_t)s;
        if (i < 8) dma16(dca, st + (64 * w + 8 * i) * 128, cvoff[i], kb);
        else dma16(dcw, st + L::kOffW + ((TN / 4) * w + 8 * (i - 8)) * 128, cvoffw[i - 8], kb);
    };
    // scales of stage s, 1 KB per load: A rows 128 (w & 1) .. by waves 0 and 1, W rows
    // 128 (w & 1) .. by waves 2 and 3 (TN = 256) or all TN rows by wave 2 (TN = 128;
    // wave 3's load is then past the record count and lands in the spare LDS).
    // Written without branches (the wave index is uniform: scalar selects), so
    // that the loop body stays one block and the order fixed below holds.
    const int srow = 128 * (w & 1) + 2 * lane;
    const bool sw_a = w < 2, sw_none = TN == 128 && w == 3;
    const i32x4_t dss = sw_a ? dsa : dsw;
    const uint32_t srow_off = (uint32_t)(8 * ((sw_a ? m0 : n0) + srow)), s_stride = (uint32_t)(8 * (sw_a ? g.m : g.n));
    const uint32_t s_lds = sw_none ? (uint32_t)(2 * kStage) : (uint32_t)((sw_a ? L::kOffSA : L::kOffSW) + 1024 * (w & 1));
    // (NS) four loads of 256 bytes per wave and stage: load j, lane l: row
    // 128 (w & 1) + 32 j + l / 2 of the wave's operand, its dword l & 1 of the stage,
    // into the same [rows][8] bytes of LDS (blocks in order instead of even first)
    const uint32_t ns_row = (uint32_t)(((sw_a ? m0 : n0) + 128 * (w & 1) + (lane >> 1)) * (int64_t)(8 * g.stages)) +
                            4u * (uint32_t)(lane & 1);
    auto issue_scl_ns = [&](int s, int j) {
        const uint32_t voff = sw_none ? 0x80000000u : ns_row + (uint32_t)(32 * j * 8 * g.stages + 8 * s);
        dma4(dss, lds0 + (uint32_t)((s & 1) * kStage) * !sw_none + s_lds + 256u * (uint32_t)j, voff);
    };
    auto issue_scl = [&](int s) {
        if constexpr (NS) {
#pragma unroll
            for (int j = 0; j < 4; ++j) issue_scl_ns(s, j);
            return;
        }
        const uint32_t voff = sw_none ? 0x80000000u : srow_off + s_stride * (uint32_t)s;
        dma16(dss, lds0 + (uint32_t)((s & 1) * kStage) * !sw_none + s_lds, voff, 0u);
    };

    const int r = lane & 31, hi = lane >> 5;
    const int wm = (w >> 1) * 128, wn = (w & 1) * (TN / 2);
    int rdo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) rdo[j] = r * 128 + 16 * ((2 * j + hi) ^ swz8(r & 15));

    // stage s: the scale dword of the lane's block parity hi (byte j is block 2 j + hi)
    // (NS) the dword of parity hi gathered from the row's two dwords: bytes of
    // blocks hi, 2 + hi (first dword) and 4 + hi, 6 + hi (second)
    const uint32_t ns_sel = hi ? 0x07050301u : 0x06040200u;
    auto read_scl = [&](int s, Scl<NB> &S) {
        if constexpr (NS) {
            const uint8_t *sc = smem + (s & 1) * kStage + 8 * r;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const uint2 d = *reinterpret_cast<const uint2 *>(sc + L::kOffSA + 8 * (wm + 32 * a));
                S.sa[a] = __builtin_amdgcn_perm(d.y, d.x, ns_sel);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint2 d = *reinterpret_cast<const uint2 *>(sc + L::kOffSW + 8 * (wn + 32 * b));
                S.sb[b] = __builtin_amdgcn_perm(d.y, d.x, ns_sel);
            }
            return;
        }
        const uint8_t *sc = smem + (s & 1) * kStage + 4 * hi + 8 * r;
#pragma unroll
        for (int a = 0; a < 4; ++a) S.sa[a] = *reinterpret_cast<const uint32_t *>(sc + L::kOffSA + 8 * (wm + 32 * a));
#pragma unroll
        for (int b = 0; b < NB; ++b) S.sb[b] = *reinterpret_cast<const uint32_t *>(sc + L::kOffSW + 8 * (wn + 32 * b));
    };
    // step j of stage s: 16-byte fragments (k group 2 j + hi)
    auto read_frags = [&](int s, int j, Frag<NB> &F) {
        const uint8_t *st = smem + (s & 1) * kStage;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const uint4 q = *reinterpret_cast<const uint4 *>(st + (wm + 32 * a) * 128 + rdo[j]);
            F.a[a] = i32x8_t{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint4 q = *reinterpret_cast<const uint4 *>(st + L::kOffW + (wn + 32 * b) * 128 + rdo[j]);
            F.b[b] = i32x8_t{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        }
    };

    floatx16_t acc[4][NB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    // the scale of group 2 j + hi is byte j of the lane's scale dword: the byte
    // select (op_sel) of the instruction's scale operands, uniform across lanes
    auto mma = [&](const Frag<NB> &F, const Scl<NB> &S, auto jc, int a, int b) {
        constexpr int j = decltype(jc)::value;
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[b], F.a[a], acc[a][b], 4, 4, j, (int)S.sb[b],
                                                                    j, (int)S.sa[a]);
    };
    // ties the matrix instruction that wrote acc[a][b] to this point of the
    // program: it emits nothing, but the accumulator is an operand of a volatile
    // statement, so the instruction cannot drift past the loads issued after it
    auto pin = [&](int a, int b) { asm volatile("" : "+a"(acc[a][b])); };
    auto step = [&](const Frag<NB> &F, const Scl<NB> &S, auto jc) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b) mma(F, S, jc, a, b);
    };
    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    using J2 = std::integral_constant<int, 2>;
    using J3 = std::integral_constant<int, 3>;

    // LDS after the product: Z hi [256][64] bf16, Z lo likewise, deq(L) [256][64]
    // bf16, rows of 128 bytes with the 16-byte chunks permuted as the codes are
    uint8_t *zh = smem, *zl = smem + 32768, *ll = smem + 65536;
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(static_cast<const float *>(lr0) + m0 * g.r), (short)0, (int)(rows_a * g.r * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t rcl = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(static_cast<const uint8_t *>(lr1) + n0 * (g.r / 2)), (short)0, (int)(rows_w * (g.r / 2)),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rsl = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(static_cast<const uint8_t *>(lr2) + n0 * (g.r / 32)), (short)0, (int)(rows_w * (g.r / 32)),
        0x00020000);
    // (LR) a chunk (64 of r) is staged by 8 passes of 32 rows: lane t & 7 of row
    // 32 p + t / 8 takes 8 consecutive columns, so 8 lanes read a row's 256
    // bytes of Z (32 of L's code bytes) together; the next chunk's loads go
    // out before this chunk's matrix work (a chunk past r reads zeros)
    u32x4_t zr[8][2];
    uint32_t lc[8], ls[8];
    const int cc = t & 7;
    auto load_chunk = [&](int r0) {
        const int kc = r0 + 8 * cc;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int row = 32 * p + (t >> 3);
            const uint32_t zo = kc < g.r ? (uint32_t)((row * g.r + kc) * 4) : 0x80000000u;
            zr[p][0] = __builtin_amdgcn_raw_buffer_load_b128(rz, zo, 0, 0);
            zr[p][1] = __builtin_amdgcn_raw_buffer_load_b128(rz, zo + 16u, 0, 0);
            const uint32_t co = kc < g.r ? (uint32_t)(row * (g.r / 2) + kc / 2) : 0x80000000u;
            const uint32_t so = kc < g.r ? (uint32_t)(row * (g.r / 32) + kc / 32) : 0x80000000u;
            lc[p] = __builtin_amdgcn_raw_buffer_load_b32(rcl, co, 0, 0);
            ls[p] = __builtin_amdgcn_raw_buffer_load_b8(rsl, so, 0, 0);
        }
    };

    // (LRS) the low-rank operands arrive split in bf16 -- Zh = bf16(Z), Zl = bf16(Z - Zh)
    // [m][r] and deq(L) [n][r] -- and move 32 of r at a time straight into a stage
    // buffer, like the codes: Zh at 0, Zl at 16 KB, L at 32 KB, rows of 64 bytes with
    // 16-byte chunk c of row i at slot c ^ ((i / 4) % 4), so a 32-row fragment read
    // is free of bank conflicts. A chunk takes 4 + 4 + TN / 64 loads per wave of
    // 16 rows each; the first goes out during the last k stage, each next one during
    // the current one's matrix work. Same instructions, same order as the fp32-Z
    // path: bit-identical sums.
    constexpr int kLrLoads = 8 + TN / 64;
    const i32x4_t dzh = sdesc(static_cast<const uint16_t *>(lr0) + m0 * g.r, (uint32_t)(rows_a * g.r * 2));
    const i32x4_t dzl = sdesc(static_cast<const uint16_t *>(lr1) + m0 * g.r, (uint32_t)(rows_a * g.r * 2));
    const i32x4_t dll = sdesc(static_cast<const uint16_t *>(lr2) + n0 * g.r, (uint32_t)(rows_w * g.r * 2));
    auto lr_issue = [&](int c, int l) {  // load l of chunk c, into the buffer of stage stages + c
        const uint32_t st = lds0 + (uint32_t)(((g.stages + c) & 1) * kStage);
        const int fr = (lane >> 4) & 3;  // (row / 4) % 4 of the lane's row (rows of a load start at multiples of 16)
        const uint32_t inrow = (uint32_t)(2 * (32 * c + 8 * ((lane & 3) ^ fr)));
        if (l < 8) {
            const int j = l & 3, row = 64 * w + 16 * j + (lane >> 2);
            dma16(l < 4 ? dzh : dzl, st + (l < 4 ? 0u : 16384u) + (uint32_t)((64 * w + 16 * j) * 64),
                  (uint32_t)(row * g.r * 2) + inrow, 0u);
        } else {
            const int j = l - 8, row = (TN / 4) * w + 16 * j + (lane >> 2);
            dma16(dll, st + 32768u + (uint32_t)(((TN / 4) * w + 16 * j) * 64), (uint32_t)(row * g.r * 2) + inrow, 0u);
        }
    };

    if (g.stages > 0) {  // k == 0: O = 0
    issue_scl(0);
#pragma unroll
    for (int i = 0; i < 8 + LW; ++i) issue_code(0, i);
    wait_loads_and_lds_then_barrier();
    Frag<NB> F0, F1;
    Scl<NB> S, Sn;
    read_scl(0, S);
    read_frags(0, 0, F0);

    // load l of stage s: 0 .. 8 + LW - 1 the code loads, 8 + LW the scale load
    constexpr int kLoads = 8 + LW + (NS ? 4 : 1), kPerStep = (kLoads + kLoadSteps - 1) / kLoadSteps;
    static_assert(kPerStep <= 4 * NB && kLoadSteps <= 3, "every load of a stage needs a slot before the wait");
    auto issue_load = [&](int s, int l) {
        if (l < 8 + LW) issue_code(s, l);
        else if (NS) issue_scl_ns(s, l - (8 + LW));
        else issue_scl(s);
    };
    // step j of stage s with stage s + 1's loads kPerStep j .. placed one after
    // each matrix instruction (the loads are spread over the first kLoadSteps
    // steps, so that the texture unit's queue never stalls the matrix issue)
    auto step_loading = [&](const Frag<NB> &F, const Scl<NB> &S, auto jc, int s) {
        constexpr int j = decltype(jc)::value;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int l = kPerStep * j + NB * a + b;
                mma(F, S, jc, a, b);
                if (j < kLoadSteps && NB * a + b < kPerStep && l < kLoads) {
                    pin(a, b);
                    issue_load(s + 1, l);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    };

    // Stage s (s + 1 < stages): the buffer of stage s + 1 held stage s - 1, whose
    // last reads came before the previous barrier, so its loads go out during
    // steps 0 .. kLoadSteps - 1; the barrier after step 2 makes them visible and
    // ends every wave's reads of stage s before stage s + 2 reuses the buffer.
    for (int s = 0; s + 1 < g.stages; ++s) {
        read_frags(s, 1, F1);
        __builtin_amdgcn_sched_barrier(0);
        step_loading(F0, S, J0(), s);
        read_frags(s, 2, F0);
        __builtin_amdgcn_sched_barrier(0);
        step_loading(F1, S, J1(), s);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(s, 3, F1);
        __builtin_amdgcn_sched_barrier(0);
        step_loading(F0, S, J2(), s);
        __builtin_amdgcn_sched_barrier(0);
        // step 3 split around the wait (3 of its 4 row blocks before): the loads
        // get most of a step more, and the reads of stage s + 1's first
        // fragments overlap the last row block
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b) mma(F1, S, J3(), a, b);
        __builtin_amdgcn_sched_barrier(0);
        wait_loads_and_lds_then_barrier();
        read_scl(s + 1, Sn);
        read_frags(s + 1, 0, F0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < NB; ++b) mma(F1, S, J3(), 3, b);
        __builtin_amdgcn_sched_barrier(0);
        S = Sn;
    }
    {
        const int s = g.stages - 1;
        // the branch's first chunk is in flight during the last stage
        if (LR && !LRS) load_chunk(0);
        read_frags(s, 1, F1);
        // (LRS) the first chunk's loads, one after each of the first kLrLoads
        // matrix instructions of steps 0 and 1
        auto step_lr = [&](const Frag<NB> &F, auto jc, int j0) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    mma(F, S, jc, a, b);
                    const int l = j0 + NB * a + b;
                    if (l < kLrLoads) {
                        pin(a, b);
                        lr_issue(0, l);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
        };
        static_assert(kLrLoads <= 8 * NB, "the first chunk's loads fit two steps");
        if constexpr (LRS) step_lr(F0, J0(), 0);
        else step(F0, S, J0());
        read_frags(s, 2, F0);
        if constexpr (LRS) step_lr(F1, J1(), 4 * NB);
        else step(F1, S, J1());
        read_frags(s, 3, F1);
        step(F0, S, J2());
        step(F1, S, J3());
    }
    } else if (LR) {
        if constexpr (LRS) {
#pragma unroll
            for (int l = 0; l < kLrLoads; ++l) lr_issue(0, l);
        } else {
            load_chunk(0);
        }
    }

    if constexpr (LRS) {
        const int nch = g.r / 32, f = (r >> 2) & 3;
        for (int c = 0; c < nch; ++c) {
            // chunk c has landed; every wave is done with the other buffer, which
            // takes the next chunk's loads at once (a chunk's matrix work hides them)
            wait_loads_and_lds_then_barrier();
            if (c + 1 < nch) {
#pragma unroll
                for (int l = 0; l < kLrLoads; ++l) lr_issue(c + 1, l);
            }
            const uint8_t *st = smem + ((g.stages + c) & 1) * kStage;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int off = 16 * ((2 * kk + hi) ^ f);
                bf16x8v_t lf[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    lf[b] = *reinterpret_cast<const bf16x8v_t *>(st + 32768 + (wn + 32 * b + r) * 64 + off);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const bf16x8v_t hf = *reinterpret_cast<const bf16x8v_t *>(st + (wm + 32 * a + r) * 64 + off);
                    const bf16x8v_t lo =
                        *reinterpret_cast<const bf16x8v_t *>(st + 16384 + (wm + 32 * a + r) * 64 + off);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[b], hf, acc[a][b], 0, 0, 0);
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[b], lo, acc[a][b], 0, 0, 0);
                    }
                }
            }
        }
    }

    if (LR && !LRS) {
        for (int r0 = 0; r0 < g.r; r0 += 64) {
            // every wave is done with the previous contents of LDS
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int row = 32 * p + (t >> 3);
                const float x[8] = {__uint_as_float(zr[p][0][0]), __uint_as_float(zr[p][0][1]),
                                    __uint_as_float(zr[p][0][2]), __uint_as_float(zr[p][0][3]),
                                    __uint_as_float(zr[p][1][0]), __uint_as_float(zr[p][1][1]),
                                    __uint_as_float(zr[p][1][2]), __uint_as_float(zr[p][1][3])};
                bf16x8_t h, l;
                split_bf16x8_cvt(x, h, l);
                const int slot = row * 128 + 16 * (cc ^ swz8(row & 15));
                *reinterpret_cast<bf16x8_t *>(zh + slot) = h;
                *reinterpret_cast<bf16x8_t *>(zl + slot) = l;
                *reinterpret_cast<bf16x8_t *>(ll + slot) = decode_fp4x8_bf16_cvt(lc[p], ls[p]);
            }
            load_chunk(r0 + 64);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int off = 16 * ((2 * kk + hi) ^ swz8(r & 15));
                bf16x8v_t lf[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    lf[b] = *reinterpret_cast<const bf16x8v_t *>(ll + (wn + 32 * b + r) * 128 + off);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const bf16x8v_t hf = *reinterpret_cast<const bf16x8v_t *>(zh + (wm + 32 * a + r) * 128 + off);
                    const bf16x8v_t lo = *reinterpret_cast<const bf16x8v_t *>(zl + (wm + 32 * a + r) * 128 + off);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[b], hf, acc[a][b], 0, 0, 0);
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[b], lo, acc[a][b], 0, 0, 0);
                    }
                }
            }
        }
    }

    // Output through LDS, so that a store instruction writes whole rows (4 rows
    // of 256 bytes: 8 full cache lines) instead of 32 rows x 32 bytes. Lane (r,
    // hi) holds O row wm + 32 a + r, columns wn + 32 b + 8 q + 4 hi + 0..3. Wave w
    // stages its 128 x 128 block (fp32: 64 columns per pass) in its own 32 KB at
    // 32 KB w, rows of 256 bytes with 16-byte chunk c at c ^ (row & 15). Every
    // wave is done with the operand stages (and the branch's staging) first.
    constexpr int esz = B16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char *>(O) + (m0 * g.ldo + n0) * esz, (short)0,
        (int)(((int64_t)(rows_a - 1) * g.ldo + (g.n - n0)) * esz), 0x00020000);
    // whole 16-byte pieces: columns inside n and aligned rows; otherwise element by
    // element, columns checked (rows past m are past the record count, or checked)
    const bool whole = g.rows16 && n0 + TN <= g.n;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    uint8_t *reg = smem + 32768 * w;
    constexpr int kPasses = B16 ? 1 : NB / 2, kPerPass = NB / kPasses;
    // 16-byte chunks per staged row (bf16 at TN = 128: 8), rows per store
    constexpr int kCpr = B16 ? 4 * NB : 16, kRpi = 64 / kCpr;
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int bb = 0; bb < kPerPass; ++bb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int b = pass * kPerPass + bb, row = 32 * a + r;
                    if (B16) {
                        // round to nearest even in the hardware convert, one per pair
                        const bf16x2_t p0 = {(__bf16)acc[a][b][4 * q], (__bf16)acc[a][b][4 * q + 1]};
                        const bf16x2_t p1 = {(__bf16)acc[a][b][4 * q + 2], (__bf16)acc[a][b][4 * q + 3]};
                        typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
                        const int chunk = 4 * b + q;
                        *reinterpret_cast<u32x2_t *>(reg + row * 256 + 16 * (chunk ^ (row & 15)) + 8 * hi) =
                            u32x2_t{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
                    } else {
                        const int chunk = 8 * bb + 2 * q + hi;
                        *reinterpret_cast<floatx4_t *>(reg + row * 256 + 16 * (chunk ^ (row & 15))) =
                            floatx4_t{acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                                      acc[a][b][4 * q + 3]};
                    }
                }
        // the wave reads back only what it wrote (its LDS operations complete in order)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int c = lane % kCpr;
#pragma unroll 8
        for (int i = 0; i < 128 / kRpi; ++i) {
            const int row = kRpi * i + lane / kCpr;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(reg + row * 256 + 16 * (c ^ (row & 15)));
            const int col = B16 ? wn + 8 * c : wn + 64 * pass + 4 * c;  // from n0
            const int orow = wm + row;                                    // from m0
            if (whole) {
                // non-temporal: O is not read again here, so it should not push the
                // operand lines that the other workgroups still read out of L2
                __builtin_amdgcn_raw_buffer_store_b128(v, ro, (uint32_t)((orow * g.ldo + col) * esz), 0, kNonTemporal);
            } else if (B16) {
                // plain stores: with 2-byte buffer stores the compiler kept the
                // descriptor in vector registers and looped over it
                if (orow < rows_a) {
                    uint16_t *o16 = static_cast<uint16_t *>(O) + (m0 + orow) * g.ldo + n0 + col;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n0 + col + e < g.n) o16[e] = (uint16_t)(v[e / 2] >> (16 * (e & 1)));
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n0 + col + e < g.n)
                        __builtin_amdgcn_raw_buffer_store_b32(v[e], ro, (uint32_t)((orow * g.ldo + col + e) * 4), 0, 0);
            }
        }
    }
}

// One workgroup per tile (or half tile) in the launch's work order.
template <bool LR, bool B16, bool LRS = false, bool NS = false>
__global__ __launch_bounds__(kThreads) void gemm256_kernel(const uint8_t *__restrict__ ca,
                                                           const uint8_t *__restrict__ psa,
                                                           const uint8_t *__restrict__ cw,
                                                           const uint8_t *__restrict__ psw, Geom g,
                                                           const void *__restrict__ lr0,
                                                           const void *__restrict__ lr1,
                                                           const void *__restrict__ lr2,
                                                           void *__restrict__ O) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * Lay<256>::kStage + 1024];
    const TileWork wk = tile_work((int)blockIdx.x, g.order);
    if (wk.half < 0) gemm256_tile<LR, 256, B16, LRS, NS>(ca, psa, cw, psw, g, lr0, lr1, lr2, O, wk.tile, 0, smem);
    else gemm256_tile<LR, 128, B16, LRS, NS>(ca, psa, cw, psw, g, lr0, lr1, lr2, O, wk.tile, wk.half, smem);
}

// Compute units of the current device (cached per device; 256 on MI355X).
static int cu_count() {
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

// scales [rows][kblocks] -> [kblocks / 8][rows][8], even blocks first: one 8-byte run per thread
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t *__restrict__ in, int64_t rows,
                                                          int64_t kblocks, uint8_t *__restrict__ out) {
    const int64_t total = rows * (kblocks / 8);
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = i / rows, row = i % rows;
        uint2 v;
        __builtin_memcpy(&v, in + row * kblocks + 8 * s, 8);
        // bytes b0..b7 -> b0 b2 b4 b6 | b1 b3 b5 b7
        uint2 o;
        o.x = (v.x & 0xFFu) | ((v.x >> 8) & 0xFF00u) | ((v.y << 16) & 0xFF0000u) | ((v.y << 8) & 0xFF000000u);
        o.y = ((v.x >> 8) & 0xFFu) | ((v.x >> 16) & 0xFF00u) | ((v.y << 8) & 0xFF0000u) | (v.y & 0xFF000000u);
        *reinterpret_cast<uint2 *>(out + 8 * i) = o;
    }
}

}  // namespace g256
}  // namespace kq

namespace {
using kqhost::aligned;
using kqhost::launched;
}  // namespace

extern "C" {

kq_status kq_pack_mxfp4_scales(const uint8_t *scales, int64_t rows, int64_t k, uint8_t *packed,
                               kq_stream_t stream) {
    if (rows < 0 || k < 0 || k % 256 != 0) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({rows, k})) return KQ_ERR_UNSUPPORTED;
    if (rows == 0 || k == 0) return KQ_OK;
    if (!scales || !packed) return KQ_ERR_NULL;
    if (!aligned(packed, 8)) return KQ_ERR_ALIGN;
    if (rows > INT64_MAX / (k / 32)) return KQ_ERR_SHAPE;
    const int64_t total = rows * (k / 256);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(kq::g256::pack_scales_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                       dim3(256), 0, (hipStream_t)stream, scales, rows, k / 32, packed);
    return launched();
}

}  // extern "C"

namespace {

// kq_mxfp4_gemm_packed and its bf16-output form: checks, then whole rounds of full
// tiles and the last partial round as half-width tiles when twice its tile count
// still fits one round of CUs (e.g. 864 tiles on 256 CUs: 768 full, then 96 tiles as
// 192 halves, about half a round instead of a whole one).
// NS: the scales in the MX layout [rows][k / 32] (4-byte aligned) instead of packed.
template <bool B16, bool NS = false>
kq_status gemm_packed(const uint8_t *codes_a, const uint8_t *packed_scales_a, const uint8_t *codes_w,
                      const uint8_t *packed_scales_w, int64_t m, int64_t n, int64_t k, void *O, int64_t ldo,
                      kq_stream_t stream) {
    constexpr int esz = B16 ? 2 : 4;
    constexpr int sal = NS ? 4 : 16;
    if (m < 0 || n < 0 || k < 0 || k % 256 != 0 || ldo < n) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({m, n, k, ldo})) return KQ_ERR_UNSUPPORTED;
    if (m == 0 || n == 0) return KQ_OK;
    if (!O || (k > 0 && (!codes_a || !packed_scales_a || !codes_w || !packed_scales_w))) return KQ_ERR_NULL;
    if (!aligned(codes_a, 16) || !aligned(codes_w, 16) || !aligned(packed_scales_a, sal) ||
        !aligned(packed_scales_w, sal) || !aligned(O, esz))
        return KQ_ERR_ALIGN;
    // buffer record counts and offsets are 32-bit
    const int64_t lim = (int64_t)1 << 31;
    const int64_t tiles_m = (m + 255) / 256, tiles_n = (n + 255) / 256;
    if ((int64_t)256 * (k / 2) >= lim || m * (k / 32) >= lim || n * (k / 32) >= lim ||
        ((int64_t)255 * ldo + n) * esz >= lim || tiles_m * tiles_n >= (lim >> 1))
        return KQ_ERR_UNSUPPORTED;
    kq::g256::Geom g;
    g.m = m;
    g.n = n;
    g.ldo = ldo;
    g.kbytes = (int)(k / 2);
    g.stages = (int)(k / 256);
    g.tiles_m = (int)tiles_m;
    g.tiles_n = (int)tiles_n;
    g.nwg = (int)(tiles_m * tiles_n);
    g.rows16 = aligned(O, 16) && (ldo * esz) % 16 == 0;
    g.r = 0;
    g.order = kq::g256::make_tile_order(g.nwg, kq::g256::cu_count());
    hipLaunchKernelGGL((kq::g256::gemm256_kernel<false, B16, false, NS>),
                       dim3((unsigned)kq::g256::tile_order_groups(g.order)), dim3(kq::g256::kThreads), 0,
                       (hipStream_t)stream, codes_a, packed_scales_a, codes_w, packed_scales_w, g, nullptr, nullptr,
                       nullptr, O);
    return launched();
}

// NS: the scales in the MX layout [rows][k / 32] (4-byte aligned) instead of packed.
template <bool NS>
kq_status gemm_lowrank(const uint8_t *codes_a, const uint8_t *packed_scales_a, const uint8_t *codes_w,
                       const uint8_t *packed_scales_w, int64_t m, int64_t n, int64_t k, const float *Z,
                       const uint8_t *codes_l, const uint8_t *scales_l, int64_t r, float *O, int64_t ldo,
                       kq_stream_t stream) {
    constexpr int sal = NS ? 4 : 16;
    if (m < 0 || n < 0 || k < 0 || k % 256 != 0 || ldo < n || r <= 0 || r % 32 != 0) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({m, n, k, ldo, r})) return KQ_ERR_UNSUPPORTED;
    if (m == 0 || n == 0) return KQ_OK;
    if (!O || !Z || !codes_l || !scales_l || (k > 0 && (!codes_a || !packed_scales_a || !codes_w || !packed_scales_w)))
        return KQ_ERR_NULL;
    if (!aligned(codes_a, 16) || !aligned(codes_w, 16) || !aligned(packed_scales_a, sal) ||
        !aligned(packed_scales_w, sal) || !aligned(O, 4) || !aligned(Z, 16) || !aligned(codes_l, 4))
        return KQ_ERR_ALIGN;
    const int64_t lim = (int64_t)1 << 31;
    const int64_t tiles_m = (m + 255) / 256, tiles_n = (n + 255) / 256;
    if ((int64_t)256 * (k / 2) >= lim || m * (k / 32) >= lim || n * (k / 32) >= lim ||
        ((int64_t)255 * ldo + n) * 4 >= lim || tiles_m * tiles_n >= (lim >> 1) || (int64_t)256 * r * 4 + 32 >= lim)
        return KQ_ERR_UNSUPPORTED;
    kq::g256::Geom g;
    g.m = m;
    g.n = n;
    g.ldo = ldo;
    g.kbytes = (int)(k / 2);
    g.stages = (int)(k / 256);
    g.tiles_m = (int)tiles_m;
    g.tiles_n = (int)tiles_n;
    g.nwg = (int)(tiles_m * tiles_n);
    g.rows16 = aligned(O, 16) && ldo % 4 == 0;
    g.r = (int)r;
    g.order = kq::g256::make_tile_order(g.nwg, kq::g256::cu_count());
    hipLaunchKernelGGL((kq::g256::gemm256_kernel<true, false, false, NS>),
                       dim3((unsigned)kq::g256::tile_order_groups(g.order)), dim3(kq::g256::kThreads), 0,
                       (hipStream_t)stream, codes_a, packed_scales_a, codes_w, packed_scales_w, g, Z, codes_l,
                       scales_l, O);
    return launched();
}

}  // namespace

namespace kqhost {
// The MX-layout product on the 256 x 256-tile kernel (k % 256 == 0), for kq_mxfp4_gemm.
kq_status gemm256_mx(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w, const uint8_t *scales_w,
                     int64_t m, int64_t n, int64_t k, float *O, int64_t ldo, kq_stream_t stream) {
    return gemm_packed<false, true>(codes_a, scales_a, codes_w, scales_w, m, n, k, O, ldo, stream);
}
// The same with the low-rank term (fp32 Z, MXFP4 L), for kq_mxfp4_gemm_lowrank.
kq_status gemm256_mx_lowrank(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                             const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, const float *Z,
                             const uint8_t *codes_l, const uint8_t *scales_l, int64_t r, float *O, int64_t ldo,
                             kq_stream_t stream) {
    return gemm_lowrank<true>(codes_a, scales_a, codes_w, scales_w, m, n, k, Z, codes_l, scales_l, r, O, ldo, stream);
}
}  // namespace kqhost

extern "C" {

kq_status kq_mxfp4_gemm_packed(const uint8_t *codes_a, const uint8_t *packed_scales_a, const uint8_t *codes_w,
                               const uint8_t *packed_scales_w, int64_t m, int64_t n, int64_t k, float *O,
                               int64_t ldo, kq_stream_t stream) {
    return gemm_packed<false>(codes_a, packed_scales_a, codes_w, packed_scales_w, m, n, k, O, ldo, stream);
}

kq_status kq_mxfp4_gemm_packed_bf16(const uint8_t *codes_a, const uint8_t *packed_scales_a,
                                    const uint8_t *codes_w, const uint8_t *packed_scales_w, int64_t m, int64_t n,
                                    int64_t k, uint16_t *O, int64_t ldo, kq_stream_t stream) {
    return gemm_packed<true>(codes_a, packed_scales_a, codes_w, packed_scales_w, m, n, k, O, ldo, stream);
}

kq_status kq_mxfp4_gemm_packed_lowrank(const uint8_t *codes_a, const uint8_t *packed_scales_a,
                                       const uint8_t *codes_w, const uint8_t *packed_scales_w, int64_t m, int64_t n,
                                       int64_t k, const float *Z, const uint8_t *codes_l, const uint8_t *scales_l,
                                       int64_t r, float *O, int64_t ldo, kq_stream_t stream) {
    return gemm_lowrank<false>(codes_a, packed_scales_a, codes_w, packed_scales_w, m, n, k, Z, codes_l, scales_l, r, O,
                               ldo, stream);
}


kq_status kq_mxfp4_gemm_packed_lowrank_split(const uint8_t *codes_a, const uint8_t *packed_scales_a,
                                             const uint8_t *codes_w, const uint8_t *packed_scales_w, int64_t m,
                                             int64_t n, int64_t k, const uint16_t *Zh, const uint16_t *Zl,
                                             const uint16_t *L16, int64_t r, float *O, int64_t ldo,
                                             kq_stream_t stream) {
    if (m < 0 || n < 0 || k < 0 || k % 256 != 0 || ldo < n || r <= 0 || r % 32 != 0) return KQ_ERR_SHAPE;
    if (!kqhost::sizes_fit({m, n, k, ldo, r})) return KQ_ERR_UNSUPPORTED;
    if (m == 0 || n == 0) return KQ_OK;
    if (!O || !Zh || !Zl || !L16 || (k > 0 && (!codes_a || !packed_scales_a || !codes_w || !packed_scales_w)))
        return KQ_ERR_NULL;
    if (!aligned(codes_a, 16) || !aligned(codes_w, 16) || !aligned(packed_scales_a, 16) ||
        !aligned(packed_scales_w, 16) || !aligned(O, 4) || !aligned(Zh, 16) || !aligned(Zl, 16) ||
        !aligned(L16, 16))
        return KQ_ERR_ALIGN;
    const int64_t lim = (int64_t)1 << 31;
    const int64_t tiles_m = (m + 255) / 256, tiles_n = (n + 255) / 256;
    if ((int64_t)256 * (k / 2) >= lim || m * (k / 32) >= lim || n * (k / 32) >= lim ||
        ((int64_t)255 * ldo + n) * 4 >= lim || tiles_m * tiles_n >= (lim >> 1) || (int64_t)256 * r * 2 >= lim)
        return KQ_ERR_UNSUPPORTED;
    kq::g256::Geom g;
    g.m = m;
    g.n = n;
    g.ldo = ldo;
    g.kbytes = (int)(k / 2);
    g.stages = (int)(k / 256);
    g.tiles_m = (int)tiles_m;
    g.tiles_n = (int)tiles_n;
    g.nwg = (int)(tiles_m * tiles_n);
    g.rows16 = aligned(O, 16) && ldo % 4 == 0;
    g.r = (int)r;
    g.order = kq::g256::make_tile_order(g.nwg, kq::g256::cu_count());
    hipLaunchKernelGGL((kq::g256::gemm256_kernel<true, false, true>),
                       dim3((unsigned)kq::g256::tile_order_groups(g.order)), dim3(kq::g256::kThreads), 0,
                       (hipStream_t)stream, codes_a, packed_scales_a, codes_w, packed_scales_w, g, Zh, Zl, L16, O);
    return launched();
}

}  // extern "C"
