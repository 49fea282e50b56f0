// Device building blocks for the KroQuant quantizer kernels on gfx950 (CDNA4).
//
// Lane layout shared by the bf16 kernels: a 32-channel block is held by a quad
// of four consecutive lanes, lane `sub` (0..3) owning channels 8*sub .. 8*sub+7
// (one 16-byte bf16 load). Channel bits 4 and 3 are therefore the two bits of
// `sub`, bits 2..0 the position inside the lane. Cross-lane traffic never
// leaves the quad, so it is done with DPP quad permutes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// ---------------------------------------------------------------------------
// Cross-lane moves inside a quad (DPP quad_perm; all four lanes must be active)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}

// bf16 pairs packed in one dword -> two fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void widen8(const uint4 &q, float x[8]) {
    x[0] = bf16_lo(q.x); x[1] = bf16_hi(q.x);
    x[2] = bf16_lo(q.y); x[3] = bf16_hi(q.y);
    x[4] = bf16_lo(q.z); x[5] = bf16_hi(q.z);
    x[6] = bf16_lo(q.w); x[7] = bf16_hi(q.w);
}

// ---------------------------------------------------------------------------
// MXFP4 block quantizer (OCP MX: E8M0 shared scale, E2M1 elements)
// ---------------------------------------------------------------------------

// E8M0 byte of a block from its largest magnitude (amax >= 0, finite):
// e = max(floor(log2 amax) - 2, -127), byte = e + 127. For a normal amax the
// biased exponent field E gives floor(log2 amax) = E - 127, so byte = E - 2; a
// zero or subnormal amax (E = 0), and E = 1 or 2, clamp to byte 0.
__device__ __forceinline__ uint32_t e8m0_byte(float amax) {
    uint32_t E = __float_as_uint(amax) >> 23;
    return E > 2u ? E - 2u : 0u;
}

// 2^-e as fp32 for scale byte s = e + 127 (exponent field 254 - s, always normal).
__device__ __forceinline__ float inv_scale_of(uint32_t sbyte) {
    return __uint_as_float((254u - sbyte) << 23);
}

// E2M1 code of y given mul = 2^-e. v = |y| 2^-e is exact (power-of-two scaling;
// results below 2^-126 may round but are far below the first rounding boundary
// 0.25). Rounding to the E2M1 grid with ties to even: the grid step in the
// binade of v is 2^(max(floor(log2 v), 0) - 1), i.e. 0.5 below 2, 1 in [2,4),
// 2 in [4,8). Adding and subtracting M = 2^(max(floor(log2 v),0) + 22) rounds v
// to a multiple of that step with the fp32 adder's round-to-nearest-even, and
// the parity of the multiple equals the parity of the E2M1 code, so ties land
// on the even code. The result is then saturated at 6 (v < 8 always holds).
__device__ __forceinline__ uint32_t e2m1_code(float y, float mul) {
    float v = fabsf(y) * mul;
    uint32_t fl = __float_as_uint(v) & 0x7F800000u;
    fl = fl > 0x3F800000u ? fl : 0x3F800000u;
    float M = __uint_as_float(fl + (22u << 23));
    float r = (v + M) - M;
    r = fminf(r, 6.0f);
    // r in {0, .5, 1, 1.5, 2, 3, 4, 6}: fp32 bits >> 22 are {0, 252, 254..259}
    uint32_t t = __float_as_uint(r) >> 22;
    uint32_t idx = (t > 251u ? t : 251u) - 251u;  // 0, 1, 3, 4, 5, 6, 7, 8
    uint32_t code = idx - (idx > 2u ? 1u : 0u);
    return code | ((__float_as_uint(y) >> 31) << 3);
}

// Quantize the 8 values a lane holds of a quad-held block. Returns the lane's
// 8 codes packed as a dword (element 2k in the low nibble of byte k) and the
// block's scale byte (identical in all four lanes).
__device__ __forceinline__ uint32_t quantize_quad8(const float y[8], uint32_t &sbyte) {
    float amax = fabsf(y[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
    amax = fmaxf(amax, quad_xor1(amax));
    amax = fmaxf(amax, quad_xor2(amax));
    sbyte = e8m0_byte(amax);
    const float mul = inv_scale_of(sbyte);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= e2m1_code(y[i], mul) << (4 * i);
    return packed;
}

// ---------------------------------------------------------------------------
// Kronecker block K = G1 (x) ... (x) G5 applied as five 2x2 stages (Eq. 12):
// stage k mixes each pair of channels that differ only in channel bit 5-k,
// (x0, x1) -> (x0 G[0][0] + x1 G[1][0], x0 G[0][1] + x1 G[1][1]).
// ---------------------------------------------------------------------------
struct KronLane {
    float s1, o1;  // G1 (bit 4 = bit 1 of sub): this lane's and the partner's weight
    float s2, o2;  // G2 (bit 3 = bit 0 of sub)
    float g3[4], g4[4], g5[4];  // in-lane stages, entries [0][0],[0][1],[1][0],[1][1]
};

// f20 = the block's factors, G_k[r][c] at f20[4*(k-1) + 2*r + c]. A lane whose
// channel bit is b computes y = x_self G[b][b] + x_partner G[1-b][b].
__device__ __forceinline__ void kron_lane_setup(const float *f20, int sub, KronLane &L) {
    const int b4 = (sub >> 1) & 1, b3 = sub & 1;
    L.s1 = f20[0 + 2 * b4 + b4];
    L.o1 = f20[0 + 2 * (1 - b4) + b4];
    L.s2 = f20[4 + 2 * b3 + b3];
    L.o2 = f20[4 + 2 * (1 - b3) + b3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        L.g3[i] = f20[8 + i];
        L.g4[i] = f20[12 + i];
        L.g5[i] = f20[16 + i];
    }
}

template <int STRIDE>
__device__ __forceinline__ void inlane_stage(float x[8], const float g[4]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i & STRIDE) continue;
        const float x0 = x[i], x1 = x[i + STRIDE];
        x[i] = fmaf(x1, g[2], x0 * g[0]);
        x[i + STRIDE] = fmaf(x1, g[3], x0 * g[1]);
    }
}

__device__ __forceinline__ void kron_apply8(float x[8], const KronLane &L) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(quad_xor2(x[i]), L.o1, x[i] * L.s1);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(quad_xor1(x[i]), L.o2, x[i] * L.s2);
    inlane_stage<4>(x, L.g3);
    inlane_stage<2>(x, L.g4);
    inlane_stage<1>(x, L.g5);
}

}  // namespace kq
