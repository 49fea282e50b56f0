// Device building blocks for the KroQuant quantizer kernels on gfx950 (CDNA4).
//
// Quad layout (quantize-only, SmoothQuant, butterfly transform, fp32 kernels):
// a 32-channel block is held by four consecutive lanes, lane `sub` (0..3)
// owning channels 8*sub .. 8*sub+7 (one 16-byte bf16 load). Channel bits 4 and
// 3 are the two bits of `sub`, bits 2..0 the position inside the lane, and
// cross-lane traffic stays inside the quad (DPP quad permutes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// What a quad kernel applies before quantizing: nothing (quantize-only), a
// per-channel scale (SmoothQuant) or the Kronecker transform.
enum Mode { kQuantOnly = 0, kSmooth = 1, kKron = 2 };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Cross-lane moves (all lanes taking part must be active)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t quad_xor1_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_xor2_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float quad_xor1(float v) { return __uint_as_float(quad_xor1_u(__float_as_uint(v))); }
__device__ __forceinline__ float quad_xor2(float v) { return __uint_as_float(quad_xor2_u(__float_as_uint(v))); }

// max over lanes l, l^16, l^32, l^48 (gfx950 row/half-wave swaps)
__device__ __forceinline__ float max_xor16_xor32(float v) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// 16-byte load; NT marks it non-temporal (streamed once, no reuse expected).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4 *p, bool nt) {
    if (!nt) return *p;
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
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

// E8M0 byte from the biased exponent field E of the block's largest magnitude:
// e = max(floor(log2 amax) - 2, -127) and floor(log2 amax) = E - 127 for a
// normal amax, so byte = e + 127 = E - 2; E <= 2 (including zero and
// subnormal amax) clamps to byte 0.
__device__ __forceinline__ uint32_t e8m0_from_exponent(uint32_t E) { return E > 2u ? E - 2u : 0u; }
__device__ __forceinline__ uint32_t e8m0_byte(float amax) {
    return e8m0_from_exponent(__float_as_uint(amax) >> 23);
}

// Scale operand of the gfx950 scaled FP4 converts: they divide by 2^(x - 127)
// where x is the operand's fp32 exponent field, i.e. the E8M0 byte placed
// there. Byte 0 (2^-127) works although the operand then reads as +0.0.
__device__ __forceinline__ float cvt_scale(uint32_t sbyte) { return __uint_as_float(sbyte << 23); }

// v_cvt_scalef32_pk_fp4_*: each call converts two values to E2M1 (first in the
// low nibble) with round-to-nearest-even and saturation at 6, writing byte
// `sel` of the result and keeping the other bytes of `old`. The four calls
// write all four bytes, so the first one's `old` can be any register: the
// first input's (dead after that call), so no zeroing or copying move.
__device__ __forceinline__ uint32_t cvt8_f32(const float y[8], float sc) {
    uint32_t r = __float_as_uint(y[0]);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[0], y[1], sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[2], y[3], sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[4], y[5], sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[6], y[7], sc, 3);
    return r;
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
    bf16x2_t v;
    __builtin_memcpy(&v, &w, 4);
    return v;
}

__device__ __forceinline__ uint32_t cvt8_bf16(const uint4 &q, float sc) {
    uint32_t r = q.x;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(q.x), sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(q.y), sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(q.z), sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(q.w), sc, 3);
    return r;
}

// Largest |x| of 8 fp32 values.
__device__ __forceinline__ float absmax8(const float y[8]) {
    float a = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fabsf(y[2]));
    float b = fmaxf(fmaxf(fabsf(y[3]), fabsf(y[4])), fabsf(y[5]));
    float c = fmaxf(fabsf(y[6]), fabsf(y[7]));
    return fmaxf(fmaxf(a, b), c);
}

// max(v, v of the partner lane) over a quad in one v_max_f32 with a DPP
// operand each (s_nop 1: a DPP read after a VALU write of its source).
__device__ __forceinline__ float quad_max(float v) {
    asm("s_nop 1\n"
        "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "s_nop 1\n"
        "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "+v"(v));
    return v;
}

// Scale operand straight from the block maximum's bits: the scaled converts
// read only the exponent field of their scale operand (a GPU probe over 2^20
// random inputs, scale exponents 0 .. 254 with random mantissa bits, matched
// the mantissa-free operand in every case), so subtracting 2 from the
// exponent field with an unsigned saturating subtract (E <= 2 gives 0, i.e.
// byte 0) leaves the E8M0 byte in bits 30..23 and garbage only in the
// mantissa, which the converts ignore.
__device__ __forceinline__ uint32_t cvt_scale_bits(float amax) {
    return __builtin_elementwise_sub_sat(__float_as_uint(amax), 2u << 23);
}

// Quad-held block from fp32 values: codes dword of this lane, scale byte.
__device__ __forceinline__ uint32_t quantize_quad_f32(const float y[8], uint32_t &sbyte) {
    const float amax = quad_max(absmax8(y));
    const uint32_t sc = cvt_scale_bits(amax);
    sbyte = sc >> 23;
    return cvt8_f32(y, __uint_as_float(sc));
}

// Quad-held block straight from bf16: the magnitude bits of finite bf16 values
// order like unsigned integers, so the block maximum is an integer max.
__device__ __forceinline__ uint32_t quantize_quad_bf16(const uint4 &q, uint32_t &sbyte) {
    const uint32_t k = 0x7FFF7FFFu;
    u16x2_t a, b, c, d;
    const uint32_t ma = q.x & k, mb = q.y & k, mc = q.z & k, md = q.w & k;
    __builtin_memcpy(&a, &ma, 4);
    __builtin_memcpy(&b, &mb, 4);
    __builtin_memcpy(&c, &mc, 4);
    __builtin_memcpy(&d, &md, 4);
    u16x2_t mx = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    uint32_t m2;
    __builtin_memcpy(&m2, &mx, 4);
    uint32_t m = max(m2 & 0xFFFFu, m2 >> 16);
    m = max(m, quad_xor1_u(m));
    m = max(m, quad_xor2_u(m));
    sbyte = e8m0_from_exponent(m >> 7);  // bf16 exponent field = fp32 exponent field
    return cvt8_bf16(q, cvt_scale(sbyte));
}

// ---------------------------------------------------------------------------
// Butterfly form of K = G1 (x) ... (x) G5 (Eq. 12): stage k mixes each pair of
// channels that differ only in channel bit 5-k,
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
    // partner * weight is a VOP2 multiply whose first operand can take the DPP
    // permute directly (v_mul_f32_dpp), then one fma adds this lane's term
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], L.s1, quad_xor2(x[i]) * L.o1);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], L.s2, quad_xor1(x[i]) * L.o2);
    inlane_stage<4>(x, L.g3);
    inlane_stage<2>(x, L.g4);
    inlane_stage<1>(x, L.g5);
}

// ---------------------------------------------------------------------------
// Unit-diagonal shear stages (the kernels' shear form of the butterfly):
// (x0, x1) -> (x0 + q x1, x1 + p x0) for each pair of channels that differ in
// the stage's bit.
// ---------------------------------------------------------------------------
// The block's 20 factor entries with five 16-byte loads (factors are 16-byte aligned).
__device__ __forceinline__ void load_factors20(const float *p, float f[20]) {
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const float4 v = reinterpret_cast<const float4 *>(p)[k];
        f[4 * k] = v.x; f[4 * k + 1] = v.y; f[4 * k + 2] = v.z; f[4 * k + 3] = v.w;
    }
}

template <int STRIDE>
__device__ __forceinline__ void shear_stage(float x[8], float p, float q) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i & STRIDE) continue;
        const float x0 = x[i], x1 = x[i + STRIDE];
        x[i] = fmaf(x1, q, x0);
        x[i + STRIDE] = fmaf(x0, p, x1);
    }
}

// x[i] += c * (x[i] of the partner lane) for the 8 values, as v_fmac_f32 with a
// DPP quad permute on its first operand (one instruction per value; the
// compiler does not fold the permute into an fmac by itself). The leading
// s_nop covers the wait a DPP read needs after a VALU write of its source;
// inside the block no instruction reads what the one before it wrote.
#define KQ_FMAC_DPP8(PERM)                                                        \
    asm("s_nop 1\n"                                                              \
        "v_fmac_f32_dpp %0, %0, %8 " PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
        "v_fmac_f32_dpp %1, %1, %8 " PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
        "v_fmac_f32_dpp %2, %2, %8 " PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
        "v_fmac_f32_dpp %3, %3, %8 " PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
        "v_fmac_f32_dpp %4, %4, %8 " PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
        "v_fmac_f32_dpp %5, %5, %8 " PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
        "v_fmac_f32_dpp %6, %6, %8 " PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
        "v_fmac_f32_dpp %7, %7, %8 " PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1"   \
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),  \
          "+v"(x[6]), "+v"(x[7])                                                  \
        : "v"(c))

__device__ __forceinline__ void fmac_partner_xor2(float x[8], float c) { KQ_FMAC_DPP8("quad_perm:[2,3,0,1]"); }
__device__ __forceinline__ void fmac_partner_xor1(float x[8], float c) { KQ_FMAC_DPP8("quad_perm:[1,0,3,2]"); }

// ---------------------------------------------------------------------------
// Materialized form on MFMA: per block, D = K^T X^T with
// v_mfma_f32_16x16x32_bf16 (A operand 16x32 from K^T, B operand 32x16 from 16
// tokens' bf16 channels, fp32 accumulate). Lane l supplies B[k][n] for token
// n = l % 16, input channels k = 8 (l / 16) + t (one 16-byte load), and A[i][k]
// for output row i = l % 16; it receives D[i][n] for i = 4 (l / 16) + t.
// Output rows are mapped to channels c(h, i) = 8 (i / 4) + 4 h + i % 4 for the
// two halves h, so lane l ends up with channels 8 (l / 16) .. +7 of its token.
// K is carried as three bf16 terms (hi + mid + lo), which represent the fp32
// entries exactly; each product with a bf16 input is exact and the sums
// accumulate in fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

struct KSplit {
    bf16x8_t t[3][2];  // [term hi/mid/lo][half h]
};

// Entries K[r][c] for r = 8 g + t (t = 0..7), c = c(h, l % 16), from Eq. 12.
__device__ __forceinline__ void ksplit_setup(const float *f20, int lane, KSplit &S) {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = 8 * (i >> 2) + 4 * h + (i & 3);
        const float pc = f20[0 + 2 * (g >> 1) + ((c >> 4) & 1)] * f20[4 + 2 * (g & 1) + ((c >> 3) & 1)];
        uint16_t hv[8], mv[8], lv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float k = pc * f20[8 + 2 * ((t >> 2) & 1) + ((c >> 2) & 1)] *
                            f20[12 + 2 * ((t >> 1) & 1) + ((c >> 1) & 1)] *
                            f20[16 + 2 * (t & 1) + (c & 1)];
            hv[t] = bf16_rne_bits(k);
            const float r1 = k - __uint_as_float((uint32_t)hv[t] << 16);  // exact
            mv[t] = bf16_rne_bits(r1);
            lv[t] = bf16_rne_bits(r1 - __uint_as_float((uint32_t)mv[t] << 16));  // exact
        }
        __builtin_memcpy(&S.t[0][h], hv, 16);
        __builtin_memcpy(&S.t[1][h], mv, 16);
        __builtin_memcpy(&S.t[2][h], lv, 16);
    }
}

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

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 &q) {
    bf16x8_t v;
    __builtin_memcpy(&v, &q, 16);
    return v;
}

// y[0..7] = channels 8 (lane / 16) .. +7 of this lane's token, fp32.
__device__ __forceinline__ void kron_mfma8(const KSplit &S, const uint4 &q, float y[8]) {
    const bf16x8_t b = as_bf16x8(q);
    floatx4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(S.t[2][0], b, d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(S.t[2][1], b, d1, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(S.t[1][0], b, d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(S.t[1][1], b, d1, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(S.t[0][0], b, d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(S.t[0][1], b, d1, 0, 0, 0);
    y[0] = d0[0]; y[1] = d0[1]; y[2] = d0[2]; y[3] = d0[3];
    y[4] = d1[0]; y[5] = d1[1]; y[6] = d1[2]; y[7] = d1[3];
}

}  // namespace kq
