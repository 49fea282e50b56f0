// bf16 staging of the low-rank branch's operands (KroQuant, arXiv 2607.21446v1,
// Sec. 3.4 Eq. 11) on gfx950's hardware converts: the hi + lo split of fp32 Z
// and the decode of MXFP4 L or R, each one instruction per pair of values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_device.hpp"

namespace kq {

// fp32 x = hi + lo + e with hi = bf16(x), lo = bf16(x - hi), both rounded to nearest
// even by the hardware convert (x - hi is exact in fp32): the same split as
// split_bf16x8, one convert per value instead of the integer rounding steps.
__device__ __forceinline__ void split_bf16x8_cvt(const float x[8], bf16x8_t &hi, bf16x8_t &lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const __bf16 h = (__bf16)x[i];
        hi[i] = h;
        lo[i] = (__bf16)(x[i] - (float)h);
    }
}

// deq of 8 E2M1 codes (element i in nibble i) under E8M0 scale byte sbyte, in bf16,
// bit-identical to decode_fp4x8_bf16. Every value is lvl * 2^(sbyte - 127) with lvl
// in {0, 0.5, ..., 6}, a normal bf16 (so exact in the scaled convert) for scale bytes
// 2..252; the rest (sub-normal, overflowing and NaN scales) take the arithmetic decode.
__device__ __forceinline__ bf16x8_t decode_fp4x8_bf16_cvt(uint32_t c8, uint32_t sbyte) {
    if (sbyte < 2u || sbyte > 252u) return decode_fp4x8_bf16(c8, sbyte);
    const float scale = __uint_as_float(sbyte << 23);
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c8, scale, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c8, scale, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c8, scale, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c8, scale, 3);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

}  // namespace kq
