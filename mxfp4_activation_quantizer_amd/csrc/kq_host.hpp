// Host-side helpers shared by the library's translation units: argument
// checks (run before any HIP call) and the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

#include "kq.h"

namespace kqhost {

// hipError_t of the last KQ_ERR_HIP on this host thread (kq_last_hip_error).
inline thread_local int g_last_hip_error = 0;

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks common to every [m][ld] x d operand.
inline kq_status check_shape(int64_t m, int64_t d, int64_t ld) {
    if (m < 0 || d < 0 || ld < 0) return KQ_ERR_SHAPE;
    if (d % 32 != 0) return KQ_ERR_SHAPE;
    if (ld < d) return KQ_ERR_SHAPE;
    if (d / 32 > (int64_t)0x7FFFFFFF) return KQ_ERR_SHAPE;
    if (ld > 0 && m > INT64_MAX / 4 / ld) return KQ_ERR_SHAPE;  // byte offsets of fp32 rows fit
    return KQ_OK;
}

// bf16 input [m][lda] and MXFP4 outputs: pointers present, 16-byte rows.
inline kq_status check_bf16_io(const uint16_t *A, int64_t lda, const uint8_t *codes, const uint8_t *scales) {
    if (!A || !codes || !scales) return KQ_ERR_NULL;
    if (!aligned(A, 16) || lda % 8 != 0 || !aligned(codes, 16)) return KQ_ERR_ALIGN;
    return KQ_OK;
}

// Sizes the GEMM-family launches multiply together: each must be below 2^31,
// so that any product of two of them (times a small constant) stays far
// inside int64 before the finer limits are checked.
inline bool sizes_fit(std::initializer_list<int64_t> v) {
    for (const int64_t x : v)
        if (x >= ((int64_t)1 << 31)) return false;
    return true;
}

// Status of the launch just enqueued.
inline kq_status launched() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return KQ_ERR_HIP;
    }
    return KQ_OK;
}

}  // namespace kqhost
