// gemm_common.h - small device helpers shared by the GEMM kernels.
#pragma once

#include "mmq_internal.h"

namespace mmq {

typedef float v16f_t __attribute__((ext_vector_type(16)));

__device__ inline _Float16 half_from_bits(uint16_t b) { return __builtin_bit_cast(_Float16, b); }

// f32 -> bf16, round to nearest even (finite inputs)
__device__ inline uint16_t bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Workgroup id -> logical tile id so that consecutive logical tiles run on the same XCD
// (workgroups are dealt round-robin to the 8 XCDs, each with its own L2).
__device__ inline int xcd_swizzle(int bid, int nblk) {
    const int q = nblk >> 3;
    if (bid < (q << 3)) return (bid & 7) * q + (bid >> 3);
    return bid;
}

// 32x32 accumulator lane map shared by every v_mfma_*_32x32x* instruction: lane l, register r
// holds row 8*(r/4) + 4*(l/32) + r%4 (the A-operand / weight side) and column l%32 (the
// B-operand / token side).
__device__ inline int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace mmq
