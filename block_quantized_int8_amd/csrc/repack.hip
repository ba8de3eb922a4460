// repack.hip - one-time, untimed repack of raw weight rows into matrix-core panels.
//
// The packed buffer keeps weights in their raw precision (nibbles stay nibbles, int8 stays
// int8) and only reorders them so that one 64-lane load of a (32-row tile, 32-value block)
// fragment is exactly the A operand of v_mfma_i32_32x32x32_i8 (lane L = h*32 + r holds row
// r's values 16h..16h+15). Scales are gathered per (tile, block, row). Layout details are in
// mmq_internal.h. Packing is a pure byte permutation done once, outside the timed region
// (metainfer "INT8 W8A8 GEMM - Prefill", section 3.2: one-time pack into a graph-stable
// buffer, validated by exact comparison).
#include "mmq_internal.h"

namespace {

__device__ inline uint16_t ld_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

// One thread per (tile nt, block b, lane L): grid covers NT*KBp*64 threads.
__global__ __launch_bounds__(256) void repack_q8_0_kernel(
    const uint8_t* __restrict__ raw, int64_t N, int64_t KB, int64_t KBp, int64_t NT,
    uint8_t* __restrict__ frag, uint16_t* __restrict__ scale) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= NT * KBp * 64) return;
    const int L = (int)(gid & 63);
    const int64_t tb = gid >> 6;                 // nt*KBp + b
    const int64_t nt = tb / KBp, b = tb % KBp;
    const int h = L >> 5, r = L & 31;
    const int64_t n = nt * 32 + r;
    uint32_t w[4] = {0, 0, 0, 0};
    uint16_t d = 0;
    if (n < N && b < KB) {
        const uint8_t* blk = raw + (n * KB + b) * 34;
        d = ld_u16(blk);
        const uint8_t* q = blk + 2 + 16 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)q[4 * i] | ((uint32_t)q[4 * i + 1] << 8) | ((uint32_t)q[4 * i + 2] << 16) |
                   ((uint32_t)q[4 * i + 3] << 24);
    }
    *reinterpret_cast<uint4*>(frag + gid * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    if (h == 0) scale[tb * 32 + r] = d;
}

__global__ __launch_bounds__(256) void repack_q4_0_kernel(
    const uint8_t* __restrict__ raw, int64_t N, int64_t KB, int64_t KBp, int64_t NT,
    uint8_t* __restrict__ frag, uint16_t* __restrict__ scale) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= NT * KBp * 64) return;
    const int L = (int)(gid & 63);
    const int64_t tb = gid >> 6;
    const int64_t nt = tb / KBp, b = tb % KBp;
    const int h = L >> 5, r = L & 31;
    const int64_t n = nt * 32 + r;
    uint32_t X0 = 0, X1 = 0;
    uint16_t d = 0;
    if (n < N && b < KB) {
        const uint8_t* blk = raw + (n * KB + b) * 18;
        d = ld_u16(blk);
        uint32_t t[16];                          // 4-bit two's complement of nib - 8
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = ((blk[2 + i] >> (4 * h)) & 0xFu) ^ 0x8u;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            X0 |= ((t[bb] << 4) | t[4 + bb]) << (8 * bb);
            X1 |= ((t[8 + bb] << 4) | t[12 + bb]) << (8 * bb);
        }
    }
    *reinterpret_cast<uint2*>(frag + gid * 8) = make_uint2(X0, X1);
    if (h == 0) scale[tb * 32 + r] = d;
}

__global__ __launch_bounds__(256) void repack_i8_row_kernel(
    const int8_t* __restrict__ raw, const float* __restrict__ row_scale, int64_t N, int64_t K,
    int64_t KB, int64_t KBp, int64_t NT, uint8_t* __restrict__ frag, float* __restrict__ sw) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= NT * KBp * 64) return;
    const int L = (int)(gid & 63);
    const int64_t tb = gid >> 6;
    const int64_t nt = tb / KBp, b = tb % KBp;
    const int h = L >> 5, r = L & 31;
    const int64_t n = nt * 32 + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < N && b < KB) v = *reinterpret_cast<const uint4*>(raw + n * K + b * 32 + 16 * h);
    *reinterpret_cast<uint4*>(frag + gid * 16) = v;
    if (b == 0 && h == 0) sw[n] = (n < N) ? row_scale[n] : 0.0f;
}

}  // namespace

namespace mmq {

hipError_t launch_repack(mmq_wtype t, const void* raw, const float* row_scale, int64_t N,
                         int64_t K, void* packed, hipStream_t s) {
    const PackedLayout L = packed_layout(t, N, K);
    uint8_t* base = static_cast<uint8_t*>(packed);
    const int64_t threads = L.NT * L.KBp * 64;
    const dim3 grid((unsigned)ceil_div(threads, 256));
    const uint8_t* r8 = static_cast<const uint8_t*>(raw);
    switch (t) {
        case MMQ_Q8_0:
            hipLaunchKernelGGL(repack_q8_0_kernel, grid, dim3(256), 0, s, r8, N, L.KB, L.KBp, L.NT,
                               base + L.frag_off, reinterpret_cast<uint16_t*>(base + L.scale_off));
            break;
        case MMQ_Q4_0:
            hipLaunchKernelGGL(repack_q4_0_kernel, grid, dim3(256), 0, s, r8, N, L.KB, L.KBp, L.NT,
                               base + L.frag_off, reinterpret_cast<uint16_t*>(base + L.scale_off));
            break;
        case MMQ_I8_ROW:
            hipLaunchKernelGGL(repack_i8_row_kernel, grid, dim3(256), 0, s,
                               static_cast<const int8_t*>(raw), row_scale, N, K, L.KB, L.KBp, L.NT,
                               base + L.frag_off, reinterpret_cast<float*>(base + L.scale_off));
            break;
        default:
            return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace mmq
