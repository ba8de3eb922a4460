// quantize.hip - f32 activations -> q8_1 (per 32-value block) and per-token int8.
//
// q8_1 per block (minfer "08 . R1 - int8 MMQ prefill GEMM", section 3.2 CPU reference and
// section 2.2): amax = max|x|; d = amax/127 in f32; di = 1/d (0 when d = 0);
// q = clamp(round-half-even(x*di), -128, 127); stored scale = d rounded to f16; the block's
// integer sum is written alongside. Division is IEEE-correct (built with
// -fhip-fp32-correctly-rounded-divide-sqrt) and nothing is contracted, so the result is
// bit-identical to the definition.
//
// The q8_1 output is written directly in the matrix-core tile order the GEMM consumes
// (see mmq.h, region 0), so the GEMM streams whole fragments straight into LDS; xs is also
// written as f16 bits (region 3, exact: xs is f16-rounded by definition), the form the GEMM's
// scale outer product consumes.
#include "mmq_internal.h"

namespace {

constexpr int QROWS = 32;     // rows per CTA (one row tile)
constexpr int QBLK = 8;       // 32-value blocks per CTA along K (256 values)

// One CTA = 32 rows x 8 blocks. Thread t: row r = t/8, lane-in-block j = t%8 holds the four
// values 4j..4j+3 of each of the 8 blocks, so each load instruction reads 128 contiguous
// bytes per row. Block reductions are over the 8 consecutive lanes of a row.
__global__ __launch_bounds__(256) void quantize_q8_1_kernel(
    const float* __restrict__ x, int64_t M, int64_t KB, int64_t ldx, int64_t KBp,
    int8_t* __restrict__ xq, float* __restrict__ xs, int32_t* __restrict__ xsum,
    uint16_t* __restrict__ xs16) {
    const int t = threadIdx.x;
    const int r = t >> 3;
    const int j = t & 7;
    const int64_t mt = blockIdx.y;
    const int64_t m = mt * QROWS + r;
    const int64_t kb0 = (int64_t)blockIdx.x * QBLK;
    const bool row_ok = m < M;

    float4 v[QBLK];
#pragma unroll
    for (int i = 0; i < QBLK; ++i) {
        const int64_t kb = kb0 + i;
        if (row_ok && kb < KB) {
            v[i] = *reinterpret_cast<const float4*>(x + m * ldx + kb * 32 + 4 * j);
        } else {
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }

#pragma unroll
    for (int i = 0; i < QBLK; ++i) {
        const int64_t kb = kb0 + i;
        if (kb >= KBp) break;   // uniform across the CTA
        float amax = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));
        const float d = amax / 127.0f;
        const float di = (d != 0.0f) ? 1.0f / d : 0.0f;
        float q0 = fminf(fmaxf(__builtin_rintf(v[i].x * di), -128.f), 127.f);
        float q1 = fminf(fmaxf(__builtin_rintf(v[i].y * di), -128.f), 127.f);
        float q2 = fminf(fmaxf(__builtin_rintf(v[i].z * di), -128.f), 127.f);
        float q3 = fminf(fmaxf(__builtin_rintf(v[i].w * di), -128.f), 127.f);
        const int iq0 = (int)q0, iq1 = (int)q1, iq2 = (int)q2, iq3 = (int)q3;
        int s = iq0 + iq1 + iq2 + iq3;
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        const uint32_t packed = (uint32_t)(iq0 & 0xFF) | ((uint32_t)(iq1 & 0xFF) << 8) |
                                ((uint32_t)(iq2 & 0xFF) << 16) | ((uint32_t)(iq3 & 0xFF) << 24);
        const int64_t tile = mt * KBp + kb;
        const int h = j >> 2;                       // values 4j..4j+3 sit in half h = j/4
        uint32_t* dst = reinterpret_cast<uint32_t*>(xq + tile * 1024 + (h * 32 + r) * 16 + 4 * (j & 3));
        *dst = packed;
        if (j == 0) {
            const _Float16 dh = (_Float16)d;
            xs[tile * 32 + r] = (float)dh;
            xsum[tile * 32 + r] = s;
            xs16[tile * 32 + r] = __builtin_bit_cast(uint16_t, dh);
        }
    }
}

// Per-token int8: one CTA per row; amax over the whole row, then q = rint(x * (1/d)),
// scale kept in f32 (metainfer "INT8 W8A8 GEMM - Prefill", section 1 operator contract).
__global__ __launch_bounds__(256) void quantize_i8_token_kernel(
    const float* __restrict__ x, int64_t K, int64_t ldx, int8_t* __restrict__ a,
    float* __restrict__ sa) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const float* row = x + m * ldx;
    float amax = 0.f;
    for (int64_t k = (int64_t)threadIdx.x * 4; k < K; k += 1024) {
        float4 v = *reinterpret_cast<const float4*>(row + k);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float d = amax / 127.0f;
    const float di = (d != 0.0f) ? 1.0f / d : 0.0f;
    for (int64_t k = (int64_t)threadIdx.x * 4; k < K; k += 1024) {
        float4 v = *reinterpret_cast<const float4*>(row + k);
        int q0 = (int)fminf(fmaxf(__builtin_rintf(v.x * di), -128.f), 127.f);
        int q1 = (int)fminf(fmaxf(__builtin_rintf(v.y * di), -128.f), 127.f);
        int q2 = (int)fminf(fmaxf(__builtin_rintf(v.z * di), -128.f), 127.f);
        int q3 = (int)fminf(fmaxf(__builtin_rintf(v.w * di), -128.f), 127.f);
        *reinterpret_cast<uint32_t*>(a + m * K + k) =
            (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
            ((uint32_t)(q3 & 0xFF) << 24);
    }
    if (threadIdx.x == 0) sa[m] = d;
}

}  // namespace

namespace mmq {

hipError_t launch_quantize_q8_1(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                hipStream_t s) {
    const ActQ81Layout L = act_q8_1_layout(M, K);
    uint8_t* base = static_cast<uint8_t*>(act);
    dim3 grid((unsigned)(L.KBp / QBLK), (unsigned)L.MT);
    hipLaunchKernelGGL(quantize_q8_1_kernel, grid, dim3(256), 0, s, x, M, L.KB, ldx, L.KBp,
                       reinterpret_cast<int8_t*>(base + L.xq_off),
                       reinterpret_cast<float*>(base + L.xs_off),
                       reinterpret_cast<int32_t*>(base + L.xsum_off),
                       reinterpret_cast<uint16_t*>(base + L.xs16_off));
    return hipGetLastError();
}

hipError_t launch_quantize_i8_token(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                    hipStream_t s) {
    const ActI8Layout L = act_i8_layout(M, K);
    uint8_t* base = static_cast<uint8_t*>(act);
    hipLaunchKernelGGL(quantize_i8_token_kernel, dim3((unsigned)M), dim3(256), 0, s, x, K, ldx,
                       reinterpret_cast<int8_t*>(base + L.a_off),
                       reinterpret_cast<float*>(base + L.sa_off));
    return hipGetLastError();
}

}  // namespace mmq
