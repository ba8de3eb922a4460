// quantize.hip - f32 activations -> q8_1 (per 32-value block) and per-token int8.
//
// q8_1 per block (minfer "08 . R1 - int8 MMQ prefill GEMM", section 3.2 CPU reference and
// section 2.2): amax = max|x|; d = amax/127 in f32; di = 1/d (0 when d = 0, the largest finite
// f32 when 1/d overflows);
// q = clamp(round-half-even(x*di), -128, 127); stored scale = d rounded to f16; the block's
// integer sum is written alongside. Division is IEEE-correct (built with
// -fhip-fp32-correctly-rounded-divide-sqrt) and nothing is contracted, so the result is
// bit-identical to the definition.
//
// Work split: a unit is (32-row tile, pair of blocks); each wave walks several units, loading
// the next one before it quantises and stores the current one, so loads and stores overlap
// (with one unit per wave the whole grid would load, then store, in lockstep). In a unit, lane
// L = h*32 + r owns row r's values 16h..16h+15 of each block - exactly the 16 bytes it writes
// to the tiled xq layout and the two 8-value groups whose sums it writes to xg, so every
// block's 1 KB of xq and 256 B of xg are contiguous wave stores. The two lanes of a block (r
// and r+32) combine their half-block max and sum with one cross-half exchange. Lanes h = 0
// write the block's xs2 (f16 pair), lanes h = 1 its xsx = xs * xsum (exact in f32: an 11-bit
// significand times a |sum| <= 32*128), each a tile-major 128-byte line per block.
#include <algorithm>

#include "mmq_internal.h"

namespace {

constexpr int QG = 2;             // blocks per wave (one 32-row tile x 64 values)
constexpr int QWAVES = 16;        // waves per workgroup at most (the launch bound)
constexpr int QWAVES_TOTAL = 4096;  // waves in the grid at most (16 per CU); waves then loop over units

__device__ inline uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

// 1/d, 0 for d = 0, and the largest finite f32 where 1/d overflows (d below 2^-128: a block
// whose amax is under ~3.7e-37), so that 0 * di stays 0 and |x * di| stays within 127(1 + 2^-23)
__device__ inline float inverse_scale(float d) {
    return d != 0.0f ? fminf(1.0f / d, 3.40282347e38f) : 0.0f;
}

__device__ inline int q_of(float x, float di) {
    return (int)fminf(fmaxf(__builtin_rintf(x * di), -128.f), 127.f);
}

// an integer group sum |g| <= 1024 as the f16 bits of g * 2^-13 (exact: normal, 11 bits)
__device__ inline uint32_t group_half(int g) {
    return __builtin_bit_cast(uint16_t, (_Float16)((float)g * 0.0001220703125f));
}

__global__ __launch_bounds__(QWAVES * 64) void quantize_q8_1_kernel(
    const float* __restrict__ x, int64_t M, int64_t KB, int64_t ldx, int64_t KBp, int64_t units,
    int8_t* __restrict__ xq, uint32_t* __restrict__ xs2, float* __restrict__ xsx,
    uint32_t* __restrict__ xg) {
    const int lane = threadIdx.x & 63;
    const int nw = (int)(blockDim.x >> 6);                  // waves per workgroup
    const int64_t stride = (int64_t)gridDim.x * nw;
    int64_t u = (int64_t)blockIdx.x * nw + (threadIdx.x >> 6);
    if (u >= units) return;                                 // uniform per wave
    const int64_t G = KBp / QG;
    const int r = lane & 31, h = lane >> 5;

    auto load = [&](int64_t uu, float4 (&v)[QG][4]) __attribute__((always_inline)) {
        const int64_t mt = uu / G, kb0 = (uu % G) * QG;
        const int64_t m = mt * 32 + r;
#pragma unroll
        for (int i = 0; i < QG; ++i) {
            const bool ok = m < M && kb0 + i < KB;
            const float* p = x + m * ldx + (kb0 + i) * 32 + 16 * h;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                v[i][c] = ok ? *reinterpret_cast<const float4*>(p + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto process = [&](int64_t uu, const float4 (&v)[QG][4]) __attribute__((always_inline)) {
        const int64_t mt = uu / G, kb0 = (uu % G) * QG;
        float s_xs[QG];
        int s_sum[QG];
#pragma unroll
        for (int i = 0; i < QG; ++i) {
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i][c].x), fabsf(v[i][c].y)),
                                         fmaxf(fabsf(v[i][c].z), fabsf(v[i][c].w))));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const float d = amax / 127.0f;
            const float di = inverse_scale(d);
            uint32_t w[4];
            int gs[2] = {0, 0};                  // the lane's two 8-value groups
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int a = q_of(v[i][c].x, di), b = q_of(v[i][c].y, di);
                const int e = q_of(v[i][c].z, di), f = q_of(v[i][c].w, di);
                gs[c >> 1] += a + b + e + f;
                w[c] = pack4(a, b, e, f);
            }
            int sum = gs[0] + gs[1];
            sum += __shfl_xor(sum, 32);
            const int64_t blk = (mt * KBp + kb0 + i) * 64 + lane;
            *reinterpret_cast<uint4*>(xq + blk * 16) = make_uint4(w[0], w[1], w[2], w[3]);
            xg[blk] = group_half(gs[0]) | (group_half(gs[1]) << 16);
            s_xs[i] = (float)(_Float16)d;
            s_sum[i] = sum;
        }
        // tile-major [MT][KBp][32]: the 32 rows of a block are one 128-byte line
#pragma unroll
        for (int i = 0; i < QG; ++i) {
            const int64_t tix = (mt * KBp + kb0 + i) * 32 + r;
            if (h == 0) {
                const uint32_t b = __builtin_bit_cast(uint16_t, (_Float16)s_xs[i]);
                xs2[tix] = b | (b << 16);
            } else {
                xsx[tix] = s_xs[i] * (float)s_sum[i];
            }
        }
    };

    // each wave walks its units with the next unit's loads in flight while it quantises and
    // stores the current one
    float4 va[QG][4], vb[QG][4];
    load(u, va);
    for (;;) {
        const int64_t u1 = u + stride;
        if (u1 < units) load(u1, vb);
        process(u, va);
        if (u1 >= units) break;
        const int64_t u2 = u1 + stride;
        if (u2 < units) load(u2, va);
        process(u1, vb);
        if (u2 >= units) break;
        u = u2;
    }
}

// Per-token int8: one CTA per row (grid-stride over the Mp rows); amax over the whole row,
// then q = rint(x * (1/d)), scale kept in f32 (metainfer "INT8 W8A8 GEMM - Prefill", section
// 1 operator contract). The values go to the tiled layout (4 bytes per thread inside one
// lane's 16-byte run); rows m >= M and blocks past K/32 are written as zeros.
__global__ __launch_bounds__(256) void quantize_i8_token_kernel(
    const float* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int64_t KBp,
    int8_t* __restrict__ a, float* __restrict__ sa) {
    __shared__ float red[4];
    const int64_t Mp = (M + 31) & ~(int64_t)31;
    for (int64_t m = blockIdx.x; m < Mp; m += gridDim.x) {
        const bool live = m < M;
        const float* row = x + (live ? m : 0) * ldx;
        float amax = 0.f;
        if (live) {
            for (int64_t k = (int64_t)threadIdx.x * 4; k < K; k += 1024) {
                float4 v = *reinterpret_cast<const float4*>(row + k);
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const float d = amax / 127.0f;
        const float di = inverse_scale(d);
        uint8_t* tile = reinterpret_cast<uint8_t*>(a) + (m >> 5) * KBp * 1024;
        const int r = (int)(m & 31);
        for (int64_t k = (int64_t)threadIdx.x * 4; k < KBp * 32; k += 1024) {
            uint32_t w = 0;
            if (live && k < K) {
                float4 v = *reinterpret_cast<const float4*>(row + k);
                w = pack4(q_of(v.x, di), q_of(v.y, di), q_of(v.z, di), q_of(v.w, di));
            }
            const int kk = (int)(k & 31);
            *reinterpret_cast<uint32_t*>(tile + (((k >> 5) * 64 + (kk >> 4) * 32 + r) * 16 + (kk & 15))) = w;
        }
        if (threadIdx.x == 0) sa[m] = d;
        __syncthreads();                  // red[] is reused by the next row
    }
}

}  // namespace

namespace mmq {

hipError_t launch_quantize_q8_1(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                hipStream_t s) {
    static_assert(KB_ALIGN % QG == 0, "block padding must be whole wave groups");
    const ActQ81Layout L = act_q8_1_layout(M, K);
    uint8_t* base = static_cast<uint8_t*>(act);
    const int64_t units = L.MT * (L.KBp / QG);
    // 16-wave workgroups when there is a unit per wave for 16 waves on every CU (measured 2%
    // faster than 4-wave ones on 2048 x 4096), else 4-wave ones so that small inputs still
    // spread over all CUs
    const int nw = units >= QWAVES_TOTAL ? QWAVES : 4;
    const dim3 grid((unsigned)std::min<int64_t>(ceil_div(units, nw), QWAVES_TOTAL / nw));
    hipLaunchKernelGGL(quantize_q8_1_kernel, grid, dim3(nw * 64), 0, s, x, M, L.KB, ldx, L.KBp,
                       units, reinterpret_cast<int8_t*>(base + L.xq_off),
                       reinterpret_cast<uint32_t*>(base + L.xs2_off),
                       reinterpret_cast<float*>(base + L.xsx_off),
                       reinterpret_cast<uint32_t*>(base + L.xg_off));
    return hipGetLastError();
}

hipError_t launch_quantize_i8_token(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                    hipStream_t s) {
    const ActI8Layout L = act_i8_layout(M, K);
    uint8_t* base = static_cast<uint8_t*>(act);
    const unsigned grid = (unsigned)std::min<int64_t>(L.Mp, 65536);
    hipLaunchKernelGGL(quantize_i8_token_kernel, dim3(grid), dim3(256), 0, s, x, M, K, ldx,
                       L.KBp, reinterpret_cast<int8_t*>(base + L.a_off),
                       reinterpret_cast<float*>(base + L.sa_off));
    return hipGetLastError();
}

}  // namespace mmq
