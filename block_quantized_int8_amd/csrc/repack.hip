// repack.hip - one-time, untimed repack of raw weight rows into matrix-core panels.
//
// The packed buffer keeps weights in their raw precision (nibbles stay nibbles, ternary codes
// stay 2-bit codes, int8 stays int8) and only reorders them so that one 64-lane load of a
// (32-row tile, 32-value block) fragment is the A operand of v_mfma_i32_32x32x32_i8, lane
// L = h*32 + r holding row r's values 16h..16h+15. Scales are gathered per (tile, block, row).
// Layouts: mmq_internal.h. Packing is a byte permutation (plus exact f32 scale products for
// Q4_K) done once, outside the timed region (metainfer "INT8 W8A8 GEMM - Prefill",
// section 3.2: one-time pack into a graph-stable buffer, validated by exact comparison).
#include <algorithm>

#include "mmq_internal.h"

namespace {

using namespace mmq;

__device__ inline uint16_t ld_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
__device__ inline float half_bits_to_float(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Every kernel: one thread per (tile nt, block b, lane L), NT*KBp*64 threads in total.
struct Lane {
    int64_t tb, nt, b, n;
    int h, r, L;
    bool live;                          // a real row and a real block
};

__device__ inline Lane lane_of(int64_t gid, int64_t KBp, int64_t KB, int64_t N) {
    Lane x;
    x.L = (int)(gid & 63);
    x.tb = gid >> 6;
    x.nt = x.tb / KBp;
    x.b = x.tb % KBp;
    x.h = x.L >> 5;
    x.r = x.L & 31;
    x.n = x.nt * 32 + x.r;
    x.live = x.n < N && x.b < KB;
    return x;
}

__global__ __launch_bounds__(256) void repack_q8_0_kernel(
    const uint8_t* __restrict__ raw, int64_t N, int64_t KB, int64_t KBp, int64_t total, int64_t gid0,
    uint8_t* __restrict__ frag, uint32_t* __restrict__ scale) {
    const int64_t gid = gid0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const Lane x = lane_of(gid, KBp, KB, N);
    uint32_t w[4] = {0, 0, 0, 0};
    uint16_t d = 0;
    if (x.live) {
        const uint8_t* blk = raw + (x.n * KB + x.b) * 34;
        d = ld_u16(blk);
        const uint8_t* q = blk + 2 + 16 * x.h;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)q[4 * i] | ((uint32_t)q[4 * i + 1] << 8) | ((uint32_t)q[4 * i + 2] << 16) |
                   ((uint32_t)q[4 * i + 3] << 24);
    }
    *reinterpret_cast<uint4*>(frag + gid * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    if (x.h == 0) scale[(x.nt * KBp + x.b) * 32 + x.r] = d;            // f16 d | 0 << 16
}

__global__ __launch_bounds__(256) void repack_q4_0_kernel(
    const uint8_t* __restrict__ raw, int64_t N, int64_t KB, int64_t KBp, int64_t total, int64_t gid0,
    uint8_t* __restrict__ frag, uint32_t* __restrict__ scale) {
    const int64_t gid = gid0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const Lane x = lane_of(gid, KBp, KB, N);
    uint32_t X0 = 0, X1 = 0;
    uint16_t d = 0;
    if (x.live) {
        const uint8_t* blk = raw + (x.n * KB + x.b) * 18;
        d = ld_u16(blk);
        // value 16h + i: nibble (qs[i] >> 4h) & 15; stored as the 4-bit two's complement of nib-8
        uint32_t t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = ((blk[2 + i] >> (4 * x.h)) & 0xFu) ^ 0x8u;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            X0 |= ((t[bb] << 4) | t[4 + bb]) << (8 * bb);
            X1 |= ((t[8 + bb] << 4) | t[12 + bb]) << (8 * bb);
        }
    }
    *reinterpret_cast<uint2*>(frag + gid * 8) = make_uint2(X0, X1);
    if (x.h == 0) scale[(x.nt * KBp + x.b) * 32 + x.r] = d;            // f16 d | 0 << 16
}

__global__ __launch_bounds__(256) void repack_q4_K_kernel(
    const uint8_t* __restrict__ raw, int64_t N, int64_t KB, int64_t KBp, int64_t total, int64_t gid0,
    uint8_t* __restrict__ frag, uint32_t* __restrict__ scale, float* __restrict__ mins) {
    const int64_t gid = gid0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const Lane x = lane_of(gid, KBp, KB, N);
    uint32_t X0 = 0, X1 = 0;
    uint32_t ds2 = 0;
    float dm = 0.f;
    if (x.live) {
        const int64_t sb = x.b / 8;
        const int j = (int)(x.b % 8);
        const uint8_t* blk = raw + (x.n * (KB / 8) + sb) * 144;
        const uint8_t* qs = blk + 16 + 16 * j;
        uint32_t nib[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) nib[i] = (qs[i] >> (4 * x.h)) & 0xFu;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            X0 |= (nib[bb] | (nib[4 + bb] << 4)) << (8 * bb);
            X1 |= (nib[8 + bb] | (nib[12 + bb] << 4)) << (8 * bb);
        }
        uint64_t scw = 0, mw = 0;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            scw |= (uint64_t)blk[4 + i] << (8 * i);
            mw |= (uint64_t)blk[10 + i] << (8 * i);
        }
        const int sc = (int)((scw >> (6 * j)) & 63u), mm = (int)((mw >> (6 * j)) & 63u);
        // d*sc is exact in f32 (11-bit significand x 6-bit integer); split it into two f16 with
        // hi + lo == d*sc exactly (the remainder has at most 6 significant bits)
        const float ds = half_bits_to_float(ld_u16(blk)) * (float)sc;
        const _Float16 hi = (_Float16)ds;
        const _Float16 lo = (_Float16)(ds - (float)hi);
        ds2 = (uint32_t)__builtin_bit_cast(uint16_t, hi) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
        dm = -(half_bits_to_float(ld_u16(blk + 2)) * (float)mm);
    }
    *reinterpret_cast<uint2*>(frag + gid * 8) = make_uint2(X0, X1);
    if (x.h == 0) {
        scale[(x.nt * KBp + x.b) * 32 + x.r] = ds2;
        mins[(x.nt * KBp + x.b) * 32 + x.r] = dm;
    }
}

__global__ __launch_bounds__(256) void repack_iq1t_kernel(
    const uint8_t* __restrict__ raw, int64_t N, int64_t KB, int64_t KBp, int64_t total, int64_t gid0,
    uint8_t* __restrict__ frag, uint8_t* __restrict__ scale) {
    const int64_t gid = gid0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const Lane x = lane_of(gid, KBp, KB, N);
    uint32_t C = 0, meta = 0;
    uint16_t d = 0;
    if (x.live) {
        const uint8_t* blk = raw + (x.n * (KB / 8) + x.b / 8) * 76;
        const int e0 = (int)(x.b % 8) * 32 + 16 * x.h;    // first of the lane's 16 values
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = e0 + i;
            const uint32_t c = (blk[e >> 2] >> (2 * (e & 3))) & 3u;
            C |= c << (8 * (i & 3) + 2 * (i >> 2));
        }
        uint64_t sw = 0;
#pragma unroll
        for (int i = 0; i < 6; ++i) sw |= (uint64_t)blk[64 + i] << (8 * i);
        const uint32_t s = (uint32_t)(sw >> (3 * (e0 >> 4))) & 7u;
        const int g0 = e0 >> 3, g1 = g0 + 1;               // the lane's two 8-value sign groups
        const uint32_t sg0 = (blk[70 + (g0 >> 3)] >> (g0 & 7)) & 1u;
        const uint32_t sg1 = (blk[70 + (g1 >> 3)] >> (g1 & 7)) & 1u;
        meta = s | (sg0 << 3) | (sg1 << 4);
        d = ld_u16(blk + 74);
    }
    *reinterpret_cast<uint32_t*>(frag + gid * 4) = C;
    // scale dword of (row, block): f16 d | meta0 << 16 | meta1 << 24 (meta_h from lane half h)
    uint8_t* e = scale + ((x.nt * KBp + x.b) * 32 + x.r) * 4;
    if (x.h == 0) {
        *reinterpret_cast<uint16_t*>(e) = d;
        e[2] = (uint8_t)meta;
    } else {
        e[3] = (uint8_t)meta;
    }
}

// q6_K: lane half h carries values 16h..16h+15 of the block as int8 q-32 (q = the low nibble
// from ql, plus the high 2 bits from qh, see mmq.h); the half's scale d*sc_h is exact in f32
// (f16 d times an int8) and is split exactly into two f16, hi + lo; lanes of half 0 write it to
// the first scale region, lanes of half 1 to the second.
__global__ __launch_bounds__(256) void repack_q6_K_kernel(
    const uint8_t* __restrict__ raw, int64_t N, int64_t KB, int64_t KBp, int64_t total, int64_t gid0,
    uint8_t* __restrict__ frag, uint32_t* __restrict__ scale, uint32_t* __restrict__ scale2) {
    const int64_t gid = gid0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const Lane x = lane_of(gid, KBp, KB, N);
    uint32_t w[4] = {0, 0, 0, 0};
    uint32_t ds2 = 0;
    if (x.live) {
        const uint8_t* blk = raw + (x.n * (KB / 8) + x.b / 8) * 210;
        const int j = (int)(x.b % 8);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int u = 16 * x.h + i;                        // value inside the 32-block
            const uint32_t lo = (blk[16 * j + i] >> (4 * x.h)) & 0xFu;
            const uint32_t hi = (blk[128 + 8 * j + (u & 7)] >> (2 * (u >> 3))) & 3u;
            const uint32_t v = (uint32_t)((int)(lo | (hi << 4)) - 32) & 0xFFu;
            w[i >> 2] |= v << (8 * (i & 3));
        }
        const int8_t sc = (int8_t)blk[192 + 2 * j + x.h];
        const float ds = half_bits_to_float(ld_u16(blk + 208)) * (float)sc;
        const _Float16 hi = (_Float16)ds;
        const _Float16 lo = (_Float16)(ds - (float)hi);
        ds2 = (uint32_t)__builtin_bit_cast(uint16_t, hi) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
    }
    *reinterpret_cast<uint4*>(frag + gid * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    uint32_t* dst = x.h == 0 ? scale : scale2;
    dst[(x.nt * KBp + x.b) * 32 + x.r] = ds2;
}

// The codebook formats keep their 11-bit grid indices in the packed form (grid-index panels):
// the GEMMs look every index up in the grid themselves, so the weights stream at the raw
// format's size (plus the per-lane meta bits) instead of as expanded 2-bit codes. Every launch
// piece writes, besides its lanes: the first threads, the grid spread into the IQ1T code order
// (value j of an entry at bits 8(j%4) + 2(j/4)); lanes h = 0 of every fourth block, the row's
// f16 d (one copy per 4-block group, the GEMMs' stage).
__device__ inline uint32_t spread_entry(uint32_t e) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= ((e >> (2 * j)) & 3u) << (8 * (j & 3) + 2 * (j >> 2));
    return w;
}

__device__ inline void write_grid(const uint16_t* __restrict__ grid, uint32_t* __restrict__ gtab, int64_t gid,
                                  int64_t total) {
    for (int64_t i = gid; i < GRID_ENTRIES; i += total) gtab[i] = spread_entry(grid[i]);
}

__device__ inline uint32_t grid_word(uint32_t ia, uint32_t ib, uint32_t meta) {
    return (ia << 2) | (meta << 13) | (ib << 20);
}

// IQ1C (the IQ1_M codebook form): the lane's 16 values are the 8-value groups q0 = e0/8 and
// q0 + 1; each group's 11-bit index is its qs byte plus bits 8-10 from its qh nibble, whose bit 3
// is the group's delta sign; s is the half's 3-bit sub-scale.
__global__ __launch_bounds__(256) void repack_iq1c_kernel(
    const uint8_t* __restrict__ raw, const uint16_t* __restrict__ grid, int64_t N, int64_t KB,
    int64_t KBp, int64_t total, int64_t gid0, uint8_t* __restrict__ frag, uint16_t* __restrict__ dreg,
    uint32_t* __restrict__ gtab) {
    const int64_t gid = gid0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    write_grid(grid, gtab, gid, total);
    const Lane x = lane_of(gid, KBp, KB, N);
    uint32_t W = 0;
    uint16_t d = 0;
    if (x.live) {
        const uint8_t* blk = raw + (x.n * (KB / 8) + x.b / 8) * 56;
        const int e0 = (int)(x.b % 8) * 32 + 16 * x.h;    // first of the lane's 16 values
        uint32_t idx[2], sg[2];
#pragma unroll
        for (int gq = 0; gq < 2; ++gq) {
            const int q = (e0 >> 3) + gq;
            const uint32_t nib = (blk[32 + (q >> 1)] >> (4 * (q & 1))) & 0xFu;
            idx[gq] = blk[q] | ((nib & 7u) << 8);
            sg[gq] = nib >> 3;
        }
        uint64_t sw = 0;
#pragma unroll
        for (int i = 0; i < 6; ++i) sw |= (uint64_t)blk[48 + i] << (8 * i);
        const uint32_t s = (uint32_t)(sw >> (3 * (e0 >> 4))) & 7u;
        W = grid_word(idx[0], idx[1], s | (sg[0] << 3) | (sg[1] << 4));
        d = ld_u16(blk + 54);
    }
    *reinterpret_cast<uint32_t*>(frag + gid * 4) = W;
    if (x.h == 0 && x.b % 4 == 0) dreg[(x.nt * (KBp / 4) + x.b / 4) * 32 + x.r] = d;
}

// IQ1S (the IQ1_S codebook form): as IQ1C, with the block's one s and one delta sign (its
// uint16 qh word) for both halves and all four groups.
__global__ __launch_bounds__(256) void repack_iq1s_kernel(
    const uint8_t* __restrict__ raw, const uint16_t* __restrict__ grid, int64_t N, int64_t KB,
    int64_t KBp, int64_t total, int64_t gid0, uint8_t* __restrict__ frag, uint16_t* __restrict__ dreg,
    uint32_t* __restrict__ gtab) {
    const int64_t gid = gid0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    write_grid(grid, gtab, gid, total);
    const Lane x = lane_of(gid, KBp, KB, N);
    uint32_t W = 0;
    uint16_t d = 0;
    if (x.live) {
        const uint8_t* blk = raw + (x.n * (KB / 8) + x.b / 8) * 50;
        const int j = (int)(x.b % 8);                      // the block inside the super-block
        const uint32_t qh = ld_u16(blk + 34 + 2 * j);
        uint32_t idx[2];
#pragma unroll
        for (int gq = 0; gq < 2; ++gq) {
            const int q = 2 * x.h + gq;                    // the lane's group inside the block
            idx[gq] = blk[2 + 4 * j + q] | (((qh >> (3 * q)) & 7u) << 8);
        }
        const uint32_t s = (qh >> 12) & 7u, sg = (qh >> 15) & 1u;
        W = grid_word(idx[0], idx[1], s | (sg << 3) | (sg << 4));
        d = ld_u16(blk);
    }
    *reinterpret_cast<uint32_t*>(frag + gid * 4) = W;
    if (x.h == 0 && x.b % 4 == 0) dreg[(x.nt * (KBp / 4) + x.b / 4) * 32 + x.r] = d;
}

__global__ __launch_bounds__(256) void repack_i8_row_kernel(
    const int8_t* __restrict__ raw, const float* __restrict__ row_scale, int64_t N, int64_t K,
    int64_t KB, int64_t KBp, int64_t total, int64_t gid0, uint8_t* __restrict__ frag, float* __restrict__ sw) {
    const int64_t gid = gid0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const Lane x = lane_of(gid, KBp, KB, N);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (x.live) v = *reinterpret_cast<const uint4*>(raw + x.n * K + x.b * 32 + 16 * x.h);
    *reinterpret_cast<uint4*>(frag + gid * 16) = v;
    if (x.b == 0 && x.h == 0) sw[x.n] = (x.n < N) ? row_scale[x.n] : 0.0f;
}

}  // namespace

namespace mmq {

hipError_t launch_repack(mmq_wtype t, const void* raw, const void* aux, int64_t N,
                         int64_t K, void* packed, hipStream_t s) {
    const PackedLayout L = packed_layout(t, N, K);
    uint8_t* base = static_cast<uint8_t*>(packed);
    uint8_t* frag = base + L.frag_off;
    uint8_t* scale = base + L.scale_off;
    // one thread per (tile, block, lane); launched in pieces of at most 2^30 threads so every
    // grid stays within the launch limits whatever the matrix size
    const int64_t total = L.NT * L.KBp * 64;
    constexpr int64_t PIECE = int64_t(1) << 30;
    const uint8_t* r8 = static_cast<const uint8_t*>(raw);
    for (int64_t g0 = 0; g0 < total; g0 += PIECE) {
    const dim3 grid((unsigned)ceil_div(std::min(PIECE, total - g0), 256)), block(256);
    switch (t) {
        case MMQ_Q8_0:
            hipLaunchKernelGGL(repack_q8_0_kernel, grid, block, 0, s, r8, N, L.KB, L.KBp, total, g0, frag,
                               reinterpret_cast<uint32_t*>(scale));
            break;
        case MMQ_Q4_0:
            hipLaunchKernelGGL(repack_q4_0_kernel, grid, block, 0, s, r8, N, L.KB, L.KBp, total, g0, frag,
                               reinterpret_cast<uint32_t*>(scale));
            break;
        case MMQ_Q4_K:
            hipLaunchKernelGGL(repack_q4_K_kernel, grid, block, 0, s, r8, N, L.KB, L.KBp, total, g0, frag,
                               reinterpret_cast<uint32_t*>(scale), reinterpret_cast<float*>(base + L.min_off));
            break;
        case MMQ_IQ1T:
            hipLaunchKernelGGL(repack_iq1t_kernel, grid, block, 0, s, r8, N, L.KB, L.KBp, total, g0, frag, scale);
            break;
        case MMQ_Q6_K:
            hipLaunchKernelGGL(repack_q6_K_kernel, grid, block, 0, s, r8, N, L.KB, L.KBp, total, g0, frag,
                               reinterpret_cast<uint32_t*>(scale), reinterpret_cast<uint32_t*>(base + L.min_off));
            break;
        case MMQ_IQ1S:
            hipLaunchKernelGGL(repack_iq1s_kernel, grid, block, 0, s, r8, static_cast<const uint16_t*>(aux), N,
                               L.KB, L.KBp, total, g0, frag, reinterpret_cast<uint16_t*>(scale),
                               reinterpret_cast<uint32_t*>(base + L.min_off));
            break;
        case MMQ_IQ1C:
            hipLaunchKernelGGL(repack_iq1c_kernel, grid, block, 0, s, r8, static_cast<const uint16_t*>(aux), N,
                               L.KB, L.KBp, total, g0, frag, reinterpret_cast<uint16_t*>(scale),
                               reinterpret_cast<uint32_t*>(base + L.min_off));
            break;
        case MMQ_I8_ROW:
            hipLaunchKernelGGL(repack_i8_row_kernel, grid, block, 0, s, static_cast<const int8_t*>(raw),
                               static_cast<const float*>(aux), N, K, L.KB, L.KBp, total, g0, frag,
                               reinterpret_cast<float*>(scale));
            break;
        default:
            return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mmq
