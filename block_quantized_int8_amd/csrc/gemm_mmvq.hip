// gemm_mmvq.hip - the decode form of the MMQ contraction: batches of at most 16 token rows.
//
//   out[m,n] = sum_b (xs[m,b] * wd[n,b]) * P[m,n,b],   P = sum_{k in b} xq[m,k] * wq[n,k]
//
// The same contraction as the prefill kernels, on the same packed weights and q8_1 (or
// per-token int8) activations. A prefill tile sized for hundreds of tokens is mostly empty at
// a batch of a few tokens: a decode-shaped problem wastes all but one row of a 16-token
// matrix fragment (minfer "08 . R1", section 2.1), and llama.cpp keeps such batches (n <= 8)
// on a separate matrix-vector kernel, MMVQ ("CUDA: add IQ1_M to MMQ", PR #304, Summary). With
// so few tokens the work is bound by one pass over the weights, and the kernel is built for
// that:
//  * a workgroup owns 16 weight rows and its 16 waves split the blocks of K (chunks of 4
//    blocks dealt round-robin), so N = 4096 already gives 256 workgroups of 16 waves; a wave
//    keeps one chunk's loads in flight while it computes the previous one;
//  * every lane loads its operands straight from the packed panels into registers (no LDS
//    staging): the weight side of v_mfma_i32_16x16x32_i8 is 8 values of one row, which the
//    packed fragment keeps contiguous;
//  * tokens are the A side, so accumulator register v of lane l holds token 4*(l/16) + v and
//    row l%16 (the 16x16 accumulator lane map); with M <= 4 only registers v < M hold tokens
//    and only those are rescaled;
//  * per block: the exact int32 dot P (two chained MFMAs for iq1t's folded per-16 factor, as
//    in the prefill kernel), the scale product S = xs * wd from one f16 MFMA (exact: a product
//    of two f16; q4_K's d*sc arrives as an exact f16 pair), then acc += f32(P) * S on the live
//    registers. q4_K adds its rank-1 min term -(dmin*m) * (xs*xsum) four blocks at a time with
//    one f32 MFMA (minfer R1 section 2.2). W8A8 has no per-block scale: its int32 accumulator
//    runs through the whole of K and the epilogue applies the two per-row scales (metainfer
//    "INT8 W8A8 GEMM - Prefill", section 1);
//  * the 16 waves' partial sums meet in LDS and are added in wave order: deterministic, with
//    no atomics and no workspace.
#include <algorithm>

#include "gemm_common.h"

namespace mmq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int MV_W = 16;          // waves per workgroup (they split the blocks of K)
constexpr int MV_CH = 4;          // blocks per chunk: the unit of a wave's loads
constexpr int MV_ROWS = 16;       // weight rows per workgroup
static_assert(KB_ALIGN % MV_CH == 0, "chunks tile the padded block count");
static_assert(MV_CH % 4 == 0, "the q4_K min term takes four blocks per MFMA");

__device__ inline long pk2(uint32_t lo, uint32_t hi) {
    return (long)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// Buffer loads: a wave-uniform descriptor (base, byte range) in scalar registers plus a 32-bit
// lane offset; the hardware returns zero past the range, and no vector registers go to 64-bit
// address arithmetic (which would tie them to loads still in flight).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_W3 = 0x00020000;        // descriptor word 3: raw 32-bit data format (gfx9)
__device__ inline rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, RSRC_W3);
}
__device__ inline uint32_t ld32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ inline uint2 ld64(rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v[0], v[1]);
}

// an f16x4 operand with the dword `lo` in slots 0-1 and zeros in slots 2-3
__device__ inline h4 as_h4(uint32_t lo) {
    const v2i t = {(int)lo, 0};
    return __builtin_bit_cast(h4, t);
}

// Per weight format: where lane (row n of the tile, k-group g) finds its 8 values 8g..8g+7 of
// a block inside the (tile, block) fragment, how they become int8 MFMA operands, and the power
// of two the integer dot carries (POST undoes it).
template <mmq_wtype FMT> struct VQ;

// q8_0: lane h*32 + r of the fragment holds row r's int8 values 16h..16h+15.
template <> struct VQ<MMQ_Q8_0> {
    static constexpr int FB = 1024, NMF = 1;
    static constexpr bool MIN = false, ROW = false;
    static constexpr float POST = 1.0f;
    typedef uint2 Raw;
    __device__ static int off(int n, int g) { return ((g >> 1) * 32 + n) * 16 + (g & 1) * 8; }
    __device__ static Raw load(rsrc_t r, uint32_t off) { return ld64(r, off); }
    __device__ static void ops(Raw r, uint32_t, int, const uint2*, long* b) { b[0] = pk2(r.x, r.y); }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }
};

// per-channel int8: the q8_0 fragment layout, one f32 scale per row instead of per block
template <> struct VQ<MMQ_I8_ROW> : VQ<MMQ_Q8_0> {
    static constexpr bool ROW = true;
};

// q4_0: 8 bytes per fragment lane; dword X(g&1) holds the lane's 8 values as the 4-bit two's
// complement of nib - 8 (values +0..3 in the high nibbles, +4..7 in the low ones), so the
// masked bytes are int8 16*(nib-8).
template <> struct VQ<MMQ_Q4_0> {
    static constexpr int FB = 512, NMF = 1;
    static constexpr bool MIN = false, ROW = false;
    static constexpr float POST = 1.0f / 16;
    typedef uint32_t Raw;
    __device__ static int off(int n, int g) { return ((g >> 1) * 32 + n) * 8 + (g & 1) * 4; }
    __device__ static Raw load(rsrc_t r, uint32_t off) { return ld32(r, off); }
    __device__ static void ops(Raw r, uint32_t, int, const uint2*, long* b) {
        b[0] = pk2(r & 0xF0F0F0F0u, (r << 4) & 0xF0F0F0F0u);
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }
};

// q4_K: unsigned nibbles, values +0..3 in the low nibbles of the lane's dword, +4..7 in the
// high ones; the scale dword is the exact f16 pair (hi, lo) of d*sc, the min region -dmin*m.
template <> struct VQ<MMQ_Q4_K> {
    static constexpr int FB = 512, NMF = 1;
    static constexpr bool MIN = true, ROW = false;
    static constexpr float POST = 1.0f;
    typedef uint32_t Raw;
    __device__ static int off(int n, int g) { return ((g >> 1) * 32 + n) * 8 + (g & 1) * 4; }
    __device__ static Raw load(rsrc_t r, uint32_t off) { return ld32(r, off); }
    __device__ static void ops(Raw r, uint32_t, int, const uint2*, long* b) {
        b[0] = pk2(r & 0x0F0F0F0Fu, (r >> 4) & 0x0F0F0F0Fu);
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }
};

// iq1t: one dword of 2-bit codes per fragment lane (value 16h + 4q + b at bits 8b + 2q), so
// the lane's values 8(g&1) + j sit at q = 2(g&1) + j/4, b = j%4. The lane's half h = g/2 has
// the meta byte s | sigma0 << 3 | sigma1 << 4 in its scale dword (byte 2 + h), and its 8
// values are sign group g&1 of that half. The IQ1_M fold (llama.cpp PR #304, Design) makes
// each value the integer v = 8(c-1) + sigma (sigma = +-1) under the per-16 factor (2s+1) and
// the scale d/8; (2s+1)*v is split as 2s*v + v (|2s*v| <= 126) over two int8 MFMAs.
// tab[s | sign << 3] = (byte LUT code -> v, byte LUT code -> 2s*v).
template <> struct VQ<MMQ_IQ1T> {
    static constexpr int FB = 256, NMF = 2;
    static constexpr bool MIN = false, ROW = false;
    static constexpr float POST = 1.0f / 8;
    typedef uint32_t Raw;
    __device__ static int off(int n, int g) { return ((g >> 1) * 32 + n) * 4; }
    __device__ static Raw load(rsrc_t r, uint32_t off) { return ld32(r, off); }
    __device__ static void ops(Raw r, uint32_t wsd, int g, const uint2* tab, long* b) {
        const uint32_t meta = (wsd >> (16 + 8 * (g >> 1))) & 0xFFu;
        const uint32_t e = (meta & 7u) | (((meta >> (3 + (g & 1))) & 1u) << 3);
        const uint2 t = tab[e];
        const uint32_t sh = 4u * (uint32_t)(g & 1);
        const uint32_t s0 = (r >> sh) & 0x03030303u, s1 = (r >> (sh + 2)) & 0x03030303u;
        b[0] = pk2(__builtin_amdgcn_perm(0u, t.y, s0), __builtin_amdgcn_perm(0u, t.y, s1));
        b[1] = pk2(__builtin_amdgcn_perm(0u, t.x, s0), __builtin_amdgcn_perm(0u, t.x, s1));
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w & 0xFFFFu; }   // f16 d only
    __device__ static uint2 table(int e) {
        const int s = e & 7, sg = (e >> 3) ? -1 : 1;
        uint32_t v = 0, v2 = 0;
        for (int c = 0; c < 3; ++c) {
            const int x = 8 * (c - 1) + sg;
            v |= (uint32_t)(x & 0xFF) << (8 * c);
            v2 |= (uint32_t)((2 * s * x) & 0xFF) << (8 * c);
        }
        return make_uint2(v, v2);
    }
};

struct MvArgs {
    const uint8_t* w;           // packed weights
    int64_t w_scale_off;        // scale region (per-row f32 sw for W8A8)
    int64_t w_min_off;          // q4_K min region
    const uint8_t* xq;          // act region 0: tiled int8 values (token tile 0)
    const uint32_t* xs2;        // q8_1 region 3: xs as an f16 pair, tile-major
    const float* xsx;           // q8_1 region 4: xs * xsum, tile-major
    const float* sa;            // i8_token region 1: per-token scale
    int M, N, KBp, groups;      // groups: 16-row groups of the padded weight rows
    void* out;
    int64_t ldo;
};

// LDS barrier that leaves global loads in flight (__syncthreads() would also wait for them)
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Persistent workgroups: workgroup b handles the 16-row groups b, b + gridDim.x, ... (group q
// = rows 16q..16q+15 = half q&1 of tile q/2), all M <= 16 tokens, all of K. Each wave's work is
// one stream of items (group, chunk), its chunks being wave, wave + MV_W, ... of every group;
// loads run two items ahead across group boundaries, so the memory pipe does not drain while
// a group is reduced. NR = accumulator registers that hold a live token.
template <mmq_wtype FMT, int NR>
__global__ __launch_bounds__(MV_W * 64) void mmvq_kernel(MvArgs a) {
    using T = VQ<FMT>;
    __shared__ float red[2][MV_W][4][64];
    __shared__ uint2 tab[16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;

    if constexpr (FMT == MMQ_IQ1T) {
        if (tid < 16) tab[tid] = T::table(tid);
        __syncthreads();
    }
    const int KBp = a.KBp;
    const int nch = KBp / MV_CH;
    const int ng = (a.groups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;   // >= 1
    const int cw = wave < nch ? (nch - wave + MV_W - 1) / MV_W : 0;      // this wave's chunks per group
    const int total = ng * cw;

    // Each address is a wave-uniform base (scalar registers) plus a loop-invariant 32-bit lane
    // offset plus a per-block immediate, so no vector registers go to address arithmetic.
    // Lanes whose token does not exist (c16 >= M), and the k-groups that do not supply xs (the
    // scale MFMA takes it from k-group 0 only: S = xs * wd once), get an offset past the
    // descriptor's range: the load returns zero without touching memory, and no branch is needed.
    constexpr int LB = T::FB / 64;                                  // fragment bytes per lane
    constexpr uint32_t OOR = 0x40000000u;                           // beyond every range below
    const bool tl = c16 < a.M;
    const uint32_t o_w = (uint32_t)T::off(c16, g);                  // rows 0..15 of the half
    const uint32_t o_s = (uint32_t)c16 * 4;
    const uint32_t o_mw = (uint32_t)(g * 32 + c16) * 4;             // f32 MFMA k = g: block b0 + g
    const uint32_t o_mx = tl ? o_mw : OOR;
    const uint32_t o_x = tl ? (uint32_t)(((g >> 1) * 32 + c16) * 16 + (g & 1) * 8) : OOR;
    const uint32_t o_xs = (tl && g == 0) ? (uint32_t)c16 * 4 : OOR;
    const uint8_t* const xsb = reinterpret_cast<const uint8_t*>(a.xs2);
    const uint8_t* const xmb = reinterpret_cast<const uint8_t*>(a.xsx);
    const uint8_t* const wsb = a.w + a.w_scale_off;
    const uint8_t* const wmb = a.w + a.w_min_off;

    struct Chunk {
        typename T::Raw w[MV_CH];
        uint32_t ws[MV_CH];
        uint2 x[MV_CH];
        uint32_t xs[MV_CH];
        float xm, wm;
    };
    // item t (clamped to the last one, so that the tail issues harmless repeat loads)
    auto load = [&](int t, Chunk& k) __attribute__((always_inline)) {
        t = min(t, total - 1);
        const int i = t / cw, j = t - i * cw;
        const int q = (int)blockIdx.x + i * (int)gridDim.x;             // 16-row group
        const int half = q & 1;
        const int b0 = (wave + j * MV_W) * MV_CH;
        const int64_t tb = (int64_t)(q >> 1) * KBp + b0;                // (tile, block) index
        const rsrc_t rw = rsrc(a.w + tb * T::FB + half * (MV_ROWS * LB), MV_CH * T::FB);
        const rsrc_t rx = rsrc(a.xq + (int64_t)b0 * 1024, MV_CH * 1024);
#pragma unroll
        for (int u = 0; u < MV_CH; ++u) {
            k.w[u] = T::load(rw, o_w + u * T::FB);
            k.x[u] = ld64(rx, o_x + u * 1024);
        }
        if constexpr (!T::ROW) {
            const rsrc_t rs = rsrc(wsb + (tb * 32 + half * MV_ROWS) * 4, MV_CH * 128);
            const rsrc_t rxs = rsrc(xsb + (int64_t)b0 * 128, MV_CH * 128);
#pragma unroll
            for (int u = 0; u < MV_CH; ++u) {
                k.ws[u] = ld32(rs, o_s + u * 128);
                k.xs[u] = ld32(rxs, o_xs + u * 128);
            }
        }
        if constexpr (T::MIN) {
            k.xm = __builtin_bit_cast(float, ld32(rsrc(xmb + (int64_t)b0 * 128, 4 * 128), o_mx));
            k.wm = __builtin_bit_cast(float, ld32(rsrc(wmb + (tb * 32 + half * MV_ROWS) * 4, 4 * 128), o_mw));
        }
    };

    const v4i zi = {0, 0, 0, 0};
    const v4f zf = {0.f, 0.f, 0.f, 0.f};
    v4f acc = zf;
    v4i iacc = zi;
    auto compute = [&](const Chunk& k) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < MV_CH; ++u) {
            long bop[T::NMF];
            T::ops(k.w[u], T::ROW ? 0u : k.ws[u], g, tab, bop);
            const long aop = pk2(k.x[u].x, k.x[u].y);
            if constexpr (T::ROW) {
                iacc = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop[0], iacc, 0, 0, 0);
            } else {
                v4i D = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop[0], zi, 0, 0, 0);
                if constexpr (T::NMF == 2) D = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop[1], D, 0, 0, 0);
                const v4f S = __builtin_amdgcn_mfma_f32_16x16x16f16(as_h4(k.xs[u]), as_h4(T::scale_op(k.ws[u])),
                                                                    zf, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < NR; ++v) acc[v] = __builtin_fmaf((float)D[v], S[v], acc[v]);
            }
        }
        if constexpr (T::MIN) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.xm, k.wm, acc, 0, 0, 0);
    };

    // group i's reduction: the waves' partial sums meet in LDS buffer i&1 and are added in
    // wave order. One barrier per group suffices: buffer i&1 is written again only by group
    // i+2, after every thread has passed group i+1's barrier, i.e. finished group i's reads.
    auto finish = [&](int i) __attribute__((always_inline)) {
        const int p = i & 1;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            // element to a scalar first: a bit cast of the vector element expression itself
            // is lowered to element 0
            const int iv = iacc[v];
            red[p][wave][v][lane] = T::ROW ? __builtin_bit_cast(float, iv) : acc[v];
        }
        acc = zf;
        iacc = zi;
        lds_barrier();
        if (tid < 4 * 64) {
            const int l = tid & 63, v = tid >> 6;
            const int m = 4 * (l >> 4) + v;                      // token of register v in lane l
            const int col = ((int)blockIdx.x + i * (int)gridDim.x) * MV_ROWS + (l & 15);
            if (m < a.M && col < a.N) {
                if constexpr (T::ROW) {
                    int s = 0;
#pragma unroll
                    for (int w = 0; w < MV_W; ++w) s += __builtin_bit_cast(int, red[p][w][v][l]);
                    const float sw = reinterpret_cast<const float*>(wsb)[col];
                    reinterpret_cast<uint16_t*>(a.out)[(int64_t)m * a.ldo + col] = bf16_rne(((float)s * a.sa[m]) * sw);
                } else {
                    float s = 0.f;
#pragma unroll
                    for (int w = 0; w < MV_W; ++w) s += red[p][w][v][l];
                    reinterpret_cast<float*>(a.out)[(int64_t)m * a.ldo + col] = s * T::POST;
                }
            }
        }
    };

    if (cw == 0) {                       // fewer chunks than waves: this wave only reduces
        for (int i = 0; i < ng; ++i) finish(i);
        return;
    }
    // item t lives in buffer t % 3; step P computes buffer P and refills buffer (P+2) % 3
    Chunk k0, k1, k2;
    load(0, k0);
    load(1, k1);
    auto step = [&](int t, const Chunk& cur, Chunk& nxt) __attribute__((always_inline)) {
        load(t + 2, nxt);
        compute(cur);
        const int i = t / cw;
        if (t - i * cw == cw - 1) finish(i);
    };
    for (int t = 0;; t += 3) {
        step(t, k0, k2);
        if (t + 1 >= total) break;
        step(t + 1, k1, k0);
        if (t + 2 >= total) break;
        step(t + 2, k2, k1);
        if (t + 3 >= total) break;
    }
}

// persistent grid: one 1024-thread workgroup per compute unit
int cu_count() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cus[dev] = c;
    }
    return cus[dev];
}

template <mmq_wtype FMT>
hipError_t launch_fmt(const MvArgs& args, hipStream_t s) {
    const dim3 grid((unsigned)std::min(args.groups, cu_count())), block(MV_W * 64);
    switch (args.M) {
        case 1: hipLaunchKernelGGL((mmvq_kernel<FMT, 1>), grid, block, 0, s, args); break;
        case 2: hipLaunchKernelGGL((mmvq_kernel<FMT, 2>), grid, block, 0, s, args); break;
        case 3: hipLaunchKernelGGL((mmvq_kernel<FMT, 3>), grid, block, 0, s, args); break;
        default: hipLaunchKernelGGL((mmvq_kernel<FMT, 4>), grid, block, 0, s, args); break;
    }
    return hipGetLastError();
}

}  // namespace

int mmvq_max_tokens() { return MV_ROWS; }

hipError_t launch_mmvq(mmq_wtype t, const void* packed, const void* act, int64_t M, int64_t N,
                       int64_t K, void* out, int64_t ldo, hipStream_t s) {
    if (M < 1 || M > MV_ROWS) return hipErrorInvalidValue;
    const PackedLayout P = packed_layout(t, N, K);
    const uint8_t* ab = static_cast<const uint8_t*>(act);
    MvArgs args{};
    args.w = static_cast<const uint8_t*>(packed);
    args.w_scale_off = P.scale_off;
    args.w_min_off = P.min_off;
    args.M = (int)M;
    args.N = (int)N;
    args.KBp = (int)P.KBp;
    // groups past N (the second half of a last tile with N % 32 <= 16) hold only padding
    args.groups = (int)ceil_div(N, MV_ROWS);
    args.out = out;
    args.ldo = ldo;
    if (t == MMQ_I8_ROW) {
        const ActI8Layout L = act_i8_layout(M, K);
        args.xq = ab + L.a_off;
        args.sa = reinterpret_cast<const float*>(ab + L.sa_off);
    } else {
        const ActQ81Layout L = act_q8_1_layout(M, K);
        args.xq = ab + L.xq_off;
        args.xs2 = reinterpret_cast<const uint32_t*>(ab + L.xs2_off);
        args.xsx = reinterpret_cast<const float*>(ab + L.xsx_off);
    }
    switch (t) {
        case MMQ_Q8_0: return launch_fmt<MMQ_Q8_0>(args, s);
        case MMQ_Q4_0: return launch_fmt<MMQ_Q4_0>(args, s);
        case MMQ_Q4_K: return launch_fmt<MMQ_Q4_K>(args, s);
        case MMQ_IQ1T: return launch_fmt<MMQ_IQ1T>(args, s);
        case MMQ_I8_ROW: return launch_fmt<MMQ_I8_ROW>(args, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mmq
