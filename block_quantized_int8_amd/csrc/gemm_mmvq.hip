// gemm_mmvq.hip - the decode form of the MMQ contraction: batches of at most 16 token rows.
//
//   out[m,n] = sum_b (xs[m,b] * wd[n,b]) * P[m,n,b],   P = sum_{k in b} xq[m,k] * wq[n,k]
//
// The same contraction as the prefill kernels, on the same packed weights and q8_1 (or
// per-token int8) activations. A prefill tile sized for hundreds of tokens is mostly empty at
// a batch of a few tokens: a decode-shaped problem wastes all but one row of a 16-token
// matrix fragment (minfer "08 . R1", section 2.1), and llama.cpp keeps such batches (n <= 8)
// on a separate matrix-vector kernel, MMVQ ("CUDA: add IQ1_M to MMQ", PR #304, Summary). With
// so few tokens the work is one pass over the weights, and on gfx950 such a pass is bound by
// the number of vector-memory instructions per byte long before HBM is (a per-lane 4-byte
// load of scattered fragments moved ~80 useful bytes per instruction; plain streaming reads
// need ~250). The kernel is built around that:
//  * one v_mfma_i32_16x16x64_i8 covers a PAIR of blocks: its k-groups 0-1 carry block 2p and
//    k-groups 2-3 block 2p+1, so every lane loads one whole packed fragment lane (16 int8
//    values: 16 bytes of q8_0 / activations, 8 of q4_0 / q4_K, 4 of iq1t codes);
//  * the token side is block-diagonal: output rows 0-7 are tokens 0-7 against the first block
//    (their A operand is zero in k-groups 2-3), rows 8-15 the same tokens against the second
//    (zero in k-groups 0-1). So each block's integer dot stays exact and separate - no two
//    scales share an accumulator - and the zeros come from loads whose offset lies past the
//    buffer descriptor's range (the hardware returns 0 without a memory access), not from
//    extra instructions. Rows t and t+8 are added in the final reduction. Batches of 9-16
//    tokens run a second such operand for tokens 8-15;
//  * the scale product S = xs * wd comes from one f16 MFMA per pair (exact: a product of two
//    f16; q4_K's d*sc arrives as an exact f16 pair): the weight scales of four blocks are
//    loaded at once, block b0+g in k-group g, and the token scale of the pair's first block
//    feeds rows 0-7 through k-group 2p, the second's rows 8-15 through k-group 2p+1. Then
//    acc += f32(P) * S on the live registers. q4_K adds its rank-1 min term -(dmin*m) *
//    (xs*xsum) four blocks at a time with one f32 MFMA (minfer R1 section 2.2). W8A8 has no
//    per-block scale: its int32 accumulator runs through the whole of K and the epilogue
//    applies the two per-row scales (metainfer "INT8 W8A8 GEMM - Prefill", section 1);
//  * q6_K's scale changes every 16 values (minfer R1 sections 2.2 and 3.3: two half-block sums
//    per 32 values, each with its own d*sc). A lane's fragment bytes are one half of one block
//    (k-groups 0 and 2 hold halves 0, k-groups 1 and 3 halves 1), so each pair runs two int8
//    MFMAs over the weight operand with the other half's lanes zeroed, two scale MFMAs (the
//    half-0 and half-1 scale regions) and two FMAs into the same accumulator;
//  * persistent workgroups own 16-row weight groups; their 16 waves split the blocks of K
//    (chunks of 4 blocks dealt round-robin) and keep two chunks' loads in flight, across
//    group boundaries; the waves' partial sums meet in LDS and are added in a fixed order.
#include <algorithm>

#include "gemm_common.h"

namespace mmq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int MV_W = 16;          // waves per workgroup (they split the blocks of K)
constexpr int MV_CH = 4;          // blocks per chunk: two MFMA pairs, one scale load
constexpr int MV_ROWS = 16;       // weight rows per workgroup group
constexpr int MV_TOK = 16;        // largest batch
// Activation staging in LDS (token rows 0..8*TG-1 of every block, 16 bytes per (block, half,
// token)): capacity in blocks per token-group count, within the 160 KB LDS beside the
// reduction buffers. Longer K runs the register path (each wave loads its own operands).
template <int TG> struct XCap { static constexpr int KB = TG == 1 ? 448 : 128; };
static_assert(KB_ALIGN % MV_CH == 0, "chunks tile the padded block count");

// Buffer loads: a wave-uniform descriptor (base, byte range) in scalar registers plus a 32-bit
// lane offset; the hardware returns zero for an offset past the range, without a memory access.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_W3 = 0x00020000;        // descriptor word 3: raw 32-bit data format (gfx9)
constexpr uint32_t OOR = 0x40000000u;      // a lane offset past every range used here
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
__device__ inline v4i ld128(rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    const v4i o = {(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
    return o;
}

// an f16x4 operand with the dword `lo` in slots 0-1 and zeros in slots 2-3
__device__ inline h4 as_h4(uint32_t lo) {
    const v2i t = {(int)lo, 0};
    return __builtin_bit_cast(h4, t);
}

// Per weight format: the bytes of one packed fragment lane (row r, values 16h..16h+15 of a
// block), how they become the 16-byte int8 operand(s) in value order, and the power of two the
// integer dot carries (POST undoes it).
template <mmq_wtype FMT> struct VQ;

template <> struct VQ<MMQ_Q8_0> {
    static constexpr int FB = 1024, NMF = 1;
    static constexpr bool MIN = false, ROW = false, META = false, DUAL = false, GRID = false;
    static constexpr float POST = 1.0f;
    typedef v4i Raw;
    __device__ static Raw load(rsrc_t r, uint32_t off) { return ld128(r, off); }
    __device__ static void ops(Raw r, uint32_t, const uint2*, const uint32_t*, v4i* b) { b[0] = r; }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }
};

// per-channel int8: the q8_0 fragment layout, one f32 scale per row instead of per block
template <> struct VQ<MMQ_I8_ROW> : VQ<MMQ_Q8_0> {
    static constexpr bool ROW = true;
};

// q6_K: int8 q - 32 in the q8_0 fragment layout; scale dwords per 16-value half (half 0 in the
// scale region, half 1 in the second region), each the exact f16 pair (hi, lo) of d*sc_h
template <> struct VQ<MMQ_Q6_K> : VQ<MMQ_Q8_0> {
    static constexpr bool DUAL = true;
};

// q4_0: X0 holds values 0-3 in its high nibbles and 4-7 in its low ones (X1: 8-15), each the
// 4-bit two's complement of nib - 8, so the masked bytes are int8 16*(nib-8).
template <> struct VQ<MMQ_Q4_0> {
    static constexpr int FB = 512, NMF = 1;
    static constexpr bool MIN = false, ROW = false, META = false, DUAL = false, GRID = false;
    static constexpr float POST = 1.0f / 16;
    typedef uint2 Raw;
    __device__ static Raw load(rsrc_t r, uint32_t off) { return ld64(r, off); }
    __device__ static void ops(Raw r, uint32_t, const uint2*, const uint32_t*, v4i* b) {
        b[0][0] = (int)(r.x & 0xF0F0F0F0u);
        b[0][1] = (int)((r.x << 4) & 0xF0F0F0F0u);
        b[0][2] = (int)(r.y & 0xF0F0F0F0u);
        b[0][3] = (int)((r.y << 4) & 0xF0F0F0F0u);
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }
};

// q4_K: unsigned nibbles, values 0-3 in the low nibbles of X0 and 4-7 in its high ones; the
// scale dword is the exact f16 pair (hi, lo) of d*sc, the min region -dmin*m.
template <> struct VQ<MMQ_Q4_K> {
    static constexpr int FB = 512, NMF = 1;
    static constexpr bool MIN = true, ROW = false, META = false, DUAL = false, GRID = false;
    static constexpr float POST = 1.0f;
    typedef uint2 Raw;
    __device__ static Raw load(rsrc_t r, uint32_t off) { return ld64(r, off); }
    __device__ static void ops(Raw r, uint32_t, const uint2*, const uint32_t*, v4i* b) {
        b[0][0] = (int)(r.x & 0x0F0F0F0Fu);
        b[0][1] = (int)((r.x >> 4) & 0x0F0F0F0Fu);
        b[0][2] = (int)(r.y & 0x0F0F0F0Fu);
        b[0][3] = (int)((r.y >> 4) & 0x0F0F0F0Fu);
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }
};

// iq1t: one dword of 2-bit codes per fragment lane (value 4q + b at bits 8b + 2q). The lane's
// half h has the meta byte s | sigma0 << 3 | sigma1 << 4 in its row's scale dword (byte
// 2 + h); values 0-7 are sign group 0, 8-15 group 1. The IQ1_M fold (llama.cpp PR #304,
// Design) makes each value the integer v = 8(c-1) + sigma (sigma = +-1) under the per-16
// factor (2s+1) and the scale d/8; (2s+1)*v is split as 2s*v + v (|2s*v| <= 126) over two
// chained int8 MFMAs. tab[s | sign << 3] = (byte LUT code -> v, byte LUT code -> 2s*v).
template <> struct VQ<MMQ_IQ1T> {
    static constexpr int FB = 256, NMF = 2;
    static constexpr bool MIN = false, ROW = false, META = true, DUAL = false, GRID = false;
    static constexpr float POST = 1.0f / 8;
    typedef uint32_t Raw;
    __device__ static Raw load(rsrc_t r, uint32_t off) { return ld32(r, off); }
    // meta: the lane's meta byte
    __device__ static void ops(Raw C, uint32_t meta, const uint2* tab, const uint32_t*, v4i* b) {
        const uint32_t s = meta & 7u;
        const uint2 t0 = tab[s | (((meta >> 3) & 1u) << 3)];
        const uint2 t1 = tab[s | (((meta >> 4) & 1u) << 3)];
        const uint32_t q0 = C & 0x03030303u, q1 = (C >> 2) & 0x03030303u;
        const uint32_t q2 = ((C >> 4) & 0x03030303u) | 0x04040404u;
        const uint32_t q3 = ((C >> 6) & 0x03030303u) | 0x04040404u;
        // selectors 0-2 pick group 0's LUT (low word), 4-6 group 1's (high word)
        b[0][0] = (int)__builtin_amdgcn_perm(t1.y, t0.y, q0);
        b[0][1] = (int)__builtin_amdgcn_perm(t1.y, t0.y, q1);
        b[0][2] = (int)__builtin_amdgcn_perm(t1.y, t0.y, q2);
        b[0][3] = (int)__builtin_amdgcn_perm(t1.y, t0.y, q3);
        b[1][0] = (int)__builtin_amdgcn_perm(t1.x, t0.x, q0);
        b[1][1] = (int)__builtin_amdgcn_perm(t1.x, t0.x, q1);
        b[1][2] = (int)__builtin_amdgcn_perm(t1.x, t0.x, q2);
        b[1][3] = (int)__builtin_amdgcn_perm(t1.x, t0.x, q3);
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

// iq1c / iq1s grid-index panels: one dword W = ia << 2 | meta << 13 | ib << 20 per fragment lane;
// the two 11-bit indices name grid entries (kept in LDS, spread into the iq1t code order), so the
// lane's code dword is entry(ia) | entry(ib) << 4 and meta sits in W itself; then the iq1t fold.
// The scale d comes per (row, 4-block group) from its own region (16 bits per row).
template <> struct VQ<MMQ_IQ1C> : VQ<MMQ_IQ1T> {
    static constexpr bool META = false, GRID = true;
    __device__ static void ops(Raw W, uint32_t, const uint2* tab, const uint32_t* gtab, v4i* b) {
        const uint32_t C = gtab[(W >> 2) & 0x7FFu] | (gtab[W >> 20] << 4);
        VQ<MMQ_IQ1T>::ops(C, (W >> 13) & 0x1Fu, tab, gtab, b);
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }             // f16 d
};

struct MvArgs {
    const uint8_t* w;           // packed weights
    int64_t w_scale_off;        // scale region (per-row f32 sw for W8A8)
    int64_t w_min_off;          // q4_K min region; q6_K half-1 scale region
    const uint8_t* xq;          // act region 0: tiled int8 values (token tile 0)
    const uint32_t* xs2;        // q8_1 region 3: xs as an f16 pair, tile-major
    const float* xsx;           // q8_1 region 4: xs * xsum, tile-major
    const float* sa;            // i8_token region 1: per-token scale
    int M, N, KBp, groups;      // groups: 16-row groups holding at least one real row
    int nb;                     // dense: token batches of MV_TOK (units = nb x groups)
    void* out;
    int64_t ldo;
    // MUL_MAT_ID with at most 8 tokens: the routing ids themselves (each workgroup groups the
    // at most 256 pairs by expert on its own, so no routing launch precedes this one)
    int64_t w_stride;           // bytes between experts' packed matrices
    const int32_t* ids;         // [P] expert of pair p = token * top_k + slot
    int E, top_k, P;
};

constexpr int MV_IDP = 256;     // MUL_MAT_ID decode: pairs (and so pair batches) at most
// MUL_MAT_ID decode: tokens at most. A workgroup stages the token rows (8, or 16 past 8 tokens)
// and its batches of up to 8 pairs read them by token id. Measured on 64 experts of 2048 x 4096,
// top-8, against the prefill gather: IQ1T 13.7 / 32.5 / 40.6 / 50.0 us at 1 / 4 / 6 / 8 tokens
// against 36 / 47 / 45.4 / 55.9; at 6 tokens Q4_K 38.9 against 50.4, IQ1C 42.9 against 43.3;
// q4_0 at 8 tokens 44.0 against 48.1. With 16 rows staged: IQ1T 52.5 / 53.9 / 54.4 / 59.4 us at
// 9 / 10 / 11 / 12 tokens against 57.8 / 56.9 / 57.3 / 58.0, IQ1C 55.3 / 57.1 / 62.6 at 9 / 10 /
// 12 against 57.9 / 57.7 / 58.1, q4_0 46.2 / 47.3 at 9 / 10 against 48.9 / 49.3, Q4_K 54.8 at
// 10 against 65.2.
constexpr int MV_ID_TOK = 10;

// LDS barrier that leaves global loads in flight (__syncthreads() would also wait for them)
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Persistent workgroups: workgroup b handles the 16-row groups b, b + gridDim.x, ... (group q
// = rows 16q..16q+15 = half q&1 of weight tile q/2), all M <= 16 tokens, all of K. Each wave's
// work is one stream of items (group, chunk), its chunks being wave, wave + MV_W, ... of every
// group; loads run two items ahead. TG = token groups of 8 (1 or 2); NR = accumulator
// registers holding a live token (min(M, 4)). BT: dense token batches of MV_TOK rows (more
// than MV_TOK tokens), a unit being (batch, group); a separate instance, so that one batch pays
// no per-item batch arithmetic.
template <mmq_wtype FMT, int TG, int NR, bool XL, bool ID, bool BT = false, bool W16 = false>
__global__ __launch_bounds__(MV_W * 64) void mmvq_kernel(MvArgs a) {
    static_assert(!ID || XL, "MUL_MAT_ID reads its gathered tokens from the staged rows");
    static_assert(!BT || (!ID && !XL && TG == 2), "token batches: dense, per-item token loads");
    using T = VQ<FMT>;
    static_assert(!W16 || (ID && TG == 1), "16 staged rows: MUL_MAT_ID batches of 8 pairs");
    constexpr int TOK = 8 * TG;                              // token rows (pairs) per item
    constexpr int SR = W16 ? 16 : TOK;                       // staged token rows
    constexpr int XSLOTS = XL ? XCap<SR / 8>::KB * 2 * SR : 0;  // 16-byte slots; slot XSLOTS is zero
    __shared__ float red[2][MV_W][4 * TG][64];
    __shared__ uint2 tab[16];
    __shared__ uint32_t gtab[T::GRID ? 2048 : 1];
    __shared__ __attribute__((aligned(16))) uint8_t xl[(XSLOTS + 1) * 16];
    // MUL_MAT_ID: per batch of at most TOK pairs of one expert (expert id, first pair in
    // expert order, pairs), the pair ids, and the scan's wave totals
    __shared__ int s_e[ID ? MV_IDP : 1], s_po[ID ? MV_IDP : 1], s_me[ID ? MV_IDP : 1];
    __shared__ int s_pp[ID ? MV_IDP : 1];
    __shared__ int s_tk[ID ? MV_IDP : 1];                            // s_pp's pair's token
    __shared__ int s_wt[MV_W + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;

    // the grid (the packed matrix's last region; MUL_MAT_ID: expert 0's); on the LDS path its
    // loads go out with the token staging loads and share their barrier (stage() below)
    const uint32_t* const gsrc = reinterpret_cast<const uint32_t*>(a.w + a.w_min_off);
    if constexpr (FMT == MMQ_IQ1T || FMT == MMQ_IQ1C) {
        if (tid < 16) tab[tid] = T::table(tid);
        if constexpr (!(XL && T::GRID)) {
            if constexpr (T::GRID)
                for (int i = tid; i < 2048; i += MV_W * 64) gtab[i] = gsrc[i];
            __syncthreads();
        }
    }
    const int KBp = a.KBp;
    const int nch = KBp / MV_CH;
    // Group of round i: off + G*i. Workgroups are dealt to the 8 XCDs round-robin (b -> b % 8),
    // and the two 16-row halves of a weight tile share their 128-byte scale lines, so with a
    // grid of whole 16s the halves of a tile go to workgroups b and b + 8 - the same XCD, whose
    // L2 then fetches each scale line once.
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const int off = (G % 16 == 0) ? 2 * (8 * (b >> 4) + (b & 7)) + ((b >> 3) & 1) : b;
    // work units: 16-row groups, or (pair batch, group) for MUL_MAT_ID, where a batch is up to
    // TOK pairs of one expert (one batch per used expert when a token's experts are distinct;
    // more for an expert named by several slots of a token)
    int units = BT ? a.groups * a.nb : a.groups;
    if constexpr (ID) {
        // Group the P <= 256 pairs by expert: key = expert << 8 | pair (ids outside [0, E) sort
        // last as expert E), rank each key by counting the smaller ones, so s_pp lists the pairs
        // in expert order; then a batch starts at every TOK-th position of an expert's run.
        const int P = a.P;
        int key = 0, e = a.E;
        if (tid < P) {
            const int id = a.ids[tid];
            e = (id >= 0 && id < a.E) ? id : a.E;
            key = (e << 8) | tid;
            s_e[tid] = key;                                          // keys, for the ranking
        }
        __syncthreads();
        int rank = 0, first = 0;                                     // first: the run's start
        if (tid < P) {
            for (int j = 0; j < P; ++j) {
                const int kj = s_e[j];
                rank += kj < key;
                first += (kj >> 8) < e;
            }
        }
        __syncthreads();
        const bool start = tid < P && e < a.E && (rank - first) % TOK == 0;
        if (tid < P) {
            s_pp[rank] = tid;                                        // pairs in expert order
            s_tk[rank] = tid / a.top_k;
            s_po[rank] = start ? 1 : 0;                              // batch-start flags
            s_me[rank] = e;
        }
        __syncthreads();
        // batch u: the u-th start flag in expert order (an exclusive scan over <= 256 flags)
        int st = 0, cnt = 0, ex = 0, len = 0;
        if (tid < P) {
            st = s_po[tid];
            ex = s_me[tid];
            for (int j = 0; j < tid; ++j) cnt += s_po[j];
            if (st) {
                int l = 1;
                while (l < TOK && tid + l < P && s_me[tid + l] == ex) ++l;
                len = l;
            }
        }
        if (tid == 0) {
            int nb = 0;
            for (int j = 0; j < P; ++j) nb += s_po[j];
            s_wt[MV_W] = nb;                                         // batches in all
        }
        __syncthreads();
        if (st) {
            s_e[cnt] = ex;
            s_po[cnt] = tid;                                         // first pair in expert order
            s_me[cnt] = len;
        }
        __syncthreads();
        units = __builtin_amdgcn_readfirstlane(s_wt[MV_W]) * a.groups;
    }
    const int ng = (units - off + G - 1) / G;                            // >= 1 for dense grids
    if (ng <= 0) return;                                                 // uniform: nothing to do
    const int cw = wave < nch ? (nch - wave + MV_W - 1) / MV_W : 0;      // this wave's chunks per group
    const int total = ng * cw;

    // ---- loop-invariant lane offsets (bytes); per-item bases are wave-uniform
    constexpr int LB = T::FB / 64;                   // packed bytes per fragment lane
    const int fb = g >> 1, fh = g & 1;               // block of the pair, half of the block
    // weight operand: fragment lane fh*32 + (row of the 16-row group) of block 2p + fb
    const uint32_t o_w = (uint32_t)(fb * T::FB + (fh * 32 + c16) * LB);
    // token operand, block-diagonal: row c16 < 8 takes token c16 against block 2p (k-groups
    // 0-1), row c16 >= 8 token c16-8 against block 2p+1 (k-groups 2-3); other lanes read zero
    const bool diag = (c16 >> 3) == fb;
    const int t0 = c16 & 7, t1 = 8 + (c16 & 7);
    const uint32_t o_x0 = (diag && t0 < a.M) ? (uint32_t)(fb * 1024 + (fh * 32 + t0) * 16) : OOR;
    const uint32_t o_x1 = (diag && t1 < a.M) ? (uint32_t)(fb * 1024 + (fh * 32 + t1) * 16) : OOR;
    // scales of four blocks at once: k-group g holds block b0 + g (weight row c16; the token
    // scales of the token of row c16, and q4_K's min term for rows 0-7, per unit in load())
    const uint32_t o_s = (uint32_t)(g * 128 + c16 * 4);
    // iq1t: the scale dword of this lane's own (block 2p + fb, row c16), for its meta byte
    const uint32_t o_wso = (uint32_t)(fb * 128 + c16 * 4);
    const uint8_t* const xsb = reinterpret_cast<const uint8_t*>(a.xs2);
    const uint8_t* const xmb = reinterpret_cast<const uint8_t*>(a.xsx);
    const uint8_t* const wsb = a.w + a.w_scale_off;

    struct Chunk {
        typename T::Raw w[2];
        v4i x[TG][2];                // register path only
        int b0, tk[TG];
        uint32_t ws, ws2, xs[TG];
        uint32_t wso[2];
        float xm[TG], wm;
    };
    // item t (clamped to the last one, so that the tail issues harmless repeat loads)
    auto load = [&](int t, Chunk& k) __attribute__((always_inline)) {
        t = min(t, total - 1);
        const int i = t / cw, j = t - i * cw;
        int q = off + i * G;                                            // 16-row group
        const uint8_t* wx = a.w;                                        // this unit's weights
        int me = a.M, po = 0;                                           // its tokens
        int ro = 0;                                                     // its first token row
        if constexpr (BT) {             // dense: token batch bt holds rows 16 bt .. 16 bt + 15
            const int bt = q / a.groups;
            q -= bt * a.groups;
            ro = bt * MV_TOK;
            me = min(a.M - ro, MV_TOK);
        }
        if constexpr (ID) {
            const int ue = q / a.groups;
            q -= ue * a.groups;
            wx += (int64_t)__builtin_amdgcn_readfirstlane(s_e[ue]) * a.w_stride;
            me = __builtin_amdgcn_readfirstlane(s_me[ue]);
            po = __builtin_amdgcn_readfirstlane(s_po[ue]);
        }
        // the token of this lane's rows (t0 / t1 of the unit), -1 past its token count; the
        // batch values are wave-uniform and the token read takes no branch (a branch here made the
        // compiler treat the item loop as divergent and wait on the in-flight loads at its head)
#pragma unroll
        for (int x = 0; x < TG; ++x) {
            const int ix = (c16 & 7) + 8 * x;
            int tk = ix < me ? ix : -1;
            if constexpr (ID) {
                const int tv = s_tk[min(po + ix, MV_IDP - 1)];
                tk = ix < me ? tv : -1;
            }
            k.tk[x] = tk;
        }
        const int half = q & 1;
        const int b0 = (wave + j * MV_W) * MV_CH;
        const int64_t tb = (int64_t)(q >> 1) * KBp + b0;                // (tile, block) index
        const rsrc_t rw = rsrc(wx + tb * T::FB + half * (MV_ROWS * LB), MV_CH * T::FB);
        // the batch's token tile and its row offset in it (0 or 16)
        const int64_t tt = ro >> 5;
        const int rr = ro & 31;
        const rsrc_t rx = rsrc(a.xq + (tt * KBp + b0) * 1024, MV_CH * 1024);
        k.b0 = b0;
        uint32_t ox0 = o_x0, ox1 = o_x1;
        if constexpr (BT) {
            ox0 = (diag && t0 < me) ? (uint32_t)(fb * 1024 + (fh * 32 + rr + t0) * 16) : OOR;
            ox1 = (diag && t1 < me) ? (uint32_t)(fb * 1024 + (fh * 32 + rr + t1) * 16) : OOR;
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            k.w[p] = T::load(rw, o_w + p * 2 * T::FB);
            if constexpr (!XL) {
                k.x[0][p] = ld128(rx, ox0 + p * 2048);
                if constexpr (TG == 2) k.x[1][p] = ld128(rx, ox1 + p * 2048);
            }
        }
        if constexpr (!T::ROW) {
            const rsrc_t rs = rsrc(wx + a.w_scale_off + (tb * 32 + half * MV_ROWS) * 4, MV_CH * 128);
            const rsrc_t rxs = rsrc(xsb + (tt * KBp + b0) * 128, MV_CH * 128);
            if constexpr (T::GRID) {       // the row's d of this 4-block group (MV_CH = 4 blocks)
                const int64_t gq = (int64_t)(q >> 1) * (KBp / 4) + b0 / 4;
                k.ws = __builtin_amdgcn_raw_buffer_load_b16(
                    rsrc(wx + a.w_scale_off + (gq * 32 + half * MV_ROWS) * 2, MV_ROWS * 2), (int)(c16 * 2), 0, 0);
            } else {
                k.ws = ld32(rs, o_s);
            }
            if constexpr (T::DUAL)
                k.ws2 = ld32(rsrc(wx + a.w_min_off + (tb * 32 + half * MV_ROWS) * 4, MV_CH * 128), o_s);
#pragma unroll
            for (int x = 0; x < TG; ++x)       // token of row c16, block b0 + g
                k.xs[x] = ld32(rxs, k.tk[x] >= 0 ? (uint32_t)(g * 128 + (rr + k.tk[x]) * 4) : OOR);
            if constexpr (T::META) {
                k.wso[0] = ld32(rs, o_wso);
                k.wso[1] = ld32(rs, o_wso + 256);
            }
        }
        if constexpr (T::MIN) {
            const rsrc_t rxm = rsrc(xmb + (tt * KBp + b0) * 128, MV_CH * 128);
#pragma unroll
            for (int x = 0; x < TG; ++x)       // rows 0-7 only: token of row c16 = k.tk[x]
                k.xm[x] = __builtin_bit_cast(float, ld32(rxm, (c16 < 8 && k.tk[x] >= 0) ? (uint32_t)(g * 128 + (rr + k.tk[x]) * 4) : OOR));
            k.wm = __builtin_bit_cast(float, ld32(rsrc(wx + a.w_min_off + (tb * 32 + half * MV_ROWS) * 4, MV_CH * 128), o_s));
        }
    };

    const v4i zi = {0, 0, 0, 0};
    const v4f zf = {0.f, 0.f, 0.f, 0.f};
    v4f acc[TG];
    v4i iacc[TG];
#pragma unroll
    for (int x = 0; x < TG; ++x) {
        acc[x] = zf;
        iacc[x] = zi;
    }
    // k-group of the token scale feeding this lane's row in pair p: 2p for rows 0-7, 2p+1 for 8-15
    const bool sel0 = g == (c16 >> 3), sel1 = g == 2 + (c16 >> 3);
    auto compute = [&](const Chunk& k) __attribute__((always_inline)) {
        // token operands of both pairs (LDS path: the diagonal lanes' slots, else the zero slot)
        v4i xo[TG][2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int x = 0; x < TG; ++x) {
                if constexpr (XL) {
                    const int sl = (diag && k.tk[x] >= 0) ? ((k.b0 + 2 * p + fb) * 2 + fh) * SR + k.tk[x] : XSLOTS;
                    xo[x][p] = *reinterpret_cast<const v4i*>(xl + sl * 16);
                } else {
                    xo[x][p] = k.x[x][p];
                }
            }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            v4i bop[T::NMF];
            uint32_t meta = 0;
            if constexpr (T::META) meta = (k.wso[p] >> (16 + 8 * fh)) & 0xFFu;
            T::ops(k.w[p], meta, tab, gtab, bop);
#pragma unroll
            for (int x = 0; x < TG; ++x) {
                if constexpr (T::ROW) {
                    iacc[x] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xo[x][p], bop[0], iacc[x], 0, 0, 0);
                } else if constexpr (T::DUAL) {
                    // half h's dot: the weight lanes of the other half read as zero
                    const v4i w0 = fh == 0 ? bop[0] : zi, w1 = fh == 0 ? zi : bop[0];
                    const v4i D0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xo[x][p], w0, zi, 0, 0, 0);
                    const v4i D1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xo[x][p], w1, zi, 0, 0, 0);
                    const uint32_t xa = (p == 0 ? sel0 : sel1) ? k.xs[x] : 0u;
                    const v4f S0 = __builtin_amdgcn_mfma_f32_16x16x16f16(as_h4(xa), as_h4(k.ws), zf, 0, 0, 0);
                    const v4f S1 = __builtin_amdgcn_mfma_f32_16x16x16f16(as_h4(xa), as_h4(k.ws2), zf, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < NR; ++v) {
                        acc[x][v] = __builtin_fmaf((float)D0[v], S0[v], acc[x][v]);
                        acc[x][v] = __builtin_fmaf((float)D1[v], S1[v], acc[x][v]);
                    }
                } else {
                    v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(xo[x][p], bop[0], zi, 0, 0, 0);
                    if constexpr (T::NMF == 2) D = __builtin_amdgcn_mfma_i32_16x16x64_i8(xo[x][p], bop[1], D, 0, 0, 0);
                    const uint32_t xa = (p == 0 ? sel0 : sel1) ? k.xs[x] : 0u;
                    const v4f S = __builtin_amdgcn_mfma_f32_16x16x16f16(as_h4(xa), as_h4(T::scale_op(k.ws)), zf, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < NR; ++v) acc[x][v] = __builtin_fmaf((float)D[v], S[v], acc[x][v]);
                }
            }
        }
        if constexpr (T::MIN) {
#pragma unroll
            for (int x = 0; x < TG; ++x) acc[x] = __builtin_amdgcn_mfma_f32_16x16x4f32(k.xm[x], k.wm, acc[x], 0, 0, 0);
        }
    };

    // group i's reduction: the waves' partial sums meet in LDS buffer i&1 and are added in a
    // fixed order. One barrier per group suffices: buffer i&1 is written again only by group
    // i+2, after every thread has passed group i+1's barrier, i.e. finished group i's reads.
    auto finish = [&](int i) __attribute__((always_inline)) {
        const int pb = i & 1;
#pragma unroll
        for (int x = 0; x < TG; ++x) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                // element to a scalar first: a bit cast of the vector element expression itself
                // is lowered to element 0
                const int iv = iacc[x][v];
                red[pb][wave][4 * x + v][lane] = T::ROW ? __builtin_bit_cast(float, iv) : acc[x][v];
            }
            acc[x] = zf;
            iacc[x] = zi;
        }
        lds_barrier();
        if (tid < MV_TOK * MV_ROWS) {
            // token m, column n: register (m & 3) of lanes 16*((m & 7) >> 2) + n (rows 0-7,
            // even blocks) and that + 32 (rows 8-15, odd blocks), token group m >> 3
            const int m = tid >> 4, n = tid & 15;
            int q = off + i * G, me = a.M, row = m;
            if constexpr (BT) {
                const int bt = q / a.groups;
                q -= bt * a.groups;
                me = min(a.M - bt * MV_TOK, MV_TOK);
                row = bt * MV_TOK + m;
            }
            if constexpr (ID) {
                const int ue = q / a.groups;
                q -= ue * a.groups;
                me = s_me[ue];
                row = m < me ? s_pp[s_po[ue] + m] : 0;     // the pair's own output row
            }
            const int col = q * MV_ROWS + n;
            if (m < me && col < a.N) {
                const int r = 4 * (m >> 3) + (m & 3);
                const int la = 16 * ((m & 7) >> 2) + n, lb = la + 32;
                if constexpr (T::ROW) {
                    int s = 0;
#pragma unroll
                    for (int w = 0; w < MV_W; ++w)
                        s += __builtin_bit_cast(int, red[pb][w][r][la]) + __builtin_bit_cast(int, red[pb][w][r][lb]);
                    const float sw = reinterpret_cast<const float*>(wsb)[col];
                    reinterpret_cast<uint16_t*>(a.out)[(int64_t)row * a.ldo + col] = bf16_rne(((float)s * a.sa[row]) * sw);
                } else {
                    float s = 0.f;
#pragma unroll
                    for (int w = 0; w < MV_W; ++w) s += red[pb][w][r][la] + red[pb][w][r][lb];
                    reinterpret_cast<float*>(a.out)[(int64_t)row * a.ldo + col] = s * T::POST;
                }
            }
        }
    };

    // LDS path: the token rows 0..SR-1 of every block go to slot (b*2 + h)*SR + t (the tiled
    // xq keeps row t's values 16h..16h+15 of block b at lane h*32 + t; rows >= M are the
    // buffer's zero padding). The staging loads (and iq1c's grid) are issued first, then the
    // first two items' weight loads, then the LDS writes (which wait only for the staging
    // loads) and a barrier that leaves the weight loads in flight.
    constexpr int PER = XL ? (XSLOTS + MV_W * 64 - 1) / (MV_W * 64) : 1;
    constexpr int GPER = (XL && T::GRID) ? 2048 / (MV_W * 64) : 1;
    v4i xv[PER];
    uint32_t gv[GPER];
    if constexpr (XL && T::GRID) {
#pragma unroll
        for (int u = 0; u < GPER; ++u) gv[u] = gsrc[tid + u * MV_W * 64];
    }
    if constexpr (XL) {
        const int nslot = KBp * 2 * SR;
        const rsrc_t rq = rsrc(a.xq, (uint32_t)KBp * 1024);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            // every thread issues PER loads (sized for the longest K); slots past this K's end
            // take an offset outside the descriptor, which returns zero without a memory request
            const int sl = tid + u * MV_W * 64;
            const int t = sl % SR, h = (sl / SR) & 1, b = sl / (2 * SR);
            xv[u] = ld128(rq, sl < nslot ? (uint32_t)((b * 64 + h * 32 + t) * 16) : OOR);
        }
    }
    auto stage = [&]() __attribute__((always_inline)) {
        if constexpr (XL) {
            const int nslot = KBp * 2 * SR;
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int sl = tid + u * MV_W * 64;
                if (sl < nslot) *reinterpret_cast<v4i*>(xl + sl * 16) = xv[u];
            }
            if (tid == 0) {
                const v4i z = {0, 0, 0, 0};
                *reinterpret_cast<v4i*>(xl + XSLOTS * 16) = z;
            }
            if constexpr (T::GRID) {
#pragma unroll
                for (int u = 0; u < GPER; ++u) gtab[tid + u * MV_W * 64] = gv[u];
            }
            lds_barrier();
        }
    };

    if (cw == 0) {                       // fewer chunks than waves: this wave only reduces
        stage();
        for (int i = 0; i < ng; ++i) finish(i);
        return;
    }
    // item t lives in buffer t % 3; each step computes one buffer and refills the one
    // computed in the step before
    Chunk k0, k1, k2;
    load(0, k0);
    load(1, k1);
    stage();
    // the wave's priority is raised while it issues the next item's loads, so that they leave
    // before the other waves' compute (Q4_K 14336 x 4096 -1.8%, the 4-token MoE -3.5%)
    auto step = [&](int t, const Chunk& cur, Chunk& nxt) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        load(t + 2, nxt);
        __builtin_amdgcn_s_setprio(0);
        compute(cur);
        const int i = t / cw;
        if (t - i * cw == cw - 1) finish(i);
    };
    // whole triples in a loop without exits, then the last 0-2 items: with exits inside the loop
    // the compiler's wait-count pass assumed the loads just issued could still be in flight at
    // the loop head and waited for them there (the 1-token MoE -13%, Q4_K 14336 x 4096 -7%)
    int t = 0;
    for (; t + 3 <= total; t += 3) {
        step(t, k0, k2);
        step(t + 1, k1, k0);
        step(t + 2, k2, k1);
    }
    if (t < total) {
        step(t, k0, k2);
        if (t + 1 < total) step(t + 1, k1, k0);
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

template <mmq_wtype FMT, bool XL, bool ID = false>
void launch_xl(const MvArgs& args, dim3 grid, hipStream_t s) {
    const dim3 block(MV_W * 64);
    if constexpr (ID) {
        // batches of up to 8 pairs whatever the token count: every register is live; more than
        // 8 tokens stage 16 rows
        if (args.M > 8) hipLaunchKernelGGL((mmvq_kernel<FMT, 1, 4, XL, ID, false, true>), grid, block, 0, s, args);
        else hipLaunchKernelGGL((mmvq_kernel<FMT, 1, 4, XL, ID>), grid, block, 0, s, args);
        return;
    }
    switch (args.M) {
        case 1: hipLaunchKernelGGL((mmvq_kernel<FMT, 1, 1, XL, ID>), grid, block, 0, s, args); break;
        case 2: hipLaunchKernelGGL((mmvq_kernel<FMT, 1, 2, XL, ID>), grid, block, 0, s, args); break;
        case 3: hipLaunchKernelGGL((mmvq_kernel<FMT, 1, 3, XL, ID>), grid, block, 0, s, args); break;
        case 4: case 5: case 6: case 7: case 8:
            hipLaunchKernelGGL((mmvq_kernel<FMT, 1, 4, XL, ID>), grid, block, 0, s, args); break;
        default: hipLaunchKernelGGL((mmvq_kernel<FMT, 2, 4, XL, ID>), grid, block, 0, s, args); break;
    }
}

template <mmq_wtype FMT>
hipError_t launch_fmt(const MvArgs& args, hipStream_t s) {
    const dim3 grid((unsigned)std::min(args.groups * args.nb, cu_count()));
    // Token rows staged in LDS only when workgroups loop over several groups: the staging and
    // its barrier are a fixed cost per workgroup that one group does not pay back (q4_0 4096 x
    // 4096, 8 tokens: 4.51 -> 3.71 us without; Q4_K 14336 x 4096, 1 token, 3.5 groups per
    // workgroup: 9.82 -> 10.16 us without)
    const int cap = args.M <= 8 ? XCap<1>::KB : XCap<2>::KB;
    if (args.nb > 1)
        hipLaunchKernelGGL((mmvq_kernel<FMT, 2, 4, false, false, true>), grid, dim3(MV_W * 64), 0, s, args);
    else if (args.KBp <= cap && args.groups > cu_count()) launch_xl<FMT, true>(args, grid, s);
    else launch_xl<FMT, false>(args, grid, s);
    return hipGetLastError();
}

}  // namespace

int mmvq_max_tokens() { return MV_TOK; }

// more than 16 tokens: batches of 16 as extra units while they take at most MV_MAX_ROUNDS rounds
// of the grid (a prefill grid of that size leaves most CUs idle: q4_0 4096 x 4096 takes ~23 us
// at 17 to 128 tokens there)
constexpr int MV_MAX_ROUNDS = 8;
constexpr int MV_MAX_BATCHES = 8;
bool mmvq_dense_ok(int64_t M, int64_t N) {
    if (M < 1) return false;
    if (M <= MV_TOK) return true;
    const int64_t nb = ceil_div(M, MV_TOK);
    return nb <= MV_MAX_BATCHES && nb * ceil_div(N, MV_ROWS) <= (int64_t)MV_MAX_ROUNDS * cu_count();
}

bool mmvq_id_ok(mmq_wtype t, int64_t T, int64_t top_k, int64_t K) {
    if (t == MMQ_I8_ROW || T < 1 || T > MV_ID_TOK || T * top_k > MV_IDP) return false;
    return round_up(K / QK, KB_ALIGN) <= (T > 8 ? XCap<2>::KB : XCap<1>::KB);   // staged rows
}

hipError_t launch_mmvq_id(mmq_wtype t, const void* packed, int64_t E, const void* act, int64_t T,
                          int64_t top_k, int64_t N, int64_t K, const int32_t* ids, void* out,
                          hipStream_t s) {
    if (!mmvq_id_ok(t, T, top_k, K)) return hipErrorInvalidValue;
    const PackedLayout P = packed_layout(t, N, K);
    const ActQ81Layout L = act_q8_1_layout(T, K);
    const uint8_t* ab = static_cast<const uint8_t*>(act);
    MvArgs args{};
    args.w = static_cast<const uint8_t*>(packed);
    args.w_scale_off = P.scale_off;
    args.w_min_off = P.min_off;
    args.w_stride = P.bytes;
    args.M = (int)T;
    args.N = (int)N;
    args.KBp = (int)P.KBp;
    args.groups = (int)ceil_div(N, MV_ROWS);
    args.nb = 1;
    args.out = out;
    args.ldo = N;
    args.xq = ab + L.xq_off;
    args.xs2 = reinterpret_cast<const uint32_t*>(ab + L.xs2_off);
    args.xsx = reinterpret_cast<const float*>(ab + L.xsx_off);
    args.ids = ids;
    args.E = (int)E;
    args.top_k = (int)top_k;
    args.P = (int)(T * top_k);
    // grid for the most units possible (a batch per pair at most); the rest leave at once
    const int64_t units = T * top_k * args.groups;
    const dim3 grid((unsigned)std::min<int64_t>(units, cu_count()));
    switch (t) {
        case MMQ_Q8_0: launch_xl<MMQ_Q8_0, true, true>(args, grid, s); break;
        case MMQ_Q4_0: launch_xl<MMQ_Q4_0, true, true>(args, grid, s); break;
        case MMQ_Q4_K: launch_xl<MMQ_Q4_K, true, true>(args, grid, s); break;
        case MMQ_IQ1T: launch_xl<MMQ_IQ1T, true, true>(args, grid, s); break;
        case MMQ_IQ1C: launch_xl<MMQ_IQ1C, true, true>(args, grid, s); break;
        case MMQ_Q6_K: launch_xl<MMQ_Q6_K, true, true>(args, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mmvq(mmq_wtype t, const void* packed, const void* act, int64_t M, int64_t N,
                       int64_t K, void* out, int64_t ldo, hipStream_t s) {
    if (!mmvq_dense_ok(M, N)) return hipErrorInvalidValue;
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
    args.nb = (int)ceil_div(M, MV_TOK);
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
        case MMQ_IQ1C: return launch_fmt<MMQ_IQ1C>(args, s);
        case MMQ_I8_ROW: return launch_fmt<MMQ_I8_ROW>(args, s);
        case MMQ_Q6_K: return launch_fmt<MMQ_Q6_K>(args, s);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace mmq
