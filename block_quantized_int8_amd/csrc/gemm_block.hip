// gemm_block.hip - the MMQ contraction for the block-quantised weight formats on CDNA4.
//
//   out[m,n] = sum_b (xs[m,b] * wd[n,b]) * P[m,n,b],   P = sum_{k in b} xq[m,k] * wq[n,k]
//
// ("A Negative Result on int8 Tensor-Core MMQ", section 2; minfer "08 . R1", sections 2.1-2.2.)
//
// Per 32-value block and 32x32 output tile (rows = weight rows n, columns = tokens m):
//  1. v_mfma_i32_32x32x32_i8 forms the exact int32 block dots P. K = 32 is exactly one block, so
//     no two scales ever share an accumulator. Its C operand holds the bits of c = 1/(2 pi)
//     (0x3E22F983, mantissa field 0x22F983): adding an integer P to those bits stays inside the
//     [1/8, 1/4) binade for -2291075 <= P < 6097533, so every result D, read as f32, equals
//     c + P * 2^-26 exactly (|P| <= 548640 for every format).
//  2. v_mfma_f32_32x32x8_f16 forms the scale outer product S = wd (x) xs from one f16 per row on
//     each side (both half-waves contribute, so S = 2 wd xs; a product of two f16 is exact).
//  3. X = D - c = P * 2^-26 exactly, on the matrix core: v_mfma_f32_32x32x8_f16 with C = D and
//     A*B = -c (see unbias_m). Then acc += X * S - one FMA per element on the known 32x32 lane
//     map, in registers: no store -> sync -> reload of the accumulator per block (the pages'
//     "wall", Hanzo paper sections 2-3; the fix is a manual MMA with a known lane map, section
//     4). The 2^26 goes into the epilogue's power-of-two scale.
// Measured on gfx950: a non-packed f32 vector op costs 4 cycles per wave64, v_cvt_f32_i32 about
// twice that, and a matrix-core op that reads a 16-register C operand from VGPRs costs the vector
// unit about 19 cycles. Per tile and block the matrix-core conversion (32 MFMA cycles + one such
// read) beats 16 vector subtractions (64 cycles); packed f32 is not used. The XM switch keeps the
// vector-subtraction form (X = D - c, 16 v_sub) for comparison.
//
//   q4_K: S = xs * (d*sc) from the exact f16 split d*sc = hi + lo (slots 0 and 1 against xs in
//     both), and the rank-1 min term -(dmin*m) * (xs*xsum) (minfer R1 section 2.2: sum w*q =
//     ds * sum nib*q - dmin * sum q) is added straight into the accumulator by
//     v_mfma_f32_32x32x2_f32 over two blocks at once (one per half-wave).
//   q6_K: the 6-bit values q-32 are int8 as they are, but the scale d*sc changes every 16 values
//     (minfer R1 sections 2.2 and 3.3: one 32-k chunk, two half-block integer sums with separate
//     accumulators, rescaled by d*sc0 and d*sc1). Each block runs as two virtual tiles: the
//     int8 MFMA over the fragment with the other half's lanes zeroed (lanes 0-31 carry values
//     0-15, lanes 32-63 values 16-31), its own scale product S_h = 2 (d*sc_h) xs from the exact
//     f16 split hi + lo = d*sc_h, its own conversion, and both FMA into the same accumulator.
//   iq1t: the IQ1_M fold (llama.cpp PR #304) turns each value into the integer
//     (2s+1)(8g + sigma) with a per-block scale d/8 (s per 16 values, sigma = +-1 per 8). Split
//     it as 8(2s+1)g + (2s+1)sigma: the first part (|.| <= 120) is the int8 operand of the one
//     int8 MFMA; the second is constant over each 8-value group j, so its dot with the tokens
//     is sum_j c_j G_j with c_j = (2s+1)sigma_j and G_j the tokens' integer group sums (act
//     region 3). That rank-4 term rides in the conversion MFMA's spare k-slots: -c is written
//     there as two exact f16 products (1303 * 2^-13 + 21 * 311 * 2^-26) and the four products
//     c_j 2^-13 * G_j 2^-13 fill the others, so X = (P + sum_j c_j G_j) 2^-26 exactly - the
//     folded per-32 integer sum_h (2s_h+1) P16_h - from three matrix-core ops per tile and
//     block (int8 dot, scale, conversion), and only d remains as a scale.
//
// Operands reach LDS by direct buffer->LDS DMA (buffer_load_dwordx4 ... lds: each lane names its
// own 16-byte source, the wave writes 1 KB of LDS), double-buffered per 4-block stage: stage
// s+1 is in flight while stage s runs its MFMAs (minfer R1 section 2.3: exposed staging
// latency was the largest single cost; metainfer section 1: global loads of stage i+1 before
// the stage-i MMACs). Nothing is staged through registers, so the copy costs no vector work.
// Token rows are fetched per lane, which is also how MUL_MAT_ID gathers its rows: in gather
// mode every token slot of a tile reads its own activation row and writes its own output row
// (see gemm_id.hip).
#include <algorithm>
#include <type_traits>

#include "gemm_common.h"

namespace mmq {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
constexpr int MAGIC_I = 0x3E22F983;        // bits of 1/(2 pi)
constexpr float MAGIC_F = 0.15915494309189535f;     // the same value as f32
constexpr float UNBIAS = 67108864.0f;      // 2^26: D - c = P * 2^-26
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int KS = 4;                      // blocks per stage: one row's scales = 16 bytes
static_assert(KB_ALIGN % (2 * KS) == 0, "stages come in pairs (two LDS buffers)");

// ------------------------------------------------------------------- weight formats
template <mmq_wtype FMT> struct BT;

// Each format reads its lane's raw fragment bytes from LDS a block ahead (fetch), may do a
// second dependent read (mid, the IQ1T table), and turns them into MFMA operands just before use
// (unpack), so no LDS latency sits in front of an unpack.
template <> struct BT<MMQ_Q8_0> {
    static constexpr int FB = 1024;        // packed fragment bytes per (tile, block)
    static constexpr int NMF = 1;          // int8 MFMAs per block
    static constexpr int SHIFT = 0;        // the MFMA computes P << SHIFT
    static constexpr bool MIN = false;     // q4_K min term
    static constexpr bool DUAL = false;    // q6_K: two half-block dots per block
    static constexpr bool GSUM = false;    // iq1t: group-sum term in the conversion MFMA
    static constexpr bool GRID = false;    // iq1c: grid indices, d per 4-block group
    static constexpr float POST = UNBIAS / 2;   // S = 2 wd xs
    struct Raw { v4i x; };
    __device__ static void fetch(const uint8_t* frag, int lane, Raw& r) {
        r.x = *reinterpret_cast<const v4i*>(frag + lane * 16);
    }
    __device__ static void mid(Raw&, uint32_t, int, const uint8_t*) {}
    __device__ static void unpack(const Raw& r, v4i* a, int) { a[0] = r.x; }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }
};

// q4_0 lane bytes: high nibbles of X0 are k = 16h+0..3, low nibbles 16h+4..7 (X1: 8..15), each
// the 4-bit two's complement of nib - 8; masking (after a shift for the low ones) yields int8
// 16*(nib-8).
template <> struct BT<MMQ_Q4_0> {
    static constexpr int FB = 512;
    static constexpr int NMF = 1;
    static constexpr int SHIFT = 4;
    static constexpr bool MIN = false;
    static constexpr bool DUAL = false;
    static constexpr bool GSUM = false;
    static constexpr bool GRID = false;
    static constexpr float POST = UNBIAS / 32;  // 16x block dot, S = 2 wd xs
    struct Raw { uint2 x; };
    __device__ static void fetch(const uint8_t* frag, int lane, Raw& r) {
        r.x = *reinterpret_cast<const uint2*>(frag + lane * 8);
    }
    __device__ static void mid(Raw&, uint32_t, int, const uint8_t*) {}
    __device__ static void unpack(const Raw& r, v4i* a, int) {
        a[0][0] = (int)(r.x.x & 0xF0F0F0F0u);
        a[0][1] = (int)((r.x.x << 4) & 0xF0F0F0F0u);
        a[0][2] = (int)(r.x.y & 0xF0F0F0F0u);
        a[0][3] = (int)((r.x.y << 4) & 0xF0F0F0F0u);
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }
};

// q4_K lane bytes: unsigned nibbles, X0 & 0x0F0F0F0F = k 16h+0..3, (X0 >> 4) & .. = 16h+4..7.
template <> struct BT<MMQ_Q4_K> {
    static constexpr int FB = 512;
    static constexpr int NMF = 1;
    static constexpr int SHIFT = 0;
    static constexpr bool MIN = true;
    static constexpr bool DUAL = false;
    static constexpr bool GSUM = false;
    static constexpr bool GRID = false;
    static constexpr float POST = UNBIAS / 2;
    struct Raw { uint2 x; };
    __device__ static void fetch(const uint8_t* frag, int lane, Raw& r) {
        r.x = *reinterpret_cast<const uint2*>(frag + lane * 8);
    }
    __device__ static void mid(Raw&, uint32_t, int, const uint8_t*) {}
    __device__ static void unpack(const Raw& r, v4i* a, int) {
        a[0][0] = (int)(r.x.x & 0x0F0F0F0Fu);
        a[0][1] = (int)((r.x.x >> 4) & 0x0F0F0F0Fu);
        a[0][2] = (int)(r.x.y & 0x0F0F0F0Fu);
        a[0][3] = (int)((r.x.y >> 4) & 0x0F0F0F0Fu);
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }     // (hi, lo) of d*sc
};

// iq1t lane data: one dword of 2-bit codes (value 4q+b at bits 8b+2q); the lane's meta byte
// m = s | sigma_a << 3 | sigma_b << 4 (its 16-value half: the sub-scale and the signs of its two
// 8-value groups) sits in its row's scale dword (byte 2 + half). Table entry m (8 bytes):
//   word 0: the int8 values 8(2s+1)(c-1) for the codes c = 0, 1, 2 (bytes 0-2), which v_perm
//           picks by code (selectors 0..2);
//   word 1: the f16 pair (c_a 2^-13, c_b 2^-13), c = (2s+1)(sigma ? -1 : 1): the lane's two
//           conversion-MFMA k-slots of the group-sum term.
template <> struct BT<MMQ_IQ1T> {
    static constexpr int FB = 256;
    static constexpr int NMF = 1;
    static constexpr int SHIFT = 0;
    static constexpr bool MIN = false;
    static constexpr bool DUAL = false;
    static constexpr bool GSUM = true;
    static constexpr bool GRID = false;
    static constexpr float POST = UNBIAS / 16;  // scale d/8, S = 2 d xs
    static constexpr int TAB_WORDS = 64;        // 32 entries x 2 words
    struct Raw { uint32_t C; uint2 t; };
    __device__ static void fetch(const uint8_t* frag, int lane, Raw& r) {
        r.C = *reinterpret_cast<const uint32_t*>(frag + lane * 4);
    }
    __device__ static void mid(Raw& r, uint32_t wsd, int lane, const uint8_t* tab) {
        const uint32_t meta = (wsd >> (16 + 8 * (lane >> 5))) & 0x1Fu;
        r.t = *reinterpret_cast<const uint2*>(tab + meta * 8);
    }
    __device__ static void unpack(const Raw& r, v4i* a, int) {
        const uint32_t C = r.C, lut = r.t.x;
        a[0][0] = (int)__builtin_amdgcn_perm(lut, lut, C & 0x03030303u);
        a[0][1] = (int)__builtin_amdgcn_perm(lut, lut, (C >> 2) & 0x03030303u);
        a[0][2] = (int)__builtin_amdgcn_perm(lut, lut, (C >> 4) & 0x03030303u);
        a[0][3] = (int)__builtin_amdgcn_perm(lut, lut, (C >> 6) & 0x03030303u);
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w & 0xFFFFu; }   // f16 d only
    __device__ static uint32_t table_word(int e, int w) {
        const int s = e & 7, k = 2 * s + 1;
        if (w == 0) return (uint32_t)((-8 * k) & 0xFF) | ((uint32_t)(8 * k) << 16);
        const uint32_t mag = __builtin_bit_cast(uint16_t, (_Float16)((float)k * 0.0001220703125f));
        const uint32_t ca = mag | (((e >> 3) & 1) ? 0x8000u : 0u), cb = mag | (((e >> 4) & 1) ? 0x8000u : 0u);
        return ca | (cb << 16);
    }
};

// iq1c / iq1s grid-index panels: one dword W = ia << 2 | meta << 13 | ib << 20 per lane, ia and
// ib the 11-bit grid indices of its two 8-value groups, meta as for iq1t. The grid sits in LDS
// after the iq1t meta table as two tables of 2048 dwords: entry e's v_perm selectors of its
// values 0-3 (byte b = code of value b) and of its values 4-7. The lane's four selector dwords
// are then lo(ia), hi(ia), lo(ib), hi(ib), read with the two index fields of W as byte offsets
// (ia * 4 and ib * 4), and everything after the lookups is the iq1t step. The scale d comes per
// (row, 4-block stage) from its own region.
template <> struct BT<MMQ_IQ1C> : BT<MMQ_IQ1T> {
    static constexpr bool GRID = true;
    static constexpr int GRID_HI = 2048 * 4;                       // offset of the hi table
    static constexpr int TAB_BYTES = TAB_WORDS * 4 + 2 * GRID_HI;
    struct Raw { uint32_t W; uint2 ga, gb, t; };
    __device__ static void fetch(const uint8_t* frag, int lane, Raw& r) {
        r.W = *reinterpret_cast<const uint32_t*>(frag + lane * 4);
    }
    __device__ static void mid(Raw& r, uint32_t, int, const uint8_t* tab) {
        const uint8_t* g = tab + TAB_WORDS * 4;
        const uint32_t oa = r.W & 0x1FFCu, ob = r.W >> 18;            // ia * 4, ib * 4
        r.ga = make_uint2(*reinterpret_cast<const uint32_t*>(g + oa), *reinterpret_cast<const uint32_t*>(g + GRID_HI + oa));
        r.gb = make_uint2(*reinterpret_cast<const uint32_t*>(g + ob), *reinterpret_cast<const uint32_t*>(g + GRID_HI + ob));
        r.t = *reinterpret_cast<const uint2*>(tab + ((r.W >> 10) & 0xF8u));  // meta * 8
    }
    __device__ static void unpack(const Raw& r, v4i* a, int) {
        const uint32_t lut = r.t.x;
        a[0][0] = (int)__builtin_amdgcn_perm(lut, lut, r.ga.x);
        a[0][1] = (int)__builtin_amdgcn_perm(lut, lut, r.ga.y);
        a[0][2] = (int)__builtin_amdgcn_perm(lut, lut, r.gb.x);
        a[0][3] = (int)__builtin_amdgcn_perm(lut, lut, r.gb.y);
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }            // f16 d
};

// q6_K lane bytes: 16 int8 values q-32 (k = 16h..16h+15), as q8_0. a[0] keeps them on lanes 0-31
// (values 0-15 of the block, half 0) and a[1] on lanes 32-63 (values 16-31, half 1); the other
// lanes are zero, so each int8 MFMA yields one half-block dot. The scale dword of half 0 sits in
// the first scale region, that of half 1 in the second (hi | lo << 16, hi + lo = d*sc_h).
template <> struct BT<MMQ_Q6_K> {
    static constexpr int FB = 1024;
    static constexpr int NMF = 2;
    static constexpr int SHIFT = 0;
    static constexpr bool MIN = false;
    static constexpr bool DUAL = true;
    static constexpr bool GSUM = false;
    static constexpr bool GRID = false;
    static constexpr float POST = UNBIAS / 2;   // S_h = 2 (d*sc_h) xs
    struct Raw { v4i x; };
    __device__ static void fetch(const uint8_t* frag, int lane, Raw& r) {
        r.x = *reinterpret_cast<const v4i*>(frag + lane * 16);
    }
    __device__ static void mid(Raw&, uint32_t, int, const uint8_t*) {}
    __device__ static void unpack(const Raw& r, v4i* a, int hmask) {
        a[0] = r.x & hmask;
        a[1] = r.x & ~hmask;
    }
    __device__ static uint32_t scale_op(uint32_t w) { return w; }     // (hi, lo) of d*sc_h
};

// ------------------------------------------------------------------- kernel configuration
// GATHER_F32: MUL_MAT_ID full units (up to unit_rows pairs of one expert); GATHER_TAIL: the
// tail unit of an expert (the at most TAIL_ROWS pairs after its full units).
enum Mode { DENSE_F32 = 0, DENSE_PARTIALS = 1, GATHER_F32 = 2, GATHER_TAIL = 3 };
constexpr bool is_gather(int mode) { return mode == GATHER_F32 || mode == GATHER_TAIL; }

// WN x WM waves, each owning RT weight tiles x CT token tiles of 32 x 32.
// LDS stage layout (bytes): weight fragments [TN][KS][FB] | token fragments [TM][KS][1024] |
// weight scale dwords | token scale dwords | (q4_K) weight mins | token xs*xsum.
// Fragments arrive in 1 KB chunks (one wave-wide 16-byte DMA each). The scale regions are
// tile-major in memory and in LDS, [tile][KS][32 rows] dwords (512 bytes per tile and stage,
// one cache line per block), so one 16-byte DMA brings a pair of tiles; gathered MUL_MAT_ID
// token rows come one dword per lane instead, a 4-byte DMA per (tile, pair of blocks). The
// per-block reads of 32 consecutive rows are free of bank conflicts.
// Chunk c goes to wave c % NW. Fragment chunk counts are multiples of NW, so the kind of those
// slots is known at compile time; the scale chunks (padded to a multiple of NW) take the last
// slots, their kind chosen per wave.
template <mmq_wtype FMT, int WN, int WM, int RT, int CT, bool GATHER>
struct Cfg {
    using T = BT<FMT>;
    static constexpr int NW = WN * WM, NTH = NW * 64;
    static constexpr int TN = WN * RT, TM = WM * CT;
    static constexpr int WF = TN * KS * T::FB;
    static constexpr int XF = TM * KS * 1024;
    static constexpr int SCB = KS * 32 * 4;                 // one tile's scale dwords per stage
    static constexpr int C_WF = WF / 1024, C_XF = TM * KS;
    // weight scales: a pair of tiles per 1 KB chunk; iq1c: the f16 d of 4 tiles x 32 rows per
    // stage, one 4-byte-per-lane chunk per four tiles
    static constexpr int C_WS = T::GRID ? TN / 4 : (TN + 1) / 2;
    static_assert(!T::GRID || TN % 4 == 0, "one d chunk covers four weight tiles");
    static constexpr int C_XS = GATHER ? TM * KS / 2 : (TM + 1) / 2;
    // second weight-side scale region: q4_K's -dmin*m, q6_K's half-1 scale dwords
    static constexpr bool W2 = T::MIN || T::DUAL;
    static constexpr int C_WM = W2 ? C_WS : 0, C_XM = T::MIN ? C_XS : 0;
    // iq1t: the tokens' group-sum dwords, [TM][KS][64 lanes] (256 bytes per tile and block): a
    // 1 KB chunk per token tile and stage, or (gathered rows) a 4-byte-per-lane chunk per tile
    // and block
    static constexpr int C_XG = T::GSUM ? (GATHER ? TM * KS : TM) : 0;
    static constexpr int RW = T::GRID ? C_WS * 256 : C_WS * 2 * SCB, RX = (TM + 1) / 2 * 2 * SCB;   // region bytes
    static constexpr int O_XF = WF, O_WS = O_XF + XF, O_XS = O_WS + RW;
    static constexpr int O_WM = O_XS + RX, O_XM = O_WM + (W2 ? RW : 0);
    static constexpr int O_XG = O_XM + (T::MIN ? RX : 0);
    static constexpr int BUF = O_XG + (T::GSUM ? TM * KS * 256 : 0);
    static constexpr int C_FR = C_WF + C_XF;
    static constexpr int C_SC = C_WS + C_XS + C_WM + C_XM + C_XG;
    static constexpr int C_ALL = C_FR + (C_SC + NW - 1) / NW * NW;
    static constexpr int CPW = C_ALL / NW;                  // chunks per wave per stage
    static_assert(WF % 1024 == 0, "weight fragments of a stage must be whole 1 KB chunks");
    static_assert(C_WF % NW == 0 && C_XF % NW == 0, "fragment chunks must split evenly over the waves");
    static_assert(KS % 2 == 0, "gathered scale chunks cover two blocks");
    enum { K_WF = 0, K_XF = 1, K_SC = 2 };                      // slot kinds
    enum { S_WS = 0, S_XS = 1, S_WM = 2, S_XM = 3, S_XG = 4, S_NONE = 5 };  // scale chunk kinds
    __host__ __device__ static constexpr int slot_kind(int j) {
        return j * NW < C_WF ? K_WF : j * NW < C_FR ? K_XF : K_SC;
    }
    __host__ __device__ static constexpr int scale_kind(int ci) {
        return ci < C_WS ? S_WS : (ci -= C_WS) < C_XS ? S_XS : (ci -= C_XS) < C_WM ? S_WM
             : (ci -= C_WM) < C_XM ? S_XM : (ci -= C_XM) < C_XG ? S_XG : S_NONE;
    }
    // LDS byte offset of the scale dword of (tile i, row r, block kb) in a region at `base`
    __host__ __device__ static constexpr int sc(int base, int i, int r, int kb) {
        return base + ((i * KS + kb) * 32 + r) * 4;
    }
};

struct BlockArgs {
    const uint8_t* w;           // packed weights (expert 0 in gather mode)
    int64_t w_scale_off;        // offsets of the scale / min regions inside one packed matrix
    int64_t w_min_off;
    int64_t w_stride;           // bytes between experts' packed matrices (gather mode)
    const uint8_t* xq;          // act region 0 (tiled int8)
    const uint32_t* xs2;        // act region 1 (xs as an f16 pair)
    const float* xsx;           // act region 2 (xs * xsum)
    const uint32_t* xg;         // act region 3 (group sums as f16 pairs)
    int M, N, KB, KBp, NT, MT, tiles_m;
    float* out;
    int64_t ldo;
    int32_t* partials;
    int64_t pld;                // partials: elements between consecutive rows m (the full N)
    // gather mode (MUL_MAT_ID)
    const int32_t* offs;        // [E+1] first pair of each expert in `pairs`
    const int32_t* uoff;        // [E+1] first unit of each expert; uoff[E] = live units
    const int32_t* ufull;       // [E+1] full-unit offsets (tail mode: full units per expert)
    const int32_t* pairs;       // pair ids in expert order (pair = token*top_k + slot)
    int E, top_k, ntiles_n, unit_rows;
};

// A buffer descriptor over one operand region (base in scalar registers, no range clamp: every
// offset used stays inside the region by construction).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t region_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
typedef __attribute__((address_space(3))) void lmem_t;
// One wave-wide buffer->LDS DMA of 16 (4) bytes per lane: lane l's bytes at region offset
// voff + soff land at lds + 16 l (4 l). voff is the lane's fixed offset, soff the wave-uniform
// offset of the stage (a scalar register, so advancing a stage costs no vector instruction).
__device__ inline void dma16(rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lmem_t*)lds, 16, (int)voff, soff, 0, 0);
}
__device__ inline void dma4(rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lmem_t*)lds, 4, (int)voff, soff, 0, 0);
}

// an f16x4 operand with the dword `lo` in slots 0-1 and zeros in slots 2-3
__device__ inline h4 as_h4(uint32_t lo) {
    const v2i t = {(int)lo, 0};
    return __builtin_bit_cast(h4, t);
}

// The kernel body, on LDS stage buffers buf0 / buf1 (C::BUF bytes each) and the IQ1T table
// (512 bytes), as workgroup `bid` of `nblk`: a function so that one launch can run two tile
// configurations (MUL_MAT_ID full and tail units, below).
template <mmq_wtype FMT, int WN, int WM, int RT, int CT, int MODE, bool XM>
__device__ __attribute__((always_inline)) inline void block_body(const BlockArgs& args, uint8_t* buf0,
                                                                 uint8_t* buf1, uint8_t* tab, int bid,
                                                                 int nblk) {
    using C = Cfg<FMT, WN, WM, RT, CT, is_gather(MODE)>;
    using T = typename C::T;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wm = wave / WN;
    const int r32 = lane & 31;

    // ---- which tile: dense grids are XCD-swizzled over (n-tile, m-tile) in groups of GM
    // m-tiles, so that an XCD's consecutive logical tiles form a GM x (64 / GM) block whose
    // operand panels its L2 shares (8 x 8 at M = 2048, N = 4096: 8 weight and 8 token panels per
    // XCD instead of 4 and all 16; q4_0 2048 x 4096 x 4096 -1.2 to -2.8%, q6_K -0.9%); gather
    // grids are (unit, n-tile) with the unit list produced on the device
    int nt_base, mt_base = 0, unit_first = 0, unit_count = 0;
    const uint8_t* wbase = args.w;
    if constexpr (is_gather(MODE)) {
        // workgroup b runs on XCD b % 8; unit u = 8 * (rest / ntiles_n) + b % 8 keeps all weight
        // tiles of a unit (which share its activation rows) on one XCD and spreads the live
        // units (the lowest ids) evenly over the XCDs
        const int b = bid, rest = b >> 3;
        const int u = (rest / args.ntiles_n) * 8 + (b & 7);
        // the unit's expert: the largest e < E with uoff[e] <= u (uoff rises from uoff[0] = 0
        // to the unit total uoff[E]). Each lane tests one offset and the wave counts the lanes
        // that pass: one round of loads for E <= 64 (issued with the total's), else a first
        // round over every st-th offset picks the segment of st that holds e.
        const int E = args.E;
        const int total = args.uoff[E];
        int base = 0, span = E;
        if (E > 64) {
            const int st = (E + 63) >> 6;
            const int i = lane * st;
            const bool pass = i < E && args.uoff[i] <= u;
            base = (__popcll(__ballot(pass)) - 1) * st;
            span = min(st, E - base);
        }
        if (u >= total) return;                         // uniform: the whole CTA leaves
        const bool pass = lane < span && args.uoff[base + lane] <= u;
        const int e = base + __popcll(__ballot(pass)) - 1;
        if constexpr (MODE == GATHER_TAIL) {
            unit_first = args.offs[e] + (args.ufull[e + 1] - args.ufull[e]) * args.unit_rows;
            unit_count = args.offs[e + 1] - unit_first;           // 1 .. TAIL_ROWS = TM*32
        } else {
            unit_first = args.offs[e] + (u - args.uoff[e]) * args.unit_rows;
            unit_count = min(args.unit_rows, args.offs[e + 1] - unit_first);
        }
        wbase = args.w + (int64_t)e * args.w_stride;
        nt_base = (rest % args.ntiles_n) * C::TN;
    } else {
        const int lid = xcd_swizzle(bid, nblk);
        constexpr int GM = 8;
        const int tiles_n = nblk / args.tiles_m;
        const int grp = lid / (GM * tiles_n), first_m = grp * GM;
        const int gm = min(GM, args.tiles_m - first_m), in = lid - grp * GM * tiles_n;
        nt_base = (in / gm) * C::TN;
        mt_base = (first_m + in % gm) * C::TM;
    }
    const int NT = args.NT, KBp = args.KBp;

    // Gather: this lane's pair of each token tile (at most two), loaded once for every chunk
    // that needs its token. The pair ids come through a descriptor whose range ends at the
    // unit's last pair (a slot past it reads 0, token 0), so the loads carry no branch; they go
    // out with the grid's loads, ahead of the table writes, whose branch would otherwise put a
    // round trip between them (as per-chunk lookups behind the wave-dependent chunk-kind
    // branches put one behind each). Two scalars, not an array: a selected array element became
    // a dynamic index, and the array was moved to LDS.
    static_assert(!is_gather(MODE) || C::TM <= 2, "gather tiles hold at most two token tiles");
    int tok0 = 0, tok1 = 0;
    if constexpr (is_gather(MODE)) {
        const rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(args.pairs + unit_first), (short)0,
                                                            unit_count * 4, 0x00020000);
        tok0 = __builtin_amdgcn_raw_buffer_load_b32(rp, r32 * 4, 0, 0);
        if constexpr (C::TM > 1) tok1 = __builtin_amdgcn_raw_buffer_load_b32(rp, (32 + r32) * 4, 0, 0);
    }
    // the packed matrix's grid (its last region) as selector tables
    constexpr int GW = T::GRID ? 2048 / C::NTH : 1;
    static_assert(!T::GRID || 2048 % C::NTH == 0, "the grid copy assumes whole rounds of the workgroup");
    uint32_t gw[GW];
    if constexpr (T::GRID) {
        const uint32_t* g = reinterpret_cast<const uint32_t*>(wbase + args.w_min_off);
#pragma unroll
        for (int k = 0; k < GW; ++k) gw[k] = g[tid + k * C::NTH];
    }
    if constexpr (FMT == MMQ_IQ1T || FMT == MMQ_IQ1C) {
        if (tid < T::TAB_WORDS) reinterpret_cast<uint32_t*>(tab)[tid] = T::table_word(tid >> 1, tid & 1);
    }
    if constexpr (T::GRID) {
        uint32_t* lg = reinterpret_cast<uint32_t*>(tab) + T::TAB_WORDS;
#pragma unroll
        for (int k = 0; k < GW; ++k) {
            lg[tid + k * C::NTH] = gw[k] & 0x03030303u;
            lg[2048 + tid + k * C::NTH] = (gw[k] >> 2) & 0x03030303u;
        }
    }
    if constexpr (is_gather(MODE)) {
        tok0 /= args.top_k;
        if constexpr (C::TM > 1) tok1 /= args.top_k;
    }
    // token slot (tile i, row r32) -> activation row to read
    auto row_token = [&](int i) __attribute__((always_inline)) -> int {
        if constexpr (is_gather(MODE)) {
            return (C::TM > 1 && i == 1) ? tok1 : tok0;
        } else {
            return min((mt_base + i) * 32 + r32, args.MT * 32 - 1);
        }
    };

    // ---- DMA plan: per chunk this lane keeps its 32-bit source offset in stage 0 from the
    // chunk's region base; stage st adds st times the region's stage stride as a wave-uniform
    // offset. The chunk's LDS offset is wave-uniform.
    uint32_t goff[C::CPW];
    int ldso[C::CPW];
    int skind[C::CPW];                                       // scale slots: kind, wave-uniform
    const uint8_t* const wsc = wbase + args.w_scale_off;
    const uint8_t* const wmn = wbase + args.w_min_off;
#pragma unroll
    for (int j = 0; j < C::CPW; ++j) {
        const int k = C::slot_kind(j);                       // compile-time per j
        const int c = j * C::NW + wave;
        const int h = lane >> 5;
        skind[j] = C::S_NONE;
        goff[j] = 0;
        ldso[j] = 0;
        if (k == C::K_WF) {
            const int byte = c * 1024 + lane * 16;
            const int tile = byte / (KS * T::FB), off = byte % (KS * T::FB);
            const int nt = min(nt_base + tile, NT - 1);
            goff[j] = (uint32_t)(nt * KBp * T::FB + off);
            ldso[j] = c * 1024;
        } else if (k == C::K_XF) {
            const int ci = c - C::C_WF;
            const int jt = ci / KS, q = ci % KS;
            const int t = row_token(jt);
            goff[j] = (uint32_t)((((t >> 5) * KBp + q) * 64 + h * 32 + (t & 31)) * 16);
            ldso[j] = C::O_XF + ci * 1024;
        } else {
            const int ci = c - C::C_FR;
            const int sk = C::scale_kind(ci);
            skind[j] = sk;
            if (T::GRID && sk == C::S_WS) {
                // iq1c, chunk ci: lane l carries rows 2(l%16), 2(l%16)+1 of tile 4 ci + l/16
                // (their f16 d of the stage's 4-block group: 64 bytes per tile and stage)
                const int nt = min(nt_base + 4 * ci + (lane >> 4), NT - 1);
                goff[j] = (uint32_t)((nt * (KBp / 4) * 32 + 2 * (lane & 15)) * 2);
                ldso[j] = C::O_WS + ci * 256;
            } else if (sk == C::S_WS || sk == C::S_WM) {
                // a pair of weight tiles: lanes 0-31 tile 2pr, lanes 32-63 tile 2pr+1, 16 bytes
                // each of the tile's contiguous 512-byte stage
                const int pr = ci - (sk == C::S_WS ? 0 : C::C_WS + C::C_XS);
                const int nt = min(nt_base + 2 * pr + h, NT - 1);
                goff[j] = (uint32_t)(nt * KBp * 128 + r32 * 16);
                ldso[j] = (sk == C::S_WS ? C::O_WS : C::O_WM) + pr * 1024;
            } else if (sk == C::S_XG) {
                const int x = ci - (C::C_WS + C::C_XS + C::C_WM + C::C_XM);
                if constexpr (is_gather(MODE)) {
                    // (tile i, block kb): lane (h, r) fetches the dword of half h of its row
                    const int i = x / KS, kb = x % KS;
                    const int m = row_token(i);
                    goff[j] = (uint32_t)((((m >> 5) * KBp + kb) * 64 + h * 32 + (m & 31)) * 4);
                    ldso[j] = C::O_XG + (i * KS + kb) * 256;
                } else {
                    const int mt = min(mt_base + x, args.MT - 1);
                    goff[j] = (uint32_t)(mt * KBp * 256 + lane * 16);
                    ldso[j] = C::O_XG + x * 1024;
                }
            } else if (sk == C::S_XS || sk == C::S_XM) {
                const int x = ci - (sk == C::S_XS ? C::C_WS : C::C_WS + C::C_XS + C::C_WM);
                const int base = sk == C::S_XS ? C::O_XS : C::O_XM;
                if constexpr (is_gather(MODE)) {
                    // (tile i, blocks 2bp and 2bp+1): each lane fetches its own gathered row's dword
                    const int i = x / (KS / 2), bp = x % (KS / 2);
                    const int m = row_token(i);
                    goff[j] = (uint32_t)((((m >> 5) * KBp + 2 * bp + h) * 32 + (m & 31)) * 4);
                    ldso[j] = base + (i * KS + 2 * bp) * 128;
                } else {
                    const int mt = min(mt_base + 2 * x + h, args.MT - 1);
                    goff[j] = (uint32_t)(mt * KBp * 128 + r32 * 16);
                    ldso[j] = base + x * 1024;
                }
            }
        }
    }
    const rsrc_t rs_w = region_rsrc(wbase), rs_x = region_rsrc(args.xq), rs_ws = region_rsrc(wsc);
    const rsrc_t rs_wm = region_rsrc(wmn), rs_xs = region_rsrc(args.xs2), rs_xm = region_rsrc(args.xsx);
    const rsrc_t rs_xg = region_rsrc(args.xg);
    // chunk j of stage st into stage buffer buf
    auto issue_chunk = [&](uint8_t* buf, int j, int st) __attribute__((always_inline)) {
        const int k = C::slot_kind(j);
        uint8_t* dst = buf + __builtin_amdgcn_readfirstlane(ldso[j]);
        if (k == C::K_WF) {
            dma16(rs_w, dst, goff[j], st * (KS * T::FB));
        } else if (k == C::K_XF) {
            dma16(rs_x, dst, goff[j], st * (KS * 1024));
        } else {
            // one wave-uniform branch per kind, each with its own descriptor (a descriptor picked
            // by a runtime kind made the compiler build a descriptor table in scratch memory)
            const int sk = __builtin_amdgcn_readfirstlane(skind[j]);
            const uint32_t v = goff[j];
            if (sk == C::S_WS) {
                if constexpr (T::GRID) dma4(rs_ws, dst, v, st * 64);
                else dma16(rs_ws, dst, v, st * C::SCB);
            } else if (sk == C::S_XS) {
                if constexpr (is_gather(MODE)) dma4(rs_xs, dst, v, st * C::SCB);
                else dma16(rs_xs, dst, v, st * C::SCB);
            } else if (C::C_WM > 0 && sk == C::S_WM) {
                dma16(rs_wm, dst, v, st * C::SCB);
            } else if (C::C_XM > 0 && sk == C::S_XM) {
                if constexpr (is_gather(MODE)) dma4(rs_xm, dst, v, st * C::SCB);
                else dma16(rs_xm, dst, v, st * C::SCB);
            } else if (C::C_XG > 0 && sk == C::S_XG) {
                if constexpr (is_gather(MODE)) dma4(rs_xg, dst, v, st * (KS * 256));
                else dma16(rs_xg, dst, v, st * (KS * 256));
            }
        }
    };
    auto issue_stage = [&](uint8_t* buf, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < C::CPW; ++j) issue_chunk(buf, j, st);
    };

    v16f acc[RT][CT];
#pragma unroll
    for (int x = 0; x < RT; ++x)
#pragma unroll
        for (int y = 0; y < CT; ++y)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

    const v16f zf = {0};
    v16i magic;
#pragma unroll
    for (int r = 0; r < 16; ++r) magic[r] = MAGIC_I;

    // Steps per block: one per tile, two per tile for q6_K (its half-blocks, "virtual tiles"
    // t = 2 * tile + half that share the tile's accumulator).
    constexpr int NH = T::DUAL ? 2 : 1;
    constexpr int NT_ = RT * CT * NH;
    const int hmask = lane < 32 ? -1 : 0;                 // q6_K: lanes of half-block 0
    // one block's operands for this wave: raw LDS words (fetched a block ahead), then the MFMA
    // operands unpacked from them one step before the block starts
    struct Raw {
        typename T::Raw w[RT];
        v4i b[CT];
        uint32_t wsd[RT], wsd2[RT], xs[CT], gx[CT];
    };
    // The f16 scale MFMA takes (scale, 0) register pairs. In the kernels of 2 x 2 tiles per wave
    // (dense 128 x 128, MUL_MAT_ID full units of 256 rows) the operand buffers live for the whole
    // K loop and only the scale halves are rewritten, so no step spends a move on the zeros
    // (q4_0 N = 11008: -2%; MoE 0 to -1.4%). The other kernels pair each scale at its MFMA: q6_K
    // needs every register it can keep, the gather kernels of one weight tile per wave hold
    // three waves per SIMD only up to 168, and the one-tile-per-wave kernels measured slower
    // with carried pairs.
    constexpr bool CARRY = !T::DUAL && RT * CT >= 4;
    constexpr bool PRIO = !is_gather(MODE);         // see the step schedule below
    using SOp = std::conditional_t<CARRY, v2i, uint32_t>;
    struct Ops {
        v4i a[RT][T::NMF];
        v4i b[CT];
        SOp ws[RT], ws2[RT], xs[CT];
        uint32_t cw[RT], gx[CT];               // iq1t: conversion k-slot pairs (weights, tokens)
    };
    auto set_lo = [](SOp& p, uint32_t v) __attribute__((always_inline)) {
        if constexpr (CARRY) p.x = (int)v;
        else p = v;
    };
    auto pair = [](const SOp& p) __attribute__((always_inline)) -> h4 {
        if constexpr (CARRY) return __builtin_bit_cast(h4, p);
        else return as_h4(p);
    };
    auto fetch = [&](const uint8_t* cur, int kb, Raw& R) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int i = wn * RT + rt;
            if constexpr (T::GRID)
                R.wsd[rt] = *reinterpret_cast<const uint16_t*>(cur + C::O_WS + (i * 32 + r32) * 2);
            else
                R.wsd[rt] = *reinterpret_cast<const uint32_t*>(cur + C::sc(C::O_WS, i, r32, kb));
            if constexpr (T::DUAL) R.wsd2[rt] = *reinterpret_cast<const uint32_t*>(cur + C::sc(C::O_WM, i, r32, kb));
            T::fetch(cur + (i * KS + kb) * T::FB, lane, R.w[rt]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int j = wm * CT + ct;
            R.b[ct] = *reinterpret_cast<const v4i*>(cur + C::O_XF + (j * KS + kb) * 1024 + lane * 16);
            R.xs[ct] = *reinterpret_cast<const uint32_t*>(cur + C::sc(C::O_XS, j, r32, kb));
            if constexpr (T::GSUM)
                R.gx[ct] = *reinterpret_cast<const uint32_t*>(cur + C::O_XG + ((j * KS + kb) * 64 + lane) * 4);
        }
    };
    auto mid = [&](Raw& R) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) T::mid(R.w[rt], R.wsd[rt], lane, tab);
    };
    auto unpack = [&](const Raw& R, Ops& o) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            T::unpack(R.w[rt], o.a[rt], hmask);
            if constexpr (T::GSUM) o.cw[rt] = R.w[rt].t.y;
            set_lo(o.ws[rt], T::scale_op(R.wsd[rt]));
            if constexpr (T::DUAL) set_lo(o.ws2[rt], T::scale_op(R.wsd2[rt]));
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            o.b[ct] = R.b[ct];
            set_lo(o.xs[ct], R.xs[ct]);
            if constexpr (T::GSUM) o.gx[ct] = R.gx[ct];
        }
    };
    auto load_ops = [&](const uint8_t* cur, int kb, Ops& o) __attribute__((always_inline)) {
        Raw R;
        fetch(cur, kb, R);
        mid(R);
        unpack(R, o);
    };

    // matrix-core half of tile t of a block: D (exact int32 dots), S (scale outer product)
    // step t -> (weight tile rt, token tile ct, half hf); hf is 0 except for q6_K
    auto mfma_dots = [&](const Ops& o, int t) __attribute__((always_inline)) -> v16i {
        const int tt = t / NH, hf = t % NH, rt = tt / CT, ct = tt % CT;
        if constexpr (T::DUAL) return __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[rt][hf], o.b[ct], magic, 0, 0, 0);
        v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[rt][0], o.b[ct], magic, 0, 0, 0);
        if constexpr (T::NMF == 2) D = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[rt][1], o.b[ct], D, 0, 0, 0);
        return D;
    };
    auto mfma_scale = [&](const Ops& o, int t) __attribute__((always_inline)) -> v16f {
        const int tt = t / NH, hf = t % NH, rt = tt / CT, ct = tt % CT;
        return __builtin_amdgcn_mfma_f32_32x32x8f16(pair(hf ? o.ws2[rt] : o.ws[rt]), pair(o.xs[ct]), zf, 0, 0, 0);
    };
    // The empty asm after a tile's last FMA pins its accumulator: FMAs are pure, and left alone
    // the compiler sinks a whole stage of them below its matrix-core work, which then has to
    // hold every X and S at once.
    // Conversion on the matrix core (XM): v_mfma_f32_32x32x8_f16 with C = D and A*B = -c, c
    // written as three exact f16 products (its 24-bit significand 0xA2F983 byte by byte, each
    // byte * 2^-13 against 8, 2^-5 and 2^-13, low half-wave only): X = D - c exactly, whatever
    // order the matrix core adds in.
    const v2i cAi = {lane < 32 ? (int)0xA7C8A510u : 0, lane < 32 ? (int)0x0000A418u : 0};
    const v2i cBi = {(int)0x28004800u, (int)0x00000800u};
    // iq1t: k-slots 0-1 (low half-wave) and 4-5 (high half-wave) carry the lane's group-sum
    // pairs c_j 2^-13 x G_j 2^-13; slots 2-3 of the low half carry -c = -(1303 * 2^-10) * 2^-3
    // - (21 * 2^-13) * (311 * 2^-13) (f16 0xBD17 x 0x3000, 0x9940 x 0x28DC); 6-7 are zero.
    const uint32_t gA1 = lane < 32 ? 0x9940BD17u : 0u, gB1 = lane < 32 ? 0x28DC3000u : 0u;
    auto unbias_m = [&](const v16i& D, const Ops& o, int t) __attribute__((always_inline)) -> v16f {
        if constexpr (T::GSUM) {
            const int tt = t / NH, rt = tt / CT, ct = tt % CT;
            const v2i ga = {(int)o.cw[rt], (int)gA1}, gb = {(int)o.gx[ct], (int)gB1};
            return __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(h4, ga), __builtin_bit_cast(h4, gb),
                                                        __builtin_bit_cast(v16f, D), 0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(h4, cAi), __builtin_bit_cast(h4, cBi),
                                                        __builtin_bit_cast(v16f, D), 0, 0, 0);
        }
    };
    // D -> X = D - c, in place: 16 independent subtractions. (The whole vector is
    // reinterpreted at once: hipcc's __builtin_bit_cast of a single vector element reads element
    // 0 whatever the index.)
    auto unbias = [&](const v16i& D) __attribute__((always_inline)) -> v16f {
        return __builtin_bit_cast(v16f, D) - MAGIC_F;
    };
    // acc += X * S: 16 independent FMAs. The empty asm after them pins the accumulator: FMAs are
    // pure, and left alone the compiler sinks a whole stage of them below its matrix-core work,
    // which then has to hold every D and S at once.
    auto fma_tile = [&](int t, const v16f& X, const v16f& S, int r0 = 0, int r1 = 16) __attribute__((always_inline)) {
        const int tt = t / NH, rt = tt / CT, ct = tt % CT;
#pragma unroll
        for (int r = r0; r < r1; ++r) acc[rt][ct][r] = __builtin_fmaf(X[r], S[r], acc[rt][ct][r]);
        if (r1 == 16) asm volatile("" : "+v"(acc[rt][ct]));
    };
    // partials mode: the exact int32 dots of block kbg go straight to memory
    // (q6_K: the dot of half hf of block kbg goes to index 2 kbg + hf of 2 KB per (m, n))
    // (iq1t: the dot of the int8 MFMA lacks the group-sum term, so the folded integer is taken
    // from the conversion's exact X = I * 2^-26 instead)
    auto store_partials = [&](int kbg, int t, const v16i& D, const Ops& o) __attribute__((always_inline)) {
        const int tt = t / NH, hf = t % NH, rt = tt / CT, ct = tt % CT;
        const int m = (mt_base + wm * CT + ct) * 32 + r32;
        v16i I;
        if constexpr (T::GSUM) {
            const v16f X = unbias_m(D, o, t);
#pragma unroll
            for (int r = 0; r < 16; ++r) I[r] = (int)(X[r] * UNBIAS);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) I[r] = (D[r] - MAGIC_I) >> T::SHIFT;
        }
        if (kbg < args.KB && m < args.M) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = (nt_base + wn * RT + rt) * 32 + acc_row(lane, r);
                if (n < args.N)
                    args.partials[((int64_t)m * args.pld + n) * (NH * args.KB) + NH * kbg + hf] = I[r];
            }
        }
    };
    // q4_K: the min term of blocks (2p, 2p+1) of the stage, one half-wave per block
    auto min_term = [&](const uint8_t* cur, int p) __attribute__((always_inline)) {
        if constexpr (T::MIN) {
            const int kb = 2 * p + (lane >> 5);
            float wv[RT], xv[CT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                wv[rt] = *reinterpret_cast<const float*>(cur + C::sc(C::O_WM, wn * RT + rt, r32, kb));
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)      // * 2^-25, like S = 2 wd xs times D - c = P 2^-26
                xv[ct] = (2.0f / UNBIAS) * *reinterpret_cast<const float*>(cur + C::sc(C::O_XM, wm * CT + ct, r32, kb));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(wv[rt], xv[ct], acc[rt][ct], 0, 0, 0);
        }
    };

    // One stage: KS blocks x NT_ tiles as one software pipeline. Step i issues the matrix-core
    // work of step i+1 (dots, scale, conversion) around the vector FMAs of step i, so the
    // matrix core and the vector unit stay busy together. The next block's operands are read
    // from LDS at its first step and unpacked at its last.
    // `nxt` (if not null) receives the DMA of the following stage: its chunks are issued a few
    // per step (one per step when there are enough steps) over the first steps, so the
    // vector-memory issue never holds a wave for long.
    // operand buffers: for the whole K loop when the scale pairs are carried (their zero halves
    // set once), else per stage
    Ops op_keep[2];
    if constexpr (CARRY) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) op_keep[i].ws[rt] = op_keep[i].ws2[rt] = SOp{};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) op_keep[i].xs[ct] = SOp{};
        }
    }
    auto run_stage = [&](const uint8_t* cur, int s, uint8_t* nxt) __attribute__((always_inline)) {
        Ops op_own[2];
        Ops (&op)[2] = *(CARRY ? &op_keep : &op_own);
        Raw raw;
        load_ops(cur, 0, op[0]);
        v16i Dc;
        v16f Sc, Xc;
        Dc = mfma_dots(op[0], 0);
        if constexpr (MODE == DENSE_PARTIALS) store_partials(s * KS, 0, Dc, op[0]);
        else Sc = mfma_scale(op[0], 0);
        if constexpr (XM && MODE != DENSE_PARTIALS) Xc = unbias_m(Dc, op[0], 0);
#pragma unroll
        for (int kb = 0; kb < KS; ++kb) {
#pragma unroll
            for (int t = 0; t < NT_; ++t) {
                const bool more = t + 1 < NT_ || kb + 1 < KS;
                const int kn = (t + 1 < NT_) ? kb : kb + 1, tn = (t + 1) % NT_;
                if (nxt != nullptr) {
                    constexpr int PER = (C::CPW + KS * NT_ - 1) / (KS * NT_);   // chunks per step
                    const int st = kb * NT_ + t;
#pragma unroll
                    for (int j = st * PER; j < st * PER + PER; ++j)
                        if (j < C::CPW) issue_chunk(nxt, j, s + 1);
                }
                if (kb + 1 < KS) {
                    if (t == 0) fetch(cur, kb + 1, raw);
                    if (t == (NT_ >= 3 ? NT_ - 2 : 0)) mid(raw);
                    if (t == NT_ - 1) unpack(raw, op[(kb + 1) & 1]);
                }
                if constexpr (MODE == DENSE_PARTIALS) {
                    if (more) store_partials(s * KS + kn, tn, mfma_dots(op[kn & 1], tn), op[kn & 1]);
                } else {
                    v16i Dn;
                    v16f Sn;
                    if constexpr (XM) {
                        // Three fenced thirds per step: each matrix-core op of the next tile (dots,
                        // scale, conversion) over a run of this tile's FMAs (X came from the matrix
                        // core one step ago), 5 / 5 / 6 of them (with the priority below, 0.4-0.9%
                        // faster than 6 / 5 / 5 on every block workload).
                        // Wave priority: raised for the first two thirds of the step and lowered
                        // for the last, so that of two waves on a SIMD the one in its first two
                        // thirds issues first (dense kernels: q4_0 2048 x 4096 x 4096 76.8 ->
                        // 74.3 / 73.8 us, Q4_K -2.7%, q6_K -2.9%).
                        v16f Xn;
                        __builtin_amdgcn_sched_barrier(0);
                        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
                        if (more) {
                            Dn = mfma_dots(op[kn & 1], tn);
                            __builtin_amdgcn_sched_group_barrier(0x008, T::NMF, 0);
                        }
                        fma_tile(t, Xc, Sc, 0, 5);
                        __builtin_amdgcn_sched_barrier(0);
                        if (more) Sn = mfma_scale(op[kn & 1], tn);
                        fma_tile(t, Xc, Sc, 5, 10);
                        __builtin_amdgcn_sched_barrier(0);
                        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
                        if (more) Xn = unbias_m(Dn, op[kn & 1], tn);
                        fma_tile(t, Xc, Sc, 10, 16);
                        __builtin_amdgcn_sched_barrier(0);
                        Xc = Xn;
                    } else {
                        // Two fenced halves per step, each a matrix-core op over a run of
                        // independent vector ops of the previous tile: the int8 MFMA of the next
                        // tile with this tile's 16 subtractions, then the scale MFMA with its 16
                        // FMAs. (Unfenced, the scheduler threads subtractions and FMAs into one
                        // dependent chain through a single temporary.)
                        __builtin_amdgcn_sched_barrier(0);
                        const v16f X = unbias(Dc);
                        if (more) {
                            Dn = mfma_dots(op[kn & 1], tn);
                            __builtin_amdgcn_sched_group_barrier(0x008, T::NMF, 0);
                            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        fma_tile(t, X, Sc);
                        if (more) {
                            Sn = mfma_scale(op[kn & 1], tn);
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (T::MIN && t == NT_ - 1 && (kb & 1)) min_term(cur, kb >> 1);
                    Dc = Dn;
                    Sc = Sn;
                }
            }
        }
    };

    const int nstages = KBp / KS;                // even: KBp is a multiple of 8
    issue_stage(buf0, 0);
    for (int s = 0; s < nstages; s += 2) {
        __builtin_amdgcn_s_waitcnt(0x3f70);      // vmcnt(0): this wave's DMA of stage s landed
        __syncthreads();                          // ... and everyone's; stage s-1 fully consumed
        run_stage(buf0, s, buf1);                 // stage s+1 streams into buf1 meanwhile
        __builtin_amdgcn_s_waitcnt(0x3f70);
        __syncthreads();
        run_stage(buf1, s + 1, s + 2 < nstages ? buf0 : nullptr);
    }

    if constexpr (MODE != DENSE_PARTIALS) {
        const int64_t ldo = args.ldo;
        const bool vec_ok = (ldo & 3) == 0;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            int row;
            if constexpr (is_gather(MODE)) {
                const int sl = (wm * CT + ct) * 32 + r32;
                row = sl < unit_count ? args.pairs[unit_first + sl] : -1;
            } else {
                const int m = (mt_base + wm * CT + ct) * 32 + r32;
                row = m < args.M ? m : -1;
            }
            if (row < 0) continue;
            float* orow = args.out + (int64_t)row * ldo;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n0 = (nt_base + wn * RT + rt) * 32 + 8 * g + 4 * (lane >> 5);
                    const float v0 = acc[rt][ct][4 * g + 0] * T::POST, v1 = acc[rt][ct][4 * g + 1] * T::POST;
                    const float v2 = acc[rt][ct][4 * g + 2] * T::POST, v3 = acc[rt][ct][4 * g + 3] * T::POST;
                    if (vec_ok && n0 + 3 < args.N) {
                        *reinterpret_cast<float4*>(orow + n0) = make_float4(v0, v1, v2, v3);
                    } else {
                        if (n0 + 0 < args.N) orow[n0 + 0] = v0;
                        if (n0 + 1 < args.N) orow[n0 + 1] = v1;
                        if (n0 + 2 < args.N) orow[n0 + 2] = v2;
                        if (n0 + 3 < args.N) orow[n0 + 3] = v3;
                    }
                }
        }
    }
}

template <mmq_wtype FMT, int WN, int WM, int RT, int CT, int MODE, bool XM>
__global__ __launch_bounds__(WN * WM * 64, 2) void mmq_block_kernel(BlockArgs args) {
    using C = Cfg<FMT, WN, WM, RT, CT, is_gather(MODE)>;
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[C::BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[C::BUF];
    __shared__ __attribute__((aligned(16))) uint8_t tab[FMT == MMQ_IQ1C ? BT<MMQ_IQ1C>::TAB_BYTES : FMT == MMQ_IQ1T ? 256 : 16];
    block_body<FMT, WN, WM, RT, CT, MODE, XM>(args, buf0, buf1, tab, (int)blockIdx.x, (int)gridDim.x);
}

// MUL_MAT_ID in one launch: the first workgroups run the full units (CT tiles of tokens per
// wave), the next ones the tail units (TCT tiles), so the tails start as soon as full-unit
// workgroups leave, instead of after the whole full-unit launch. The grid is sized for the
// worst case (nfull full-unit and the rest tail-unit workgroups); the split point is the live
// full-unit count the routing wrote (rounded up to 8 units), so the workgroups of units that do
// not exist all come last instead of between the full and the tail units, where the dispatcher
// spent ~5 us retiring 1024 of them on the 64-expert workload before any tail started (about
// 1 us of the whole machine's time: MoE IQ1C 136.3 -> 135.7 us). Both
// split points are multiples of 8, so both parts keep the workgroup -> XCD assignment of their
// own grid. LDS holds the larger configuration.
template <mmq_wtype FMT, int WN, int WM, int RT, int CT, int TCT, bool XM>
__global__ __launch_bounds__(WN * WM * 64, 2) void mmq_gather_kernel(BlockArgs full, BlockArgs tail, int nfull) {
    using CF = Cfg<FMT, WN, WM, RT, CT, true>;
    using CTl = Cfg<FMT, WN, WM, RT, TCT, true>;
    constexpr int BUF = CF::BUF > CTl::BUF ? CF::BUF : CTl::BUF;
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[BUF];
    __shared__ __attribute__((aligned(16))) uint8_t tab[FMT == MMQ_IQ1C ? BT<MMQ_IQ1C>::TAB_BYTES : FMT == MMQ_IQ1T ? 256 : 16];
    const int b = (int)blockIdx.x;
    const int live_full = ((full.uoff[full.E] + 7) & ~7) * full.ntiles_n;   // <= nfull
    if (b < live_full) block_body<FMT, WN, WM, RT, CT, GATHER_F32, XM>(full, buf0, buf1, tab, b, nfull);
    else if (b - live_full < (int)gridDim.x - nfull)
        block_body<FMT, WN, WM, RT, TCT, GATHER_TAIL, XM>(tail, buf0, buf1, tab, b - live_full, (int)gridDim.x - nfull);
}

// Tile configuration: 2 x 2 waves, each owning 2 weight tiles x 2 token tiles -> 128 x 128
// CTA tiles.
constexpr int WN_ = 2, WM_ = 2, RT_ = 2, CT_ = 2;
constexpr bool XM_ = true;        // conversion on the matrix core (see the kernel notes)
// MUL_MAT_ID: 4 x 1 waves, each gather_rt<FMT>() weight tiles x 2 token tiles -> 256 (or 128)
// weight rows x 64 token slots per full unit. An expert sees about T*top_k/E pairs (64 +- 8 for
// 512 tokens, top-8 of 64), so 64-slot units leave fewer empty slots than 128-slot ones. An
// expert's remainder of at most 32 pairs is one tail unit (one token tile per wave); a larger
// remainder is one more full unit. Two weight tiles per wave read and unpack one weight
// fragment and one token fragment per tile-step, like the dense 2 x 2 tiles, instead of 1.5;
// they need ~230 registers (two waves per SIMD instead of three) and twice the weight staging,
// so a format takes them where two workgroups still fit in a CU's LDS (q4_0, Q4_K, IQ1T, IQ1C;
// not q8_0 and q6_K, whose 1 KB fragments would leave one). A/B on the 64-expert, 512-token
// workload against one tile per wave: IQ1T 140.8 -> 131.1 us, q4_0 weights 150.2 -> 129.8, Q4_K
// 177.3 -> 165.4; 2048 tokens (IQ1T) 490 -> 432. (96-slot full units with 64-slot tails read
// every expert's weights once on that routing, but at one weight tile per wave needed 198
// instead of 160 registers for IQ1T and measured 2.5% slower.)
constexpr int GWN_ = 4, GWM_ = 1, GRT_ = 1, GCT_ = 2;
constexpr int TCT_ = 1;
// LDS of a gather workgroup with RT weight tiles per wave: two stage buffers of the larger of the
// full-unit and tail configurations, plus the format's table
template <mmq_wtype FMT, int RT>
constexpr int gather_lds_bytes() {
    using CF = Cfg<FMT, GWN_, GWM_, RT, GCT_, true>;
    using CT = Cfg<FMT, GWN_, GWM_, RT, TCT_, true>;
    return 2 * (CF::BUF > CT::BUF ? CF::BUF : CT::BUF) +
           (FMT == MMQ_IQ1C ? BT<MMQ_IQ1C>::TAB_BYTES : FMT == MMQ_IQ1T ? 256 : 16);
}
constexpr int LDS_PER_CU = 160 * 1024;
template <mmq_wtype FMT>
constexpr int gather_rt() { return 2 * gather_lds_bytes<FMT, 2>() + 2048 <= LDS_PER_CU ? 2 : 1; }
constexpr int UNIT_ROWS = GWM_ * GCT_ * 32;
constexpr int TAIL_ROWS = GWM_ * TCT_ * 32;
static_assert(TAIL_ROWS < UNIT_ROWS, "a tail unit is smaller than a full unit");
// Small dense problems: 4 x 1 waves of one tile each, 128 weight rows x 32 token rows.
constexpr int DCT_ = 1;

template <mmq_wtype FMT>
BlockArgs dense_args(const void* packed, const void* act, int64_t M, int64_t N, int64_t K) {
    const PackedLayout P = packed_layout(FMT, N, K);
    const ActQ81Layout A = act_q8_1_layout(M, K);
    const uint8_t* ab = static_cast<const uint8_t*>(act);
    BlockArgs g{};
    g.w = static_cast<const uint8_t*>(packed) + P.frag_off;
    g.w_scale_off = P.scale_off - P.frag_off;
    g.w_min_off = P.min_off - P.frag_off;
    g.w_stride = 0;
    g.xq = ab + A.xq_off;
    g.xs2 = reinterpret_cast<const uint32_t*>(ab + A.xs2_off);
    g.xsx = reinterpret_cast<const float*>(ab + A.xsx_off);
    g.xg = reinterpret_cast<const uint32_t*>(ab + A.xg_off);
    g.M = (int)M;
    g.N = (int)N;
    g.KB = (int)A.KB;
    g.KBp = (int)A.KBp;
    g.NT = (int)P.NT;
    g.MT = (int)A.MT;
    return g;
}

template <mmq_wtype FMT, int WN, int WM, int RT, int CT>
hipError_t launch_dense_cfg(BlockArgs g, int64_t M, int64_t N, mmq_otype o, void* out, hipStream_t s) {
    const int tiles_n = (int)ceil_div(N, WN * RT * 32);
    const int tiles_m = (int)ceil_div(M, WM * CT * 32);
    g.tiles_m = tiles_m;
    const dim3 grid((unsigned)((int64_t)tiles_n * tiles_m)), block(WN * WM * 64);
    if (o == MMQ_OUT_I32_PARTIALS) {
        g.partials = static_cast<int32_t*>(out);
        hipLaunchKernelGGL((mmq_block_kernel<FMT, WN, WM, RT, CT, DENSE_PARTIALS, XM_>), grid, block, 0, s, g);
    } else {
        g.out = static_cast<float*>(out);
        hipLaunchKernelGGL((mmq_block_kernel<FMT, WN, WM, RT, CT, DENSE_F32, XM_>), grid, block, 0, s, g);
    }
    return hipGetLastError();
}

// Dense tile shape: 128 x 128 while that gives the chip about two workgroups per CU; smaller
// problems (few token or weight tiles, e.g. M = 512 with N = 4096) use 128 weight rows x 32
// token slots (4 x 1 waves, one tile each) and four times the workgroups.
constexpr int64_t DENSE_FILL = 448;

// The kernel keeps 32-bit byte offsets from each operand region's base (the DMA plan) and its
// grid stays below MAX_GRID workgroups, so a problem whose weight or activation regions reach
// 2 GiB (e.g. a 262144 x 8192 q8_0 vocabulary matrix) runs as several launches over ranges of
// weight tiles and token tiles: each launch sees its own slice of the tile-major regions.
constexpr int64_t MAX_REGION = int64_t(1) << 31;
constexpr int64_t MAX_GRID_ = (int64_t(1) << 24) - 1;

template <mmq_wtype FMT, int WN, int WM, int RT, int CT>
hipError_t launch_dense_split(const BlockArgs& g0, int64_t M, int64_t N, mmq_otype o, void* out,
                              int64_t ldo, int64_t scale_off, int64_t min_off, hipStream_t s) {
    constexpr int TN = WN * RT, TM = WM * CT;                // 32-row tiles per workgroup
    // the largest per-tile region: a tile's fragments of every block (q8_0, q6_K and the
    // activations: 1 KB per block)
    const int64_t tile_bytes = (int64_t)g0.KBp * 1024;
    const int64_t ntile_cap = std::max<int64_t>(TN, (MAX_REGION - 1) / tile_bytes / TN * TN);
    const int64_t mtile_cap = std::max<int64_t>(TM, (MAX_REGION - 1) / tile_bytes / TM * TM);
    const int64_t NT = g0.NT, MT = g0.MT;
    const int64_t nstep = std::min(ntile_cap, NT);
    const int64_t mstep = std::min(mtile_cap, std::max<int64_t>(TM, MAX_GRID_ / ceil_div(nstep, TN) / TM * TM));
    const int64_t FB = BT<FMT>::FB;
    for (int64_t mt0 = 0; mt0 < MT; mt0 += mstep) {
        for (int64_t nt0 = 0; nt0 < NT; nt0 += nstep) {
            BlockArgs g = g0;
            const int64_t NTc = std::min(nstep, NT - nt0), MTc = std::min(mstep, MT - mt0);
            const int64_t Nc = std::min(NTc * 32, N - nt0 * 32), Mc = std::min(MTc * 32, M - mt0 * 32);
            const int64_t wshift = nt0 * g0.KBp * FB;             // fragments of the skipped tiles
            // their scale dwords (iq1c: their d per 4-block group; its grid region is shared)
            const int64_t sshift = BT<FMT>::GRID ? nt0 * (g0.KBp / 4) * 64 : nt0 * g0.KBp * 128;
            g.w = g0.w + wshift;
            g.w_scale_off = scale_off + sshift - wshift;
            g.w_min_off = min_off + (BT<FMT>::GRID ? 0 : sshift) - wshift;
            g.xq = g0.xq + mt0 * g0.KBp * 1024;
            g.xs2 = g0.xs2 + mt0 * g0.KBp * 32;
            g.xsx = g0.xsx + mt0 * g0.KBp * 32;
            g.xg = g0.xg + mt0 * g0.KBp * 64;
            g.M = (int)Mc;
            g.N = (int)Nc;
            g.NT = (int)NTc;
            g.MT = (int)MTc;
            g.pld = N;
            void* o_sub;
            if (o == MMQ_OUT_I32_PARTIALS) {
                const int64_t per = (FMT == MMQ_Q6_K ? 2 : 1) * (int64_t)g0.KB;
                o_sub = static_cast<int32_t*>(out) + (mt0 * 32 * N + nt0 * 32) * per;
            } else {
                o_sub = static_cast<float*>(out) + mt0 * 32 * ldo + nt0 * 32;
            }
            const hipError_t e = launch_dense_cfg<FMT, WN, WM, RT, CT>(g, Mc, Nc, o, o_sub, s);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <mmq_wtype FMT>
hipError_t launch_dense(const void* packed, const void* act, int64_t M, int64_t N, int64_t K,
                        mmq_otype o, void* out, int64_t ldo, hipStream_t s) {
    BlockArgs g = dense_args<FMT>(packed, act, M, N, K);
    g.ldo = ldo;
    const int64_t scale_off = g.w_scale_off, min_off = g.w_min_off;
    if (ceil_div(N, WN_ * RT_ * 32) * ceil_div(M, WM_ * CT_ * 32) >= DENSE_FILL)
        return launch_dense_split<FMT, WN_, WM_, RT_, CT_>(g, M, N, o, out, ldo, scale_off, min_off, s);
    return launch_dense_split<FMT, GWN_, GWM_, GRT_, DCT_>(g, M, N, o, out, ldo, scale_off, min_off, s);
}

template <mmq_wtype FMT>
hipError_t launch_gather(const void* packed, int64_t E, const void* act, int64_t T, int64_t top_k,
                         int64_t N, int64_t K, const int32_t* offs, const int32_t* ufull,
                         const int32_t* utail, const int32_t* pairs, int max_full, int max_tail,
                         void* out, hipStream_t s) {
    BlockArgs g = dense_args<FMT>(packed, act, T, N, K);
    g.w_stride = (int64_t)packed_layout(FMT, N, K).bytes;
    g.offs = offs;
    g.ufull = ufull;
    g.pairs = pairs;
    g.E = (int)E;
    g.top_k = (int)top_k;
    constexpr int GRT = gather_rt<FMT>();
    g.ntiles_n = (int)ceil_div(N, GWN_ * GRT * 32);
    g.unit_rows = UNIT_ROWS;
    g.out = static_cast<float*>(out);
    g.ldo = N;
    const dim3 block(GWN_ * GWM_ * 64);
    BlockArgs t = g;
    g.uoff = ufull;
    t.uoff = utail;
    const int nfull = (int)(round_up(max_full, 8) * g.ntiles_n);
    const int ntail = (int)(round_up(max_tail, 8) * g.ntiles_n);
    hipLaunchKernelGGL((mmq_gather_kernel<FMT, GWN_, GWM_, GRT, GCT_, TCT_, XM_>), dim3((unsigned)(nfull + ntail)),
                       block, 0, s, g, t, nfull);
    return hipGetLastError();
}

}  // namespace

// Pairs per full MUL_MAT_ID unit (one full-unit workgroup's token extent), and the largest
// remainder that goes to a tail unit.
int gather_unit_tokens() { return UNIT_ROWS; }
int gather_tail_tokens() { return TAIL_ROWS; }

// A grid stays below 2^32 work-items: 2^24 workgroups of 256 threads.
constexpr int64_t MAX_GRID = (int64_t(1) << 24) - 1;

// the one MUL_MAT_ID launch holds the full-unit grid and the tail grid (at most as many units);
// counted at 128 weight rows per unit, an upper bound of every format's grid
bool gather_grid_ok(int64_t max_units, int64_t N) {
    return 2 * round_up(max_units, 8) * ceil_div(N, GWN_ * GRT_ * 32) <= MAX_GRID;
}

// The gather kernel addresses one expert's packed matrix and the T token rows with 32-bit
// offsets from each region's base (it is not split into several launches: the unit list lives
// on the device), so every such region must stay below 2 GiB.
bool gather_regions_ok(mmq_wtype t, int64_t T, int64_t N, int64_t K) {
    const PackedLayout P = packed_layout(t, N, K);
    const ActQ81Layout A = act_q8_1_layout(T, K);
    return P.NT * P.KBp * P.frag_bytes < MAX_REGION && P.Np * P.KBp * 4 < MAX_REGION &&
           A.MT * A.KBp * 1024 < MAX_REGION && A.Mp * A.KBp * 4 < MAX_REGION;
}

hipError_t launch_block_gemm(mmq_wtype t, const void* packed, const void* act, int64_t M, int64_t N,
                             int64_t K, mmq_otype o, void* out, int64_t ldo, hipStream_t s) {
    switch (t) {
        case MMQ_Q8_0: return launch_dense<MMQ_Q8_0>(packed, act, M, N, K, o, out, ldo, s);
        case MMQ_Q4_0: return launch_dense<MMQ_Q4_0>(packed, act, M, N, K, o, out, ldo, s);
        case MMQ_Q4_K: return launch_dense<MMQ_Q4_K>(packed, act, M, N, K, o, out, ldo, s);
        case MMQ_IQ1T: return launch_dense<MMQ_IQ1T>(packed, act, M, N, K, o, out, ldo, s);
        case MMQ_IQ1C: return launch_dense<MMQ_IQ1C>(packed, act, M, N, K, o, out, ldo, s);
        case MMQ_Q6_K: return launch_dense<MMQ_Q6_K>(packed, act, M, N, K, o, out, ldo, s);
        default: return hipErrorNotSupported;
    }
}

hipError_t launch_block_gather(mmq_wtype t, const void* packed, int64_t E, const void* act, int64_t T,
                               int64_t top_k, int64_t N, int64_t K, const int32_t* offs,
                               const int32_t* ufull, const int32_t* utail, const int32_t* pairs,
                               int max_full, int max_tail, void* out, hipStream_t s) {
#define MMQ_GATHER(F) launch_gather<F>(packed, E, act, T, top_k, N, K, offs, ufull, utail, pairs, max_full, max_tail, out, s)
    switch (t) {
        case MMQ_Q8_0: return MMQ_GATHER(MMQ_Q8_0);
        case MMQ_Q4_0: return MMQ_GATHER(MMQ_Q4_0);
        case MMQ_Q4_K: return MMQ_GATHER(MMQ_Q4_K);
        case MMQ_IQ1T: return MMQ_GATHER(MMQ_IQ1T);
        case MMQ_IQ1C: return MMQ_GATHER(MMQ_IQ1C);
        case MMQ_Q6_K: return MMQ_GATHER(MMQ_Q6_K);
        default: return hipErrorNotSupported;
    }
#undef MMQ_GATHER
}

}  // namespace mmq
