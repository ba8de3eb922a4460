// gemm_block.hip - the MMQ contraction for the block-quantised weight formats on CDNA4.
//
//   out[m,n] = sum_b (xs[m,b] * wd[n,b]) * P[m,n,b],   P = sum_{k in b} xq[m,k] * wq[n,k]
//
// ("A Negative Result on int8 Tensor-Core MMQ", section 2; minfer "08 . R1", sections 2.1-2.2.)
//
// Per 32-value block and 32x32 output tile, v_mfma_i32_32x32x32_i8 computes the exact int32
// block dots P (K = 32 is exactly one block, so no two scales ever share an accumulator). The
// block scale is an outer product of a weight-row vector and a token vector; a second MFMA on
// the same 32x32 lane map forms it exactly, and the correction acc += f32(P) * s is applied in
// registers - no store -> sync -> reload of the accumulator per block (the pages' "wall",
// Hanzo paper sections 2-3; the fix is a manual MMA with a known lane map, section 4).
//   q8_0, q4_0, iq1t: scale operands are f16 (d and xs are f16 values); each lane's operand
//     holds its row's value in slot 0 and zeros elsewhere, so v_mfma_f32_32x32x16_f16 returns
//     exactly 2*wd*xs (k = 0 and k = 8, one per half-wave; a product of two f16 is exact in f32).
//   q4_K: d*sc and dmin*m are exact f32 but not f16, so v_mfma_f32_32x32x2_f32 forms
//     2*(d*sc)*xs, and a second one adds the rank-1 min term 2*(-dmin*m)*(xs*xsum) straight into
//     the accumulator through its C operand (minfer R1 section 2.2: sum w*q = ds*sum nib*q -
//     dmin*sum q, with the activation block sum produced by the quantiser).
//   iq1t: the IQ1_M fold (llama.cpp PR #304) turns each value into the integer 8g +- 1 with a
//     per-16 factor (2s+1) and a per-block scale d/8. (2s+1)*v = 2s*v + v with |2s*v| <= 126,
//     so two chained int8 MFMAs over [2s*v] and [v] (same token operand) give the folded
//     per-32 integer sum_h (2s_h+1)*P16_h exactly, and only d remains as a scale.
//
// Operands stream through LDS with register staging: the next stage's global loads are issued
// before the current stage's MFMA sequence and written to the other LDS buffer after it
// (minfer R1 section 2.3: exposed staging latency was the largest single cost; metainfer
// section 1: global loads of stage i+1 before the stage-i MMAs, wait, write, barrier).
//
// Inside a stage the tiles are software-pipelined: the MFMAs of tile t+1 are issued into a
// second register set before the VALU correction of tile t, so the matrix core works while
// the vector unit converts and rescales (per 32x32 tile and block: one int8 MFMA and one
// scale MFMA against 16 cvt + 16 fma per lane, i.e. the VALU side is the longer one).
//
// The same kernel serves MUL_MAT_ID: in gather mode every token slot of a tile reads its own
// activation row and writes its own output row (see gemm_id.hip).
#include <type_traits>

#include "gemm_common.h"

namespace mmq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------- weight formats
template <mmq_wtype FMT> struct BT;

template <> struct BT<MMQ_Q8_0> {
    static constexpr int FB = 1024;        // packed fragment bytes per (tile, block)
    static constexpr int NMF = 1;          // int8 MFMAs per block
    static constexpr int SB = 2;           // packed scale bytes per (tile, block, row)
    static constexpr bool F32S = false;    // f32 (q4_K) or replicated f16 scale operands
    static constexpr int SHIFT = 0;        // the MFMA computes P << SHIFT
    static constexpr float POST = 1.0f / 2;     // scale operand 2*wd*xs
    __device__ static void operands(const uint8_t* frag, int lane, const uint8_t*, v4i* a) {
        a[0] = *reinterpret_cast<const v4i*>(frag + lane * 16);
    }
};

// q4_0 lane bytes: high nibbles of X0 are k = 16h+0..3, low nibbles 16h+4..7 (X1: 8..15), each
// the 4-bit two's complement of nib - 8; masking (after a shift for the low ones) yields int8
// 16*(nib-8).
template <> struct BT<MMQ_Q4_0> {
    static constexpr int FB = 512;
    static constexpr int NMF = 1;
    static constexpr int SB = 2;
    static constexpr bool F32S = false;
    static constexpr int SHIFT = 4;
    static constexpr float POST = 1.0f / 32;    // 16x block dot, 2*wd*xs
    __device__ static void operands(const uint8_t* frag, int lane, const uint8_t*, v4i* a) {
        const uint2 X = *reinterpret_cast<const uint2*>(frag + lane * 8);
        a[0][0] = (int)(X.x & 0xF0F0F0F0u);
        a[0][1] = (int)((X.x << 4) & 0xF0F0F0F0u);
        a[0][2] = (int)(X.y & 0xF0F0F0F0u);
        a[0][3] = (int)((X.y << 4) & 0xF0F0F0F0u);
    }
};

// q4_K lane bytes: unsigned nibbles, X0 & 0x0F0F0F0F = k 16h+0..3, (X0 >> 4) & .. = 16h+4..7.
template <> struct BT<MMQ_Q4_K> {
    static constexpr int FB = 512;
    static constexpr int NMF = 1;
    static constexpr int SB = 8;           // f32 d*sc, f32 -dmin*m
    static constexpr bool F32S = true;
    static constexpr int SHIFT = 0;
    static constexpr float POST = 1.0f / 2;
    __device__ static void operands(const uint8_t* frag, int lane, const uint8_t*, v4i* a) {
        const uint2 X = *reinterpret_cast<const uint2*>(frag + lane * 8);
        a[0][0] = (int)(X.x & 0x0F0F0F0Fu);
        a[0][1] = (int)((X.x >> 4) & 0x0F0F0F0Fu);
        a[0][2] = (int)(X.y & 0x0F0F0F0Fu);
        a[0][3] = (int)((X.y >> 4) & 0x0F0F0F0Fu);
    }
};

// iq1t lane data: one dword of 2-bit codes (value 4q+b at bits 8b+2q) and a meta byte
// s | sigma0 << 3 | sigma1 << 4 (sigma_i: sign bit of the lane's 8-value group i). The table
// entry for a meta byte holds four byte-LUTs indexed by the code: v = 8(c-1) + sigma for both
// sign groups, and 2s*v for both. v_perm picks the bytes: selectors 0..2 address the first
// group's LUT, 4..6 the second's.
template <> struct BT<MMQ_IQ1T> {
    static constexpr int FB = 320;         // 64 lanes x 4 B codes + 64 meta bytes
    static constexpr int NMF = 2;
    static constexpr int SB = 2;
    static constexpr bool F32S = false;
    static constexpr int SHIFT = 0;
    static constexpr float POST = 1.0f / 16;    // scale d/8, operand 2*d*xs
    __device__ static void operands(const uint8_t* frag, int lane, const uint8_t* tab, v4i* a) {
        const uint32_t C = *reinterpret_cast<const uint32_t*>(frag + lane * 4);
        const uint32_t meta = frag[256 + lane];
        const v4i t = *reinterpret_cast<const v4i*>(tab + meta * 16);   // v0, v1, 2s*v0, 2s*v1
        const uint32_t s0 = C & 0x03030303u;
        const uint32_t s1 = (C >> 2) & 0x03030303u;
        const uint32_t s2 = ((C >> 4) & 0x03030303u) | 0x04040404u;
        const uint32_t s3 = ((C >> 6) & 0x03030303u) | 0x04040404u;
        a[0][0] = (int)__builtin_amdgcn_perm((uint32_t)t[3], (uint32_t)t[2], s0);
        a[0][1] = (int)__builtin_amdgcn_perm((uint32_t)t[3], (uint32_t)t[2], s1);
        a[0][2] = (int)__builtin_amdgcn_perm((uint32_t)t[3], (uint32_t)t[2], s2);
        a[0][3] = (int)__builtin_amdgcn_perm((uint32_t)t[3], (uint32_t)t[2], s3);
        a[1][0] = (int)__builtin_amdgcn_perm((uint32_t)t[1], (uint32_t)t[0], s0);
        a[1][1] = (int)__builtin_amdgcn_perm((uint32_t)t[1], (uint32_t)t[0], s1);
        a[1][2] = (int)__builtin_amdgcn_perm((uint32_t)t[1], (uint32_t)t[0], s2);
        a[1][3] = (int)__builtin_amdgcn_perm((uint32_t)t[1], (uint32_t)t[0], s3);
    }
    // table entry e (meta byte) word w: w=0,1: LUT of v for sign group 0/1; w=2,3: LUT of 2s*v
    __device__ static uint32_t table_word(int e, int w) {
        const int s = e & 7;
        const int sig = ((w & 1) ? (e >> 4) : (e >> 3)) & 1;
        const int d = sig ? -1 : 1;
        const int mul = (w >= 2) ? 2 * s : 1;
        const int b0 = (-8 + d) * mul, b1 = d * mul, b2 = (8 + d) * mul;
        return (uint32_t)(b0 & 0xFF) | ((uint32_t)(b1 & 0xFF) << 8) | ((uint32_t)(b2 & 0xFF) << 16);
    }
};

// ------------------------------------------------------------------- kernel configuration
enum Mode { DENSE_F32 = 0, DENSE_PARTIALS = 1, GATHER_F32 = 2 };

template <mmq_wtype FMT, int WN, int WM, int RT, int CT, int KS>
struct Cfg {
    using T = BT<FMT>;
    static constexpr int NW = WN * WM, NTH = NW * 64;
    static constexpr int TN = WN * RT;                    // weight tiles per CTA
    static constexpr int TM = WM * CT;                    // token tiles per CTA
    static constexpr int WF = TN * KS * T::FB;            // LDS: weight fragments
    static constexpr int XF = TM * KS * 1024;             // LDS: token fragments
    // scale operands: one f16 per row (2 B) or an f32 pair (8 B per row)
    static constexpr int ROWB = T::F32S ? 8 : 2;
    static constexpr int WS = TN * KS * 32 * ROWB;
    static constexpr int XS = TM * KS * 32 * ROWB;
    static constexpr int BUF = WF + XF + WS + XS;
    static constexpr int UW = WF / 16;                    // 16-byte weight units per stage
    static constexpr int UX = TM * KS * 64;               // 16-byte token units per stage
    static constexpr int UPT_W = (UW + NTH - 1) / NTH;
    static constexpr int UPT_X = (UX + NTH - 1) / NTH;
    static constexpr int SI = (TN + TM) * KS * 32;        // scale items (rows) per stage
    static constexpr int SPT = (SI + NTH - 1) / NTH;
    static_assert(WF % 16 == 0, "fragment stage must be whole 16-byte units");
};

struct BlockArgs {
    const uint8_t* w;           // packed weights (expert 0 in gather mode)
    int64_t w_scale_off;        // offset of the scale region inside one packed matrix
    int64_t w_stride;           // bytes between experts' packed matrices (gather mode)
    const uint8_t* xq;          // act region 0 (tiled int8)
    const float* xs;            // act region 1
    const int32_t* xsum;        // act region 2
    const uint16_t* xs16;       // act region 3 (f16 xs)
    int M, N, KB, KBp, NT, MT, tiles_m;
    float* out;
    int64_t ldo;
    int32_t* partials;
    // gather mode (MUL_MAT_ID)
    const int32_t* offs;        // [E+1] first pair of each expert in `pairs`
    const int32_t* uoff;        // [E+1] first unit of each expert; uoff[E] = live units
    const int32_t* pairs;       // pair ids in expert order (pair = token*top_k + slot)
    int E, top_k, ntiles_n;
};

template <mmq_wtype FMT, int WN, int WM, int RT, int CT, int KS, int MODE>
__global__ __launch_bounds__(WN * WM * 64, 2) void mmq_block_kernel(BlockArgs args) {
    using C = Cfg<FMT, WN, WM, RT, CT, KS>;
    using T = typename C::T;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][C::BUF];
    __shared__ __attribute__((aligned(16))) uint8_t tab[FMT == MMQ_IQ1T ? 512 : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wm = wave / WN;

    // ---- which tile: dense grids are XCD-swizzled over (n-tile, m-tile); gather grids are
    // (unit, n-tile) with the unit list produced on the device
    int nt_base, mt_base = 0, unit_first = 0, unit_count = 0;
    const uint8_t* wbase = args.w;
    if constexpr (MODE == GATHER_F32) {
        // workgroup b runs on XCD b % 8; unit u = 8 * (rest / ntiles_n) + b % 8 keeps all weight
        // tiles of a unit (which share its activation rows) on one XCD and spreads the live
        // units (the lowest ids) evenly over the XCDs
        const int b = blockIdx.x, rest = b >> 3;
        const int u = (rest / args.ntiles_n) * 8 + (b & 7);
        if (u >= args.uoff[args.E]) return;             // uniform: the whole CTA leaves
        int lo = 0, hi = args.E;                        // largest e with uoff[e] <= u
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (args.uoff[mid] <= u) lo = mid; else hi = mid;
        }
        const int e = lo;
        unit_first = args.offs[e] + (u - args.uoff[e]) * (C::TM * 32);
        unit_count = min(C::TM * 32, args.offs[e + 1] - unit_first);
        wbase = args.w + (int64_t)e * args.w_stride;
        nt_base = (rest % args.ntiles_n) * C::TN;
    } else {
        const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
        nt_base = (lid / args.tiles_m) * C::TN;
        mt_base = (lid % args.tiles_m) * C::TM;
    }
    const uint8_t* wfrag = wbase;
    const uint8_t* wscale = wbase + args.w_scale_off;
    const int NT = args.NT, KBp = args.KBp;

    // token slot (tile j, row r) -> activation row to read
    auto src_token = [&](int j, int r) -> int {
        if constexpr (MODE == GATHER_F32) {
            const int s = j * 32 + r;
            return s < unit_count ? args.pairs[unit_first + s] / args.top_k : 0;
        } else {
            return min((mt_base + j) * 32 + r, args.MT * 32 - 1);
        }
    };

    if constexpr (FMT == MMQ_IQ1T) {
        if (tid < 128) reinterpret_cast<uint32_t*>(tab)[tid] = T::table_word(tid >> 2, tid & 3);
    }

    // ---- copy plan: per-thread source pointers, advanced by a fixed stride every stage
    const uint8_t* wsrc[C::UPT_W];
    int wdst[C::UPT_W];
#pragma unroll
    for (int i = 0; i < C::UPT_W; ++i) {
        const int u = min(tid + i * C::NTH, C::UW - 1);
        constexpr int per = KS * T::FB / 16;               // units per tile per stage
        const int nt = min(nt_base + u / per, NT - 1);
        wsrc[i] = wfrag + (int64_t)nt * KBp * T::FB + (u % per) * 16;
        wdst[i] = (tid + i * C::NTH < C::UW) ? u * 16 : -1;
    }
    const uint8_t* xsrc[C::UPT_X];
    int xdst[C::UPT_X];
#pragma unroll
    for (int i = 0; i < C::UPT_X; ++i) {
        const int u = min(tid + i * C::NTH, C::UX - 1);
        const int L = u & 63, q = (u >> 6) % KS, j = (u >> 6) / KS;
        const int t = src_token(j, L & 31);
        xsrc[i] = args.xq + ((int64_t)(t >> 5) * KBp + q) * 1024 + ((L >> 5) * 32 + (t & 31)) * 16;
        xdst[i] = (tid + i * C::NTH < C::UX) ? C::WF + (j * KS + q) * 1024 + L * 16 : -1;
    }
    // scale items: (side, tile, block-in-stage, row)
    const uint8_t* ssrc[C::SPT];
    const uint8_t* ssrc2[C::SPT];
    int sdst[C::SPT];
    bool sw_[C::SPT];
#pragma unroll
    for (int i = 0; i < C::SPT; ++i) {
        const int it = min(tid + i * C::NTH, C::SI - 1);
        const int r = it & 31, q = (it >> 5) % KS, tile = (it >> 5) / KS;
        const bool wside = tile < C::TN;
        sw_[i] = wside;
        if (wside) {
            const int nt = min(nt_base + tile, NT - 1);
            ssrc[i] = wscale + (((int64_t)nt * KBp + q) * 32 + r) * T::SB;
            ssrc2[i] = ssrc[i];
            // f16: one 16-byte entry per row; f32: a (64-float) pair of 32-float arrays per
            // (tile, block), value at [r] and partner at [32 + r]
            sdst[i] = C::WF + C::XF + (T::F32S ? ((tile * KS + q) * 64 + r) * 4 : ((tile * KS + q) * 32 + r) * 2);
        } else {
            const int j = tile - C::TN;
            const int t = src_token(j, r);
            const int64_t idx = ((int64_t)(t >> 5) * KBp + q) * 32 + (t & 31);
            ssrc[i] = T::F32S ? reinterpret_cast<const uint8_t*>(args.xs + idx)
                              : reinterpret_cast<const uint8_t*>(args.xs16 + idx);
            ssrc2[i] = reinterpret_cast<const uint8_t*>(args.xsum + idx);
            sdst[i] = C::WF + C::XF + C::WS + (T::F32S ? ((j * KS + q) * 64 + r) * 4 : ((j * KS + q) * 32 + r) * 2);
        }
        if (tid + i * C::NTH >= C::SI) sdst[i] = -1;
    }
    // per-stage advance of the scale sources (bytes)
    constexpr int WSTEP = KS * 32 * T::SB;
    constexpr int XSTEP = KS * 32 * (T::F32S ? 4 : 2);

    v4i wreg[C::UPT_W], xreg[C::UPT_X];
    uint32_t sreg[C::SPT], sreg2[C::SPT];
    auto load_stage = [&]() {
#pragma unroll
        for (int i = 0; i < C::UPT_W; ++i) {
            wreg[i] = *reinterpret_cast<const v4i*>(wsrc[i]);
            wsrc[i] += KS * T::FB;
        }
#pragma unroll
        for (int i = 0; i < C::UPT_X; ++i) {
            xreg[i] = *reinterpret_cast<const v4i*>(xsrc[i]);
            xsrc[i] += KS * 1024;
        }
#pragma unroll
        for (int i = 0; i < C::SPT; ++i) {
            if constexpr (T::F32S) {
                if (sw_[i]) {
                    const uint2 v = *reinterpret_cast<const uint2*>(ssrc[i]);
                    sreg[i] = v.x;
                    sreg2[i] = v.y;
                } else {
                    sreg[i] = *reinterpret_cast<const uint32_t*>(ssrc[i]);
                    sreg2[i] = *reinterpret_cast<const uint32_t*>(ssrc2[i]);
                    ssrc2[i] += XSTEP;
                }
            } else {
                sreg[i] = *reinterpret_cast<const uint16_t*>(ssrc[i]);
            }
            ssrc[i] += sw_[i] ? WSTEP : XSTEP;
        }
    };
    auto store_stage = [&](uint8_t* buf) {
#pragma unroll
        for (int i = 0; i < C::UPT_W; ++i)
            if (C::UW % C::NTH == 0 || wdst[i] >= 0) *reinterpret_cast<v4i*>(buf + wdst[i]) = wreg[i];
#pragma unroll
        for (int i = 0; i < C::UPT_X; ++i)
            if (C::UX % C::NTH == 0 || xdst[i] >= 0) *reinterpret_cast<v4i*>(buf + xdst[i]) = xreg[i];
#pragma unroll
        for (int i = 0; i < C::SPT; ++i) {
            if (C::SI % C::NTH == 0 || sdst[i] >= 0) {
                if constexpr (T::F32S) {
                    // weights: d*sc, -dmin*m; tokens: xs, xs*xsum (exact in f32)
                    float* d = reinterpret_cast<float*>(buf + sdst[i]);
                    const float a = __builtin_bit_cast(float, sreg[i]);
                    const float b = sw_[i] ? __builtin_bit_cast(float, sreg2[i])
                                           : a * (float)(int32_t)sreg2[i];
                    d[0] = a;
                    d[32] = b;
                } else {
                    *reinterpret_cast<uint16_t*>(buf + sdst[i]) = (uint16_t)sreg[i];
                }
            }
        }
    };

    v16f acc[RT][CT];
#pragma unroll
    for (int x = 0; x < RT; ++x)
#pragma unroll
        for (int y = 0; y < CT; ++y)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

    const v16i zi = {0};
    const v16f zf = {0};
    const int nstages = KBp / KS;

    // one block's operands for this wave: weight fragments, token fragments, scale operands
    struct Ops {
        v4i a[RT][T::NMF];
        v4i b[CT];
        h8 wsv[RT], xsv[CT];            // f16 scale operands (slot 0 live)
        float wsf[RT], wmf[RT], xsf[CT], sxf[CT];   // Q4_K: d*sc, -dmin*m, xs, xs*xsum
    };
    auto load_w = [&](const uint8_t* cur, int kb, int rt, Ops& o) {
        const int i = wn * RT + rt;
        T::operands(cur + (i * KS + kb) * T::FB, lane, tab, o.a[rt]);
        const uint8_t* wsl = cur + C::WF + C::XF;
        if constexpr (T::F32S) {
            const float* p = reinterpret_cast<const float*>(wsl) + (i * KS + kb) * 64 + (lane & 31);
            o.wsf[rt] = p[0];
            o.wmf[rt] = p[32];
        } else {
            const uint16_t v = *reinterpret_cast<const uint16_t*>(wsl + ((i * KS + kb) * 32 + (lane & 31)) * 2);
            v4i t4 = {(int)v, 0, 0, 0};
            o.wsv[rt] = __builtin_bit_cast(h8, t4);
        }
    };
    auto load_x = [&](const uint8_t* cur, int kb, int ct, Ops& o) {
        const int j = wm * CT + ct;
        o.b[ct] = *reinterpret_cast<const v4i*>(cur + C::WF + (j * KS + kb) * 1024 + lane * 16);
        const uint8_t* xsl = cur + C::WF + C::XF + C::WS;
        if constexpr (T::F32S) {
            const float* p = reinterpret_cast<const float*>(xsl) + (j * KS + kb) * 64 + (lane & 31);
            o.xsf[ct] = p[0];
            o.sxf[ct] = p[32];
        } else {
            const uint16_t v = *reinterpret_cast<const uint16_t*>(xsl + ((j * KS + kb) * 32 + (lane & 31)) * 2);
            v4i t4 = {(int)v, 0, 0, 0};
            o.xsv[ct] = __builtin_bit_cast(h8, t4);
        }
    };
    // matrix-core half of one (tile, block): exact int32 dots D, scale outer product S, and
    // for Q4_K the rank-1 min term added into the accumulator through the C operand
    auto issue = [&](const Ops& o, int t, v16i& D, v16f& S) {
        const int rt = t / CT, ct = t % CT;
        D = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[rt][0], o.b[ct], zi, 0, 0, 0);
        if constexpr (T::NMF == 2) D = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[rt][1], o.b[ct], D, 0, 0, 0);
        if constexpr (MODE != DENSE_PARTIALS) {
            if constexpr (T::F32S) {
                S = __builtin_amdgcn_mfma_f32_32x32x2f32(o.wsf[rt], o.xsf[ct], zf, 0, 0, 0);
                acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(o.wmf[rt], o.sxf[ct], acc[rt][ct], 0, 0, 0);
            } else {
                S = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.wsv[rt], o.xsv[ct], zf, 0, 0, 0);
            }
        }
    };
    // vector half: acc += f32(D) * S (or the partials store)
    auto finish = [&](int s, int kb, int t, const v16i& D, const v16f& S) {
        const int rt = t / CT, ct = t % CT;
        if constexpr (MODE == DENSE_PARTIALS) {
            const int kbg = s * KS + kb;
            const int m = (mt_base + wm * CT + ct) * 32 + (lane & 31);
            if (kbg < args.KB && m < args.M) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = (nt_base + wn * RT + rt) * 32 + acc_row(lane, r);
                    if (n < args.N) args.partials[((int64_t)m * args.N + n) * args.KB + kbg] = D[r] >> T::SHIFT;
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rt][ct][r] = __builtin_fmaf((float)D[r], S[r], acc[rt][ct][r]);
        }
    };

    // Tile t of a block is (rt, ct) = (t / CT, t % CT). Step t issues tile t+1 (or tile 0 of
    // the next block) and then finishes tile t. Right after the issue of the last tile that
    // reads an operand (a[rt]: tile rt*CT + CT-1; b[ct]: tile (RT-1)*CT + ct), that operand is
    // reloaded for the next block, so one register set serves and every LDS read has at least
    // two steps of VALU work to land before its next use.
    constexpr int NT_ = RT * CT;
    // One stage: its KS blocks through the tile pipeline. `last` is a compile-time flag so the
    // steady-state loop body has no branches (a branch lets the compiler sink the VALU half of
    // the pipeline past it).
    auto run_stage = [&](int s, auto last_tag) {
        constexpr bool LAST = decltype(last_tag)::value;
        const uint8_t* cur = lds[s & 1];
        if constexpr (!LAST) load_stage();              // in flight during this stage's MFMAs
        Ops op;
        v16i D[2];
        v16f S[2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) load_w(cur, 0, rt, op);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) load_x(cur, 0, ct, op);
        issue(op, 0, D[0], S[0]);
#pragma unroll
        for (int kb = 0; kb < KS; ++kb) {
#pragma unroll
            for (int t = 0; t < NT_; ++t) {
                const int i = kb * NT_ + t;
                if (t + 1 < NT_ || kb + 1 < KS) issue(op, (t + 1) % NT_, D[(i + 1) & 1], S[(i + 1) & 1]);
                if (kb + 1 < KS) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        if (t == (rt * CT + CT - 2 > 0 ? rt * CT + CT - 2 : 0)) load_w(cur, kb + 1, rt, op);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        if (t == ((RT - 1) * CT + ct - 1 > 0 ? (RT - 1) * CT + ct - 1 : 0)) load_x(cur, kb + 1, ct, op);
                }
                // keep the next tile's MFMAs ahead of this tile's VALU work
                __builtin_amdgcn_sched_barrier(0);
                finish(s, kb, t, D[i & 1], S[i & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (!LAST) store_stage(lds[(s + 1) & 1]);
        __syncthreads();
    };

    load_stage();
    store_stage(lds[0]);
    __syncthreads();
    for (int s = 0; s + 1 < nstages; ++s) run_stage(s, std::false_type{});
    run_stage(nstages - 1, std::true_type{});

    if constexpr (MODE != DENSE_PARTIALS) {
        const int64_t ldo = args.ldo;
        const bool vec_ok = (ldo & 3) == 0;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            int row;
            if constexpr (MODE == GATHER_F32) {
                const int sl = (wm * CT + ct) * 32 + (lane & 31);
                row = sl < unit_count ? args.pairs[unit_first + sl] : -1;
            } else {
                const int m = (mt_base + wm * CT + ct) * 32 + (lane & 31);
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

// Tile configuration: 2 x 2 waves, each owning 2 weight tiles x 2 token tiles -> 128 x 128
// CTA tiles, 2 blocks per stage.
constexpr int WN_ = 2, WM_ = 2, RT_ = 2, CT_ = 2, KS_ = 2;

template <mmq_wtype FMT>
BlockArgs dense_args(const void* packed, const void* act, int64_t M, int64_t N, int64_t K) {
    const PackedLayout P = packed_layout(FMT, N, K);
    const ActQ81Layout A = act_q8_1_layout(M, K);
    const uint8_t* ab = static_cast<const uint8_t*>(act);
    BlockArgs g{};
    g.w = static_cast<const uint8_t*>(packed) + P.frag_off;
    g.w_scale_off = P.scale_off - P.frag_off;
    g.w_stride = 0;
    g.xq = ab + A.xq_off;
    g.xs = reinterpret_cast<const float*>(ab + A.xs_off);
    g.xsum = reinterpret_cast<const int32_t*>(ab + A.xsum_off);
    g.xs16 = reinterpret_cast<const uint16_t*>(ab + A.xs16_off);
    g.M = (int)M;
    g.N = (int)N;
    g.KB = (int)A.KB;
    g.KBp = (int)A.KBp;
    g.NT = (int)P.NT;
    g.MT = (int)A.MT;
    return g;
}

template <mmq_wtype FMT>
hipError_t launch_dense(const void* packed, const void* act, int64_t M, int64_t N, int64_t K,
                        mmq_otype o, void* out, int64_t ldo, hipStream_t s) {
    BlockArgs g = dense_args<FMT>(packed, act, M, N, K);
    const int tiles_n = (int)ceil_div(N, WN_ * RT_ * 32);
    const int tiles_m = (int)ceil_div(M, WM_ * CT_ * 32);
    g.tiles_m = tiles_m;
    g.ldo = ldo;
    const dim3 grid((unsigned)((int64_t)tiles_n * tiles_m)), block(WN_ * WM_ * 64);
    if (o == MMQ_OUT_I32_PARTIALS) {
        g.partials = static_cast<int32_t*>(out);
        hipLaunchKernelGGL((mmq_block_kernel<FMT, WN_, WM_, RT_, CT_, KS_, DENSE_PARTIALS>), grid, block, 0, s, g);
    } else {
        g.out = static_cast<float*>(out);
        hipLaunchKernelGGL((mmq_block_kernel<FMT, WN_, WM_, RT_, CT_, KS_, DENSE_F32>), grid, block, 0, s, g);
    }
    return hipGetLastError();
}

template <mmq_wtype FMT>
hipError_t launch_gather(const void* packed, int64_t E, const void* act, int64_t T, int64_t top_k,
                         int64_t N, int64_t K, const int32_t* offs, const int32_t* uoff,
                         const int32_t* pairs, int max_units, void* out, hipStream_t s) {
    BlockArgs g = dense_args<FMT>(packed, act, T, N, K);
    g.w_stride = (int64_t)packed_layout(FMT, N, K).bytes;
    g.offs = offs;
    g.uoff = uoff;
    g.pairs = pairs;
    g.E = (int)E;
    g.top_k = (int)top_k;
    g.ntiles_n = (int)ceil_div(N, WN_ * RT_ * 32);
    g.out = static_cast<float*>(out);
    g.ldo = N;
    const int64_t nblk = round_up(max_units, 8) * g.ntiles_n;
    const dim3 grid((unsigned)nblk), block(WN_ * WM_ * 64);
    hipLaunchKernelGGL((mmq_block_kernel<FMT, WN_, WM_, RT_, CT_, KS_, GATHER_F32>), grid, block, 0, s, g);
    return hipGetLastError();
}

}  // namespace

// Tokens per MUL_MAT_ID unit (one CTA's token extent).
int gather_unit_tokens() { return WM_ * CT_ * 32; }

// One-dimensional grids stay below 2^31 workgroups.
constexpr int64_t MAX_GRID = int64_t(1) << 31;

bool dense_grid_ok(int64_t M, int64_t N) {
    return ceil_div(N, WN_ * RT_ * 32) * ceil_div(M, WM_ * CT_ * 32) < MAX_GRID;
}

bool gather_grid_ok(int64_t max_units, int64_t N) {
    return round_up(max_units, 8) * ceil_div(N, WN_ * RT_ * 32) < MAX_GRID;
}

hipError_t launch_block_gemm(mmq_wtype t, const void* packed, const void* act, int64_t M, int64_t N,
                             int64_t K, mmq_otype o, void* out, int64_t ldo, hipStream_t s) {
    switch (t) {
        case MMQ_Q8_0: return launch_dense<MMQ_Q8_0>(packed, act, M, N, K, o, out, ldo, s);
        case MMQ_Q4_0: return launch_dense<MMQ_Q4_0>(packed, act, M, N, K, o, out, ldo, s);
        case MMQ_Q4_K: return launch_dense<MMQ_Q4_K>(packed, act, M, N, K, o, out, ldo, s);
        case MMQ_IQ1T: return launch_dense<MMQ_IQ1T>(packed, act, M, N, K, o, out, ldo, s);
        default: return hipErrorNotSupported;
    }
}

hipError_t launch_block_gather(mmq_wtype t, const void* packed, int64_t E, const void* act, int64_t T,
                               int64_t top_k, int64_t N, int64_t K, const int32_t* offs,
                               const int32_t* uoff, const int32_t* pairs, int max_units, void* out,
                               hipStream_t s) {
    switch (t) {
        case MMQ_Q8_0: return launch_gather<MMQ_Q8_0>(packed, E, act, T, top_k, N, K, offs, uoff, pairs, max_units, out, s);
        case MMQ_Q4_0: return launch_gather<MMQ_Q4_0>(packed, E, act, T, top_k, N, K, offs, uoff, pairs, max_units, out, s);
        case MMQ_Q4_K: return launch_gather<MMQ_Q4_K>(packed, E, act, T, top_k, N, K, offs, uoff, pairs, max_units, out, s);
        case MMQ_IQ1T: return launch_gather<MMQ_IQ1T>(packed, E, act, T, top_k, N, K, offs, uoff, pairs, max_units, out, s);
        default: return hipErrorNotSupported;
    }
}

}  // namespace mmq
