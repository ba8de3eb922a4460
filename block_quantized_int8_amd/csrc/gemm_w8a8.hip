// gemm_w8a8.hip - per-channel W8A8 GEMM (int8 weights with an f32 scale per output channel,
// int8 activations with an f32 scale per token) on CDNA4 matrix cores.
//
// No per-block scale: the int32 accumulators run over all of K inside
// v_mfma_i32_32x32x32_i8 (C = D chaining; |acc| <= K * 128 * 128 < 2^31 for K < 131072) and the
// epilogue is bf16_rne((f32(acc) * sa[m]) * sw[n]) - two f32 multiplies in that order, no bias
// (metainfer "INT8 W8A8 GEMM - Prefill", section 1: fragment -> scale -> bf16).
//
// The int8 MFMA needs no vector work per block, so the kernel is bound by how fast operands
// reach the matrix core. Measured on gfx950: one v_mfma_i32_32x32x32_i8 issues every 32 cycles
// per wave; global->LDS DMA moves at most about 64 bytes per clock per CU (bound by the texture
// addresser, also for L2 hits), and about half that inside this kernel, where every CU of an
// XCD streams its panels through the shared L2 at once; a CU reads up to ~240 B/clk of LDS. A
// 7B tensor-parallel share (M = 3072, N = 1536) holds only 18 32x32 output tiles per CU, so
// each workgroup is one CU's share, 96 weight rows x 192 token rows. Its twelve waves split it
// as 6 token tiles x 2 halves of K (three waves per SIMD, each 3 weight tiles x 1 token tile);
// the two K halves are added in LDS before the epilogue. A CU then needs 2 x (96 + 192) x 32
// bytes = 18 KB of operands per 288 matrix-core cycles (9 MFMAs per SIMD), more than the DMA
// delivers, so the kernel's job is to keep the DMA busy and the matrix core fed:
//  - the DMA of each 2-block stage is spread evenly between the MFMAs (a vector-memory
//    instruction the texture unit cannot take yet stalls the wave's in-order issue, so a burst
//    of them would hold the matrix core idle), and three waves per SIMD cover each other's
//    stalls (12 waves measured 2.3% faster than 4 waves of 3 x 3 tiles);
//  - four LDS stage buffers: stage t's DMA is issued over the blocks of stages t-4 and t-3 and
//    waited for in the middle of stage t-1, about 2.5 stages later; the wait and the barrier
//    sit in the middle of a stage, so the next stage's first fragments are read before it
//    starts.
// (Same section: stage i+1 global loads before the stage-i MMACs.)
//
// Both operands are in the matrix core's fragment order, 1 KB per (32-row tile, block):
// weights from the repack, activations from the int8 quantiser (the same tiled layout as the
// q8_1 values), so every DMA reads 1 KB of whole cache lines (the DMA's rate is per cache line
// touched: 16 rows x 64 bytes per 1 KB runs at 2/3 of the contiguous rate). The bf16 result
// tile is staged in LDS and written as whole row segments.
#include <algorithm>

#include "gemm_common.h"

namespace mmq {
namespace {

typedef __attribute__((address_space(3))) void lmem_t;

// Workgroup barrier for the staging pipeline: LDS is the only memory shared through it, so it
// carries no fence (__syncthreads' release fence would also wait for every DMA in flight). The
// memory clobber keeps the compiler from moving memory operations across it.
__device__ inline void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt immediate: wait until at most n vector-memory operations are outstanding
constexpr int vm_wait(int n) { return 0x3f70 | (n & 15) | ((n >> 4) << 14); }

// One wave-wide buffer->LDS DMA of 16 bytes per lane: lane l's bytes at base + voff + soff land
// at lds + 16 l; voff is the lane's fixed offset, soff the wave-uniform stage offset (a scalar
// register, so advancing a stage costs no vector instruction).
__device__ inline void buf_dma16(const uint8_t* base, uint8_t* lds, uint32_t voff, int soff) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lmem_t*)lds, 16, (int)voff, soff, 0, 0);
}

constexpr int KS = 2;                  // blocks per stage: a token chunk row is 2 x 32 bytes
constexpr int NBUF = 4;                // LDS stage buffers

// RT weight tiles x CT token tiles per wave; WM waves along the tokens, KSP along K.
template <int RT, int CT, int WM, int KSP>
struct W8Cfg {
    static constexpr int NW = WM * KSP, NTH = NW * 64;
    static constexpr int TN = RT, TM = WM * CT;             // workgroup tile, in 32-row tiles
    static constexpr int NT_ = RT * CT;                      // MFMAs per block per wave
    static constexpr int C_W = RT * KS;                      // weight chunks per K part
    static constexpr int C_X = TM * KS;                      // token chunks per K part
    static constexpr int PART = (C_W + C_X) * 1024;          // LDS bytes per K part per stage
    static constexpr int BUF = KSP * PART;
    static constexpr int CW_ALL = KSP * C_W, C_ALL = KSP * (C_W + C_X);
    static constexpr int CPW = C_ALL / NW;                   // DMA chunks per wave per stage
    static constexpr int H0 = (CPW + 1) / 2;                 // ... of which a stage's block 1 issues
    static constexpr int XCH = NW * NT_ * 8 * 64 * 4;        // K-part exchange bytes
    static constexpr int OPITCH = TN * 64 + 16;              // bf16 output staging row pitch
    static_assert(CW_ALL % NW == 0 && C_ALL % NW == 0, "chunk kinds must split evenly over the waves");
    static_assert(KSP == 1 || KSP == 2, "K is split in at most two parts");
    static_assert(H0 <= NT_ && CPW - H0 <= NT_, "at most one DMA per MFMA");
    static_assert(XCH + TM * 32 * OPITCH <= NBUF * BUF, "the epilogue reuses the stage buffers");
};

struct W8Args {
    const uint8_t* wf;          // weight fragments [NT][KBp][1 KB]
    const float* sw;            // [Np]
    const uint8_t* a;           // token fragments [MT][KBp][1 KB]
    const float* sa;            // [M]
    int M, N, KBp, NT, MT, tiles_n, tiles_m;
    void* out;                  // bf16 [M][ldo] or int32 [M][ldo]
    int64_t ldo;
};

template <int RT, int CT, int WM, int KSP, bool PARTIALS>
__global__ __launch_bounds__(WM * KSP * 64, 1) void w8a8_kernel(W8Args g) {
    using C = W8Cfg<RT, CT, WM, KSP>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * C::BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, kp = wave / WM;
    const int r32 = lane & 31, h = lane >> 5;

    // Tile order: panels of 8 weight tiles x all token tiles, so that the 32 consecutive
    // logical tiles one XCD receives share 8 weight tiles and 4 token tiles.
    const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
    constexpr int GN = 8;
    const int per_panel = GN * g.tiles_m;
    const int panel = lid / per_panel, idx = lid % per_panel;
    const int width = min(GN, g.tiles_n - panel * GN);
    const int tn = panel * GN + idx % width, tm = idx / width;
    const int nt_base = tn * C::TN, m_base = tm * C::TM * 32;
    const int KBh = g.KBp / KSP;                              // blocks per K part
    const int nst = KBh / KS;                                 // stages per K part

    // ---- DMA plan. Chunk c = j * NW + wave: the first CW_ALL are weight chunks, the rest
    // token chunks, each (K part, tile, block) of a stage: one 1 KB fragment.
    uint32_t goff[C::CPW];      // byte offset of the lane's 16 bytes in stage 0
    int ldso[C::CPW];
    const int mt_base = tm * C::TM;
#pragma unroll
    for (int j = 0; j < C::CPW; ++j) {
        const int c = j * C::NW + wave;
        if (j * C::NW < C::CW_ALL) {
            const int p = c / C::C_W, i = (c % C::C_W) / KS, q = c % KS;
            const int nt = min(nt_base + i, g.NT - 1);
            goff[j] = (uint32_t)((nt * g.KBp + p * KBh + q) * 1024 + lane * 16);
            ldso[j] = p * C::PART + (i * KS + q) * 1024;
        } else {
            const int cx = c - C::CW_ALL;
            const int p = cx / C::C_X, i = (cx % C::C_X) / KS, q = cx % KS;
            const int mt = min(mt_base + i, g.MT - 1);
            goff[j] = (uint32_t)((mt * g.KBp + p * KBh + q) * 1024 + lane * 16);
            ldso[j] = p * C::PART + (C::C_W + i * KS + q) * 1024;
        }
    }
    // chunk j of stage t into stage buffer t % NBUF. Every stage issues the same instructions:
    // those of the stages past the end all read the first 16 bytes of the operand (one cached
    // line) into buffers nobody reads any more.
    auto issue_chunk = [&](int j, int t) __attribute__((always_inline)) {
        const uint8_t* base = j * C::NW < C::CW_ALL ? g.wf : g.a;
        const int soff = __builtin_amdgcn_readfirstlane(t < nst ? t * (KS * 1024) : 0);
        uint8_t* dst = smem + (t & (NBUF - 1)) * C::BUF + __builtin_amdgcn_readfirstlane(ldso[j]);
        buf_dma16(base, dst, goff[j], soff);
    };

    // fragment read offsets inside a stage buffer (lane * 16 inside each 1 KB fragment)
    const int woff = kp * C::PART + lane * 16;
    const int xoff = kp * C::PART + (C::C_W + wm * CT * KS) * 1024 + lane * 16;

    // epilogue operands, loaded now so their latency hides behind the main loop
    const int r_lo = KSP == 2 ? 8 * kp : 0;                  // accumulator registers this wave
    constexpr int NG = KSP == 2 ? 2 : 4;                      // finishes: r_lo .. r_lo + 4*NG - 1
    float sam[CT];
    float4 swv[RT][NG];
    if constexpr (!PARTIALS) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) sam[ct] = g.sa[min(m_base + (wm * CT + ct) * 32 + r32, g.M - 1)];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const int n0 = min(nt_base + rt, g.NT - 1) * 32 + 2 * r_lo + 8 * q + 4 * h;    // < Np
                swv[rt][q] = *reinterpret_cast<const float4*>(g.sw + n0);
            }
    }

    v16i acc[RT][CT];
#pragma unroll
    for (int x = 0; x < RT; ++x)
#pragma unroll
        for (int y = 0; y < CT; ++y) acc[x][y] = (v16i){0};

    struct Ops { v4i a[RT], b[CT]; };
    auto load_ops = [&](const uint8_t* buf, int kb, Ops& o) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            o.a[rt] = *reinterpret_cast<const v4i*>(buf + woff + (rt * KS + kb) * 1024);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
            o.b[ct] = *reinterpret_cast<const v4i*>(buf + xoff + (ct * KS + kb) * 1024);
    };
    // one block: the wave's RT x CT MFMAs, each followed by its share of the next block's
    // fragment reads (block nkb of `nbuf`) and of the DMA chunks of stage t (chunks j0..j1-1),
    // each step fenced so the scheduler keeps that order
    auto block = [&](const Ops& o, Ops& on, const uint8_t* nbuf, int nkb, int j0, int j1, int t)
        __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::NT_; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            const int rt = i / CT, ct = i % CT;
            acc[rt][ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[rt], o.b[ct], acc[rt][ct], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            // the RT + CT fragment reads spread evenly over the NT_ steps
            constexpr int F = RT + CT;
#pragma unroll
            for (int f = (i * F) / C::NT_; f < ((i + 1) * F) / C::NT_; ++f) {
                if (f < RT)
                    on.a[f] = *reinterpret_cast<const v4i*>(nbuf + woff + (f * KS + nkb) * 1024);
                else
                    on.b[f - RT] = *reinterpret_cast<const v4i*>(nbuf + xoff + ((f - RT) * KS + nkb) * 1024);
            }
            const int nd = j1 - j0;                          // DMAs spread evenly: one at the
            if ((i * nd) / C::NT_ != ((i + 1) * nd) / C::NT_)  // steps where i*nd/NT_ steps up
                issue_chunk(j0 + (i * nd) / C::NT_, t);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: stages 0-2 and the first part of stage 3 in flight, stage 0 landed.
#pragma unroll
    for (int j = 0; j < C::CPW; ++j) issue_chunk(j, 0);
#pragma unroll
    for (int j = 0; j < C::CPW; ++j) issue_chunk(j, 1);
#pragma unroll
    for (int j = 0; j < C::CPW; ++j) issue_chunk(j, 2);
#pragma unroll
    for (int j = 0; j < C::H0; ++j) issue_chunk(j, 3);
    __builtin_amdgcn_s_waitcnt(vm_wait(2 * C::CPW + C::H0));
    stage_barrier();
    Ops o0, o1;
    load_ops(smem, 0, o0);

    // Stage s: block 0 issues the rest of stage s+3's DMA; then the wait for stage s+1 (only
    // stages s+2 and s+3, 2 * CPW chunks, may still be in flight) and the barrier, after which
    // stage s-1's buffer is free; block 1 reads stage s+1's first fragments and issues the
    // first part of stage s+4's DMA into stage s's buffer, whose last reads were in block 0.
    for (int s = 0; s < nst; ++s) {
        const uint8_t* cur = smem + (s & (NBUF - 1)) * C::BUF;
        const uint8_t* nxt = smem + ((s + 1) & (NBUF - 1)) * C::BUF;
        block(o0, o1, cur, 1, C::H0, C::CPW, s + 3);
        __builtin_amdgcn_s_waitcnt(vm_wait(2 * C::CPW));
        stage_barrier();
        block(o1, o0, nxt, 0, 0, C::H0, s + 4);
    }
    __builtin_amdgcn_s_waitcnt(0x3f70);                      // no DMA outstanding past this point
    __syncthreads();

    // ---- K parts: each wave of a pair finishes half of every accumulator (registers
    // 8p..8p+7) and takes its partner's sum of that half through LDS, 16 bytes per lane per
    // access. fin[t][e] is the final value of register r_lo + e. Register indices stay
    // compile-time: the halves are picked with an opaque all-ones/zero mask (v_bfi), since a
    // plain select gets turned into a dynamically indexed register move.
    v16i fin[C::NT_];
    if constexpr (KSP == 2) {
        v4i* xch = reinterpret_cast<v4i*>(smem);
        const int hm = __builtin_amdgcn_readfirstlane(kp != 0 ? -1 : 0);
        auto pick = [&](int up, int lo) __attribute__((always_inline)) { return (up & hm) | (lo & ~hm); };
#pragma unroll
        for (int t = 0; t < C::NT_; ++t)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const v16i& A = acc[t / CT][t % CT];
                v4i gv;
#pragma unroll
                for (int e = 0; e < 4; ++e) gv[e] = pick(A[4 * q + e], A[8 + 4 * q + e]);
                xch[(((wm * 2 + kp) * C::NT_ + t) * 2 + q) * 64 + lane] = gv;
            }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < C::NT_; ++t)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const v4i v = xch[(((wm * 2 + (1 - kp)) * C::NT_ + t) * 2 + q) * 64 + lane];
                const v16i& A = acc[t / CT][t % CT];
#pragma unroll
                for (int e = 0; e < 4; ++e) fin[t][4 * q + e] = pick(A[8 + 4 * q + e], A[4 * q + e]) + v[e];
            }
    } else {
#pragma unroll
        for (int t = 0; t < C::NT_; ++t) fin[t] = acc[t / CT][t % CT];
    }

    // ---- epilogue on the 32x32 lane map: lane holds token m = column; register r holds row
    // n = 8 (r / 4) + 4 h + r % 4, so registers r_lo + 4q .. r_lo + 4q + 3 (fin[t][4q..4q+3])
    // are 4 consecutive n starting at 2 (r_lo + 4q) + 4 h
    const int64_t ldo = g.ldo;
    if constexpr (PARTIALS) {
        // int32 [M][ldo] (debug output): direct stores of 4 consecutive n per lane
        const bool vec_ok = (ldo & 3) == 0;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int m = m_base + (wm * CT + ct) * 32 + r32;
            if (m >= g.M) continue;
            int32_t* orow = static_cast<int32_t*>(g.out) + (int64_t)m * ldo;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    const v16i& F = fin[rt * CT + ct];
                    const int n0 = (nt_base + rt) * 32 + 2 * (r_lo + 4 * q) + 4 * h;
                    if (n0 >= g.N) continue;
                    const v4i v = {F[4 * q], F[4 * q + 1], F[4 * q + 2], F[4 * q + 3]};
                    if (vec_ok && n0 + 3 < g.N) {
                        *reinterpret_cast<v4i*>(orow + n0) = v;
                    } else {
                        for (int e = 0; e < 4; ++e)
                            if (n0 + e < g.N) orow[n0 + e] = v[e];
                    }
                }
        }
    } else {
        // bf16: scale, round, and stage the workgroup's [TM*32][TN*32] tile in LDS (after the
        // exchange area), then write whole row segments, 16 bytes per lane
        uint8_t* stg = smem + C::XCH;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int ml = (wm * CT + ct) * 32 + r32;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    const v16i& F = fin[rt * CT + ct];
                    const int nl = rt * 32 + 2 * (r_lo + 4 * q) + 4 * h;
                    const float4 w = swv[rt][q];
                    const uint32_t b0 = bf16_rne(((float)F[4 * q + 0] * sam[ct]) * w.x);
                    const uint32_t b1 = bf16_rne(((float)F[4 * q + 1] * sam[ct]) * w.y);
                    const uint32_t b2 = bf16_rne(((float)F[4 * q + 2] * sam[ct]) * w.z);
                    const uint32_t b3 = bf16_rne(((float)F[4 * q + 3] * sam[ct]) * w.w);
                    *reinterpret_cast<uint2*>(stg + ml * C::OPITCH + nl * 2) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
                }
        }
        __syncthreads();
        constexpr int PIECES = C::TN * 32 * 2 / 16;          // 16-byte pieces per tile row
        constexpr int TOTAL = C::TM * 32 * PIECES;
        const bool vec_ok = (ldo & 7) == 0;
        uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
        for (int it = 0; it < (TOTAL + C::NTH - 1) / C::NTH; ++it) {
            const int i = it * C::NTH + tid;
            if (i >= TOTAL) break;
            const int row = i / PIECES, pc = i % PIECES;
            const int m = m_base + row, n = nt_base * 32 + pc * 8;
            if (m >= g.M || n >= g.N) continue;
            const v4i v = *reinterpret_cast<const v4i*>(stg + row * C::OPITCH + pc * 16);
            uint16_t* dst = out + (int64_t)m * ldo + n;
            if (vec_ok && n + 7 < g.N) {
                *reinterpret_cast<v4i*>(dst) = v;
            } else {
                for (int e = 0; e < 8; ++e)
                    if (n + e < g.N) dst[e] = (uint16_t)((uint32_t)v[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

// 96 weight rows x 192 token rows per workgroup (see the notes at the top).
constexpr int RT = 3, CT = 1, WM = 6, KSP = 2;
using Cfg = W8Cfg<RT, CT, WM, KSP>;

// Byte offsets inside one launch stay below 2^31 (they are 32-bit lane offsets) and a grid
// below 2^24 workgroups (2^32 work-items), so larger problems are cut into several launches
// over ranges of token tiles and weight tiles.
constexpr int64_t MAX_OFF = int64_t(1) << 31, MAX_WG = (int64_t(1) << 24) - 1;

template <bool PARTIALS>
hipError_t launch_w8a8(const void* packed, const void* act, int64_t M, int64_t N, int64_t K, void* out,
                       int64_t ldo, hipStream_t s) {
    const PackedLayout P = packed_layout(MMQ_I8_ROW, N, K);
    const ActI8Layout A = act_i8_layout(M, K);
    const uint8_t* pb = static_cast<const uint8_t*>(packed);
    const uint8_t* ab = static_cast<const uint8_t*>(act);
    const int64_t esz = PARTIALS ? 4 : 2;
    const int64_t tile_bytes = P.KBp * 1024;                 // one 32-row tile, all blocks
    const int64_t tstep = std::max<int64_t>(1, MAX_OFF / tile_bytes / Cfg::TN) * Cfg::TN;
    const int64_t tiles_n_max = ceil_div(std::min(tstep, P.NT), Cfg::TN);
    const int64_t mtstep = std::max<int64_t>(1, std::min(MAX_OFF / tile_bytes / Cfg::TM, MAX_WG / tiles_n_max)) * Cfg::TM;
    for (int64_t mt0 = 0; mt0 < A.MT; mt0 += mtstep) {
        for (int64_t t0 = 0; t0 < P.NT; t0 += tstep) {
            const int64_t MTc = std::min(mtstep, A.MT - mt0);
            const int64_t Mc = std::min(MTc * 32, M - mt0 * 32);
            const int64_t NTc = std::min(tstep, P.NT - t0);
            const int64_t Nc = std::min(NTc * 32, N - t0 * 32);
            W8Args g{};
            g.wf = pb + P.frag_off + t0 * tile_bytes;
            g.sw = reinterpret_cast<const float*>(pb + P.scale_off) + t0 * 32;
            g.a = ab + A.a_off + mt0 * tile_bytes;
            g.sa = reinterpret_cast<const float*>(ab + A.sa_off) + mt0 * 32;
            g.M = (int)Mc;
            g.N = (int)Nc;
            g.KBp = (int)P.KBp;
            g.NT = (int)NTc;
            g.MT = (int)MTc;
            g.tiles_n = (int)ceil_div(NTc, Cfg::TN);
            g.tiles_m = (int)ceil_div(MTc, Cfg::TM);
            g.out = static_cast<uint8_t*>(out) + (mt0 * 32 * ldo + t0 * 32) * esz;
            g.ldo = ldo;
            hipLaunchKernelGGL((w8a8_kernel<RT, CT, WM, KSP, PARTIALS>),
                               dim3((unsigned)((int64_t)g.tiles_n * g.tiles_m)), dim3(Cfg::NTH), 0, s, g);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_w8a8_gemm(const void* packed, const void* act, int64_t M, int64_t N, int64_t K,
                            mmq_otype o, void* out, int64_t ldo, hipStream_t s) {
    return o == MMQ_OUT_I32_PARTIALS ? launch_w8a8<true>(packed, act, M, N, K, out, ldo, s)
                                     : launch_w8a8<false>(packed, act, M, N, K, out, ldo, s);
}

}  // namespace mmq
