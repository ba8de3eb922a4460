// gemm.hip - the MMQ contraction on CDNA4 matrix cores.
//
//   out[m,n] = sum_b (xs[m,b] * wd[n,b]) * P[m,n,b],   P = sum_{k in b} xq[m,k] * wq[n,k]
//
// ("A Negative Result on int8 Tensor-Core MMQ", section 2; minfer "08 . R1", section 2.1.)
//
// Per 32-value block and 32x32 output tile, one v_mfma_i32_32x32x32_i8 computes the exact
// int32 block dots P (K = 32 is exactly one block, so no two scales ever share an
// accumulator). The block scale s[n][m] = wd[n]*xs[m] is an outer product of two f16
// vectors; one v_mfma_f32_32x32x16_f16 whose operands are zero except for one k slot forms
// it exactly (an f16 x f16 product is exact in f32) and - because both MFMAs are 32x32 -
// lands it on exactly the same accumulator lane map as P. The correction is then applied in
// registers, acc += f32(P) * s, with no trip through LDS (the pages identify a store ->
// sync -> reload of the accumulator per block as the wall: Hanzo paper sections 2-3; the
// fix is a manual MMA with a known fragment-to-lane map, section 4).
//
// Operands stream through LDS. The packed weights and the q8_1 activations are both stored
// in fragment order, so a stage is a handful of contiguous runs: threads copy them with
// 16-byte loads into registers, and every lane's later ds_read of a fragment is
// conflict-free. The next stage's global loads are issued before the current stage's MFMA
// sequence and written to the other LDS buffer after it (minfer R1 section 2.3: exposed
// staging latency was the largest single cost; metainfer section 1: global loads of stage
// i+1 before the stage-i MMAs, wait, then write the alternate buffer, then a barrier).
//
// Per-channel W8A8 has no per-block scale: its int32 accumulators run over all of K inside
// the MFMA (C = D chaining) and the epilogue is bf16_rne((f32(acc)*sa[m])*sw[n])
// (metainfer "INT8 W8A8 GEMM - Prefill", section 1).
#include "mmq_internal.h"

namespace {

using namespace mmq;

__device__ inline _Float16 half_from_bits(uint16_t b) {
    return __builtin_bit_cast(_Float16, b);
}

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

// ------------------------------------------------------------------- weight formats
template <mmq_wtype FMT> struct WTraits;

template <> struct WTraits<MMQ_Q8_0> {
    static constexpr int FB = 1024;      // LDS bytes per (tile, block) fragment
    static constexpr int SHIFT = 0;      // the MFMA computes P << SHIFT
    __device__ static v4i operand(const uint8_t* frag, int lane) {
        return *reinterpret_cast<const v4i*>(frag + lane * 16);
    }
};

template <> struct WTraits<MMQ_Q4_0> {
    static constexpr int FB = 512;
    static constexpr int SHIFT = 4;      // int8 operand = 16*(nib-8)
    __device__ static v4i operand(const uint8_t* frag, int lane) {
        const uint2 X = *reinterpret_cast<const uint2*>(frag + lane * 8);
        v4i a;
        a[0] = (int)(X.x & 0xF0F0F0F0u);
        a[1] = (int)((X.x << 4) & 0xF0F0F0F0u);
        a[2] = (int)(X.y & 0xF0F0F0F0u);
        a[3] = (int)((X.y << 4) & 0xF0F0F0F0u);
        return a;
    }
};

// ------------------------------------------------------------------- block-scaled MMQ
// CTA = WN x WM waves; each wave owns RT weight tiles x CT token tiles of 32x32 outputs.
// One K stage = KS blocks of 32.
template <int WF, int WS, int XF, int XS>
struct C_check {
    static constexpr bool ok = WF % 16 == 0 && WS % 16 == 0 && XF % 16 == 0 && XS % 16 == 0;
};

template <mmq_wtype FMT, int WN, int WM, int RT, int CT, int KS, bool PARTIALS>
struct BlockCfg {
    using T = WTraits<FMT>;
    static constexpr int NW = WN * WM;
    static constexpr int TN = WN * RT;                 // weight tiles per CTA
    static constexpr int TM = WM * CT;                 // token tiles per CTA
    static constexpr int WF = TN * KS * T::FB;         // LDS bytes, weight fragments
    static constexpr int XF = TM * KS * 1024;          // token fragments
    static constexpr int WS = TN * KS * 64;            // f16 weight scales
    static constexpr int XS = TM * KS * 128;           // f32 token scales
    static constexpr int BUF = WF + XF + WS + XS;
    static_assert(C_check<WF, WS, XF, XS>::ok, "stage sections must be 16-byte multiples");
};

template <mmq_wtype FMT, int WN, int WM, int RT, int CT, int KS, bool PARTIALS>
__global__ __launch_bounds__(WN * WM * 64, 2) void mmq_block_kernel(
    const uint8_t* __restrict__ wfrag, const uint16_t* __restrict__ wscale,
    const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    int M, int N, int KB, int KBp, int NT, int MT, int tiles_m,
    float* __restrict__ out, int64_t ldo, int32_t* __restrict__ partials) {
    using C = BlockCfg<FMT, WN, WM, RT, CT, KS, PARTIALS>;
    using T = typename C::T;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][C::BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wm = wave / WN;

    const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int tn = lid / tiles_m, tm = lid % tiles_m;
    const int nt_base = tn * C::TN, mt_base = tm * C::TM;

    // Stage copy plan: the LDS image of one stage is BUF bytes = U16 16-byte units, laid out as
    // [weight fragments | token fragments | weight scales | token scales]. Unit u of stage s
    // comes from a contiguous run in global memory that advances by a fixed stride per stage.
    // Thread t moves units t, t+256, ...: computed once here, then bumped every stage.
    constexpr int U16 = C::BUF / 16;
    constexpr int UPT = (U16 + C::NW * 64 - 1) / (C::NW * 64);
    const uint8_t* gsrc[UPT];
    int gstep[UPT];
    int ldst[UPT];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
        const int u = tid + i * C::NW * 64;
        const int ub = u * 16;                       // byte offset in the LDS image
        const uint8_t* src;
        int step;
        if (ub < C::WF) {
            constexpr int per = KS * T::FB;          // bytes per weight tile per stage
            const int nt = min(nt_base + ub / per, NT - 1);
            src = wfrag + (int64_t)nt * KBp * T::FB + ub % per;
            step = per;
        } else if (ub < C::WF + C::XF) {
            constexpr int per = KS * 1024;
            const int o = ub - C::WF;
            const int mt = min(mt_base + o / per, MT - 1);
            src = xq + (int64_t)mt * KBp * 1024 + o % per;
            step = per;
        } else if (ub < C::WF + C::XF + C::WS) {
            constexpr int per = KS * 64;
            const int o = ub - C::WF - C::XF;
            const int nt = min(nt_base + o / per, NT - 1);
            src = reinterpret_cast<const uint8_t*>(wscale) + (int64_t)nt * KBp * 64 + o % per;
            step = per;
        } else {
            constexpr int per = KS * 128;
            const int o = min(ub - C::WF - C::XF - C::WS, C::XS - 16);   // u >= U16 clamps in range
            const int mt = min(mt_base + o / per, MT - 1);
            src = reinterpret_cast<const uint8_t*>(xs) + (int64_t)mt * KBp * 128 + o % per;
            step = per;
        }
        gsrc[i] = src;
        gstep[i] = step;
        ldst[i] = ub;
    }
    v4i stage_regs[UPT];
    auto load_stage = [&]() {
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            stage_regs[i] = *reinterpret_cast<const v4i*>(gsrc[i]);
            gsrc[i] += gstep[i];
        }
    };
    auto store_stage = [&](uint8_t* buf) {
#pragma unroll
        for (int i = 0; i < UPT; ++i)
            if (U16 % (C::NW * 64) == 0 || i + 1 < UPT || ldst[i] < C::BUF)
                *reinterpret_cast<v4i*>(buf + ldst[i]) = stage_regs[i];
    };

    float acc[RT][CT][16];
#pragma unroll
    for (int x = 0; x < RT; ++x)
#pragma unroll
        for (int y = 0; y < CT; ++y)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

    const v16i zi = {0};
    const v16f zf = {0};
    const int nstages = KBp / KS;

    load_stage();
    store_stage(lds[0]);
    __syncthreads();
    for (int s = 0; s < nstages; ++s) {
        const uint8_t* cur = lds[s & 1];
        if (s + 1 < nstages) load_stage();        // in flight during this stage's MFMAs
        const uint8_t* wf = cur;
        const uint8_t* xf = cur + C::WF;
        const uint16_t* wsl = reinterpret_cast<const uint16_t*>(cur + C::WF + C::XF);
        const float* xsl = reinterpret_cast<const float*>(cur + C::WF + C::XF + C::WS);
#pragma unroll 1
        for (int kb = 0; kb < KS; ++kb) {
            v4i a[RT];
            v8h as[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int i = wn * RT + rt;
                a[rt] = T::operand(wf + (i * KS + kb) * T::FB, lane);
                const uint16_t sb = wsl[(i * KS + kb) * 32 + (lane & 31)];
                v8h v = {0};
                v[0] = lane < 32 ? half_from_bits(sb) : (_Float16)0;
                as[rt] = v;
            }
            v4i b[CT];
            v8h bs[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int j = wm * CT + ct;
                b[ct] = *reinterpret_cast<const v4i*>(xf + (j * KS + kb) * 1024 + lane * 16);
                const float xv = xsl[(j * KS + kb) * 32 + (lane & 31)];
                v8h v = {0};
                v[0] = lane < 32 ? (_Float16)xv : (_Float16)0;
                bs[ct] = v;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[rt], b[ct], zi, 0, 0, 0);
                    if constexpr (PARTIALS) {
                        const int kbg = s * KS + kb;
                        const int m = (mt_base + wm * CT + ct) * 32 + (lane & 31);
                        if (kbg < KB && m < M) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int n = (nt_base + wn * RT + rt) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                                if (n < N) partials[((int64_t)m * N + n) * KB + kbg] = D[r] >> T::SHIFT;
                            }
                        }
                    } else {
                        const v16f S = __builtin_amdgcn_mfma_f32_32x32x16_f16(as[rt], bs[ct], zf, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[rt][ct][r] = __builtin_fmaf((float)D[r], S[r], acc[rt][ct][r]);
                    }
                }
        }
        if (s + 1 < nstages) store_stage(lds[(s + 1) & 1]);
        __syncthreads();
    }

    if constexpr (!PARTIALS) {
        constexpr float post = 1.0f / (float)(1 << T::SHIFT);
        const bool vec_ok = (ldo & 3) == 0;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int m = (mt_base + wm * CT + ct) * 32 + (lane & 31);
                if (m >= M) continue;
                float* orow = out + (int64_t)m * ldo;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n0 = (nt_base + wn * RT + rt) * 32 + 8 * g + 4 * (lane >> 5);
                    const float v0 = acc[rt][ct][4 * g + 0] * post, v1 = acc[rt][ct][4 * g + 1] * post;
                    const float v2 = acc[rt][ct][4 * g + 2] * post, v3 = acc[rt][ct][4 * g + 3] * post;
                    if (vec_ok && n0 + 3 < N) {
                        *reinterpret_cast<float4*>(orow + n0) = make_float4(v0, v1, v2, v3);
                    } else {
                        if (n0 + 0 < N) orow[n0 + 0] = v0;
                        if (n0 + 1 < N) orow[n0 + 1] = v1;
                        if (n0 + 2 < N) orow[n0 + 2] = v2;
                        if (n0 + 3 < N) orow[n0 + 3] = v3;
                    }
                }
            }
    }
}

// ------------------------------------------------------------------- per-channel W8A8
template <int WN, int WM, int RT, int CT, int KS, bool PARTIALS>
__global__ __launch_bounds__(WN * WM * 64, 2) void w8a8_kernel(
    const uint8_t* __restrict__ wfrag, const float* __restrict__ sw, const int8_t* __restrict__ a,
    const float* __restrict__ sa, int M, int N, int K, int KB, int KBp, int NT, int tiles_m,
    uint16_t* __restrict__ out, int64_t ldo, int32_t* __restrict__ acc_out) {
    constexpr int NW = WN * WM, TN = WN * RT, TM = WM * CT;
    constexpr int WF = TN * KS * 1024, XF = TM * KS * 1024, BUF = WF + XF;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wm = wave / WN;
    const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int tn = lid / tiles_m, tm = lid % tiles_m;
    const int nt_base = tn * TN, mt_base = tm * TM;

    // Stage copy plan (16-byte units). Weight fragments are contiguous per tile. Token rows are
    // row-major: 2*KS consecutive units of a row are one row's KS*32 bytes (coalesced reads);
    // unit c of row r goes to fragment (block c/2) at lane (c%2)*32 + r%32. Rows past M are
    // clamped to row M-1, and blocks past KB to block KB-1: the weight fragments of blocks
    // >= KB are zero, so the clamped bytes contribute nothing.
    constexpr int U16 = BUF / 16;
    constexpr int UPT = (U16 + NW * 64 - 1) / (NW * 64);
    static_assert(U16 % (NW * 64) == 0, "stage must split evenly over the threads");
    int64_t goff[UPT];
    int ldst[UPT];
    bool is_w[UPT];
    int trow[UPT], tchunk[UPT];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
        const int u = tid + i * NW * 64;
        const int ub = u * 16;
        if (ub < WF) {
            constexpr int per = KS * 1024;
            const int nt = min(nt_base + ub / per, NT - 1);
            goff[i] = (int64_t)nt * KBp * 1024 + ub % per;
            ldst[i] = ub;
            is_w[i] = true;
            trow[i] = 0;
            tchunk[i] = 0;
        } else {
            const int o = u - WF / 16;                     // token unit index
            const int row = o / (2 * KS), c = o % (2 * KS);
            const int j = row / 32, r = row % 32;
            const int m = min((mt_base + j) * 32 + r, M - 1);
            goff[i] = (int64_t)m * K;
            ldst[i] = WF + (j * KS + c / 2) * 1024 + ((c & 1) * 32 + r) * 16;
            is_w[i] = false;
            trow[i] = m;
            tchunk[i] = c;
        }
    }
    v4i stage_regs[UPT];
    auto load_stage = [&](int stage) {
        const int kb0 = stage * KS;
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const uint8_t* src;
            if (is_w[i]) {
                src = wfrag + goff[i] + (int64_t)stage * KS * 1024;
            } else {
                const int kb = min(kb0 + tchunk[i] / 2, KB - 1);
                src = reinterpret_cast<const uint8_t*>(a) + goff[i] + kb * 32 + (tchunk[i] & 1) * 16;
            }
            stage_regs[i] = *reinterpret_cast<const v4i*>(src);
        }
    };
    auto store_stage = [&](uint8_t* buf) {
#pragma unroll
        for (int i = 0; i < UPT; ++i) *reinterpret_cast<v4i*>(buf + ldst[i]) = stage_regs[i];
    };

    v16i acc[RT][CT];
#pragma unroll
    for (int x = 0; x < RT; ++x)
#pragma unroll
        for (int y = 0; y < CT; ++y) acc[x][y] = (v16i){0};

    const int nstages = KBp / KS;
    load_stage(0);
    store_stage(lds[0]);
    __syncthreads();
    for (int s = 0; s < nstages; ++s) {
        const uint8_t* cur = lds[s & 1];
        if (s + 1 < nstages) load_stage(s + 1);
#pragma unroll
        for (int kb = 0; kb < KS; ++kb) {
            v4i wa[RT], xb[CT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                wa[rt] = *reinterpret_cast<const v4i*>(cur + ((wn * RT + rt) * KS + kb) * 1024 + lane * 16);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                xb[ct] = *reinterpret_cast<const v4i*>(cur + WF + ((wm * CT + ct) * KS + kb) * 1024 + lane * 16);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    acc[rt][ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wa[rt], xb[ct], acc[rt][ct], 0, 0, 0);
        }
        if (s + 1 < nstages) store_stage(lds[(s + 1) & 1]);
        __syncthreads();
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int m = (mt_base + wm * CT + ct) * 32 + (lane & 31);
            if (m >= M) continue;
            const float sam = sa[m];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = (nt_base + wn * RT + rt) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (n >= N) continue;
                if constexpr (PARTIALS) {
                    acc_out[(int64_t)m * N + n] = acc[rt][ct][r];
                } else {
                    const float t = (float)acc[rt][ct][r] * sam;
                    const float u = t * sw[n];
                    out[(int64_t)m * ldo + n] = bf16_rne(u);
                }
            }
        }
}

// ------------------------------------------------------------------- launchers
template <mmq_wtype FMT, bool PARTIALS>
hipError_t launch_block(const void* packed, const void* act, int64_t M, int64_t N, int64_t K,
                        void* out, int64_t ldo, hipStream_t s) {
    constexpr int WN = 2, WM = 2, RT = 2, CT = 2, KS = 4;
    const PackedLayout P = packed_layout(FMT, N, K);
    const ActQ81Layout A = act_q8_1_layout(M, K);
    const uint8_t* pb = static_cast<const uint8_t*>(packed);
    const uint8_t* ab = static_cast<const uint8_t*>(act);
    const int tiles_n = (int)ceil_div(N, WN * RT * 32);
    const int tiles_m = (int)ceil_div(M, WM * CT * 32);
    hipLaunchKernelGGL((mmq_block_kernel<FMT, WN, WM, RT, CT, KS, PARTIALS>),
                       dim3((unsigned)(tiles_n * tiles_m)), dim3(WN * WM * 64), 0, s,
                       pb + P.frag_off, reinterpret_cast<const uint16_t*>(pb + P.scale_off),
                       ab + A.xq_off, reinterpret_cast<const float*>(ab + A.xs_off), (int)M, (int)N,
                       (int)A.KB, (int)A.KBp, (int)P.NT, (int)A.MT, tiles_m,
                       PARTIALS ? nullptr : static_cast<float*>(out), ldo,
                       PARTIALS ? static_cast<int32_t*>(out) : nullptr);
    return hipGetLastError();
}

template <bool PARTIALS>
hipError_t launch_w8a8(const void* packed, const void* act, int64_t M, int64_t N, int64_t K,
                       void* out, int64_t ldo, hipStream_t s) {
    constexpr int WN = 2, WM = 2, RT = 2, CT = 2, KS = 4;
    const PackedLayout P = packed_layout(MMQ_I8_ROW, N, K);
    const ActI8Layout A = act_i8_layout(M, K);
    const uint8_t* pb = static_cast<const uint8_t*>(packed);
    const uint8_t* ab = static_cast<const uint8_t*>(act);
    const int tiles_n = (int)ceil_div(N, WN * RT * 32);
    const int tiles_m = (int)ceil_div(M, WM * CT * 32);
    hipLaunchKernelGGL((w8a8_kernel<WN, WM, RT, CT, KS, PARTIALS>),
                       dim3((unsigned)(tiles_n * tiles_m)), dim3(WN * WM * 64), 0, s,
                       pb + P.frag_off, reinterpret_cast<const float*>(pb + P.scale_off),
                       reinterpret_cast<const int8_t*>(ab + A.a_off),
                       reinterpret_cast<const float*>(ab + A.sa_off), (int)M, (int)N, (int)K,
                       (int)P.KB, (int)P.KBp, (int)P.NT, tiles_m,
                       PARTIALS ? nullptr : static_cast<uint16_t*>(out), ldo,
                       PARTIALS ? static_cast<int32_t*>(out) : nullptr);
    return hipGetLastError();
}

}  // namespace

namespace mmq {

hipError_t launch_gemm(mmq_wtype t, const void* packed, const void* act, int64_t M, int64_t N,
                       int64_t K, mmq_otype o, void* out, int64_t ldo, hipStream_t s) {
    const bool parts = (o == MMQ_OUT_I32_PARTIALS);
    switch (t) {
        case MMQ_Q8_0:
            return parts ? launch_block<MMQ_Q8_0, true>(packed, act, M, N, K, out, ldo, s)
                         : launch_block<MMQ_Q8_0, false>(packed, act, M, N, K, out, ldo, s);
        case MMQ_Q4_0:
            return parts ? launch_block<MMQ_Q4_0, true>(packed, act, M, N, K, out, ldo, s)
                         : launch_block<MMQ_Q4_0, false>(packed, act, M, N, K, out, ldo, s);
        case MMQ_I8_ROW:
            return parts ? launch_w8a8<true>(packed, act, M, N, K, out, ldo, s)
                         : launch_w8a8<false>(packed, act, M, N, K, out, ldo, s);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace mmq
