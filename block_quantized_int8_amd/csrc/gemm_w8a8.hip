// gemm_w8a8.hip - per-channel W8A8 GEMM (int8 weights with an f32 scale per output channel,
// int8 activations with an f32 scale per token) on CDNA4 matrix cores.
//
// No per-block scale: the int32 accumulators run over all of K inside
// v_mfma_i32_32x32x32_i8 (C = D chaining; |acc| <= 4096*127*128 < 2^31 at K = 4096) and the
// epilogue is bf16_rne((f32(acc) * sa[m]) * sw[n]) - two f32 multiplies in that order, no
// bias (metainfer "INT8 W8A8 GEMM - Prefill", section 1: fragment -> scale -> bf16). Operands
// stream through double-buffered LDS with register staging, next stage's loads issued before
// the current MFMA sequence (same section: stage i+1 global loads before the stage-i MMACs).
// The activations are the caller's row-major int8 rows: each thread copies 16 contiguous
// bytes of a row and the copy lands them in the fragment order of the matrix core.
#include "gemm_common.h"

namespace mmq {
namespace {

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

// 2 x 2 waves, each owning 2 weight tiles x 2 token tiles -> 128 x 128 CTA tiles, 4 blocks per
// stage.
constexpr int WN = 2, WM = 2, RT = 2, CT = 2, KS = 4;

template <bool PARTIALS>
hipError_t launch_w8a8(const void* packed, const void* act, int64_t M, int64_t N, int64_t K,
                       void* out, int64_t ldo, hipStream_t s) {
    const PackedLayout P = packed_layout(MMQ_I8_ROW, N, K);
    const ActI8Layout A = act_i8_layout(M, K);
    const uint8_t* pb = static_cast<const uint8_t*>(packed);
    const uint8_t* ab = static_cast<const uint8_t*>(act);
    const int tiles_n = (int)ceil_div(N, WN * RT * 32);
    const int tiles_m = (int)ceil_div(M, WM * CT * 32);
    hipLaunchKernelGGL((w8a8_kernel<WN, WM, RT, CT, KS, PARTIALS>),
                       dim3((unsigned)((int64_t)tiles_n * tiles_m)), dim3(WN * WM * 64), 0, s,
                       pb + P.frag_off, reinterpret_cast<const float*>(pb + P.scale_off),
                       reinterpret_cast<const int8_t*>(ab + A.a_off),
                       reinterpret_cast<const float*>(ab + A.sa_off), (int)M, (int)N, (int)K,
                       (int)P.KB, (int)P.KBp, (int)P.NT, tiles_m,
                       PARTIALS ? nullptr : static_cast<uint16_t*>(out), ldo,
                       PARTIALS ? static_cast<int32_t*>(out) : nullptr);
    return hipGetLastError();
}

}  // namespace

bool w8a8_grid_ok(int64_t M, int64_t N) {
    return ceil_div(N, WN * RT * 32) * ceil_div(M, WM * CT * 32) < (int64_t(1) << 31);
}

hipError_t launch_w8a8_gemm(const void* packed, const void* act, int64_t M, int64_t N, int64_t K,
                            mmq_otype o, void* out, int64_t ldo, hipStream_t s) {
    return o == MMQ_OUT_I32_PARTIALS ? launch_w8a8<true>(packed, act, M, N, K, out, ldo, s)
                                     : launch_w8a8<false>(packed, act, M, N, K, out, ldo, s);
}

}  // namespace mmq
