// api.cpp - the extern "C" entry points declared in include/mmq.h: argument validation on the
// host, then a launch on the caller's stream. Nothing here allocates device memory.
#include "mmq_internal.h"

using namespace mmq;

namespace {

// Size limits of the ABI (mmq.h states them next to each call):
//  - M, N (and T * top_k) at most 2^24 and K at most 2^23: row, column and block counts stay
//    in int32 inside the kernels, and a 128-row tile's fragments of all K blocks stay below
//    2 GiB, so the dense launches can always be split into pieces whose regions the kernels'
//    32-bit byte offsets address;
//  - MMQ_I8_ROW: K < 2^17, so the int32 accumulator over all of K cannot overflow
//    (|a * w| <= 2^14 per term);
//  - the debug partials output holds at most 2^31 int32 values.
constexpr int64_t MAX_DIM = int64_t(1) << 24;
constexpr int64_t MAX_K = int64_t(1) << 23;
constexpr int64_t MAX_K_I8_ROW = int64_t(1) << 17;
constexpr int64_t MAX_PARTIALS = int64_t(1) << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_wtype(int t) { return t >= MMQ_Q8_0 && t <= MMQ_IQ1S; }
bool valid_atype(int a) { return a == MMQ_ACT_Q8_1 || a == MMQ_ACT_I8_TOKEN; }
bool valid_otype(int o) { return o >= MMQ_OUT_F32 && o <= MMQ_OUT_I32_PARTIALS; }

int64_t k_multiple(mmq_wtype t) {
    return (t == MMQ_Q4_K || t == MMQ_IQ1T || t == MMQ_IQ1C || t == MMQ_IQ1S || t == MMQ_Q6_K) ? 256 : 32;
}

// partial sums per (row, column) in MMQ_OUT_I32_PARTIALS: one per 32-value block, q6_K one per
// 16-value half
int64_t partials_per_row(mmq_wtype t, int64_t K) { return t == MMQ_Q6_K ? K / 16 : K / QK; }

// formats whose repack takes an auxiliary input (I8_ROW: row scales; IQ1C, IQ1S: the grid)
bool needs_aux(mmq_wtype t) { return t == MMQ_I8_ROW || t == MMQ_IQ1C || t == MMQ_IQ1S; }

bool sizes_ok(int64_t M, int64_t N, int64_t K) {
    return M >= 1 && N >= 1 && K >= 32 && M <= MAX_DIM && N <= MAX_DIM && K <= MAX_K;
}

// a * b * c <= lim for non-negative operands, without overflowing int64
bool product_le(int64_t a, int64_t b, int64_t c, int64_t lim) {
    if (a == 0 || b == 0 || c == 0) return true;
    if (a > lim / b) return false;
    return a * b <= lim / c;
}

mmq_status from_hip(hipError_t e) {
    if (e == hipSuccess) return MMQ_OK;
    if (e == hipErrorNotSupported) return MMQ_EUNSUPPORTED;
    return MMQ_EHIP;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* mmq_status_string(mmq_status s) {
    switch (s) {
        case MMQ_OK: return "MMQ_OK";
        case MMQ_EINVAL: return "MMQ_EINVAL: a size, stride or enum is out of range";
        case MMQ_EUNSUPPORTED: return "MMQ_EUNSUPPORTED: this format/output combination is not implemented";
        case MMQ_EALIGN: return "MMQ_EALIGN: a pointer or leading dimension is not 16-byte aligned";
        case MMQ_EWORKSPACE: return "MMQ_EWORKSPACE: workspace missing or too small";
        case MMQ_EHIP: return "MMQ_EHIP: the HIP runtime reported an error";
    }
    return "unknown mmq_status";
}

size_t mmq_act_bytes(mmq_atype a, int64_t M, int64_t K) {
    if (!valid_atype(a) || !sizes_ok(M, 1, K) || K % QK) return 0;
    if (a == MMQ_ACT_Q8_1) return (size_t)act_q8_1_layout(M, K).bytes;
    return (size_t)act_i8_layout(M, K).bytes;
}

mmq_status mmq_act_region_offsets(mmq_atype a, int64_t M, int64_t K, size_t offsets[5]) {
    if (!offsets || !valid_atype(a) || !sizes_ok(M, 1, K) || K % QK) return MMQ_EINVAL;
    if (a == MMQ_ACT_Q8_1) {
        const ActQ81Layout L = act_q8_1_layout(M, K);
        offsets[0] = (size_t)L.xq_off;
        offsets[1] = (size_t)L.xs2_off;
        offsets[2] = (size_t)L.xsx_off;
        offsets[3] = (size_t)L.xg_off;
        offsets[4] = 0;
    } else {
        const ActI8Layout L = act_i8_layout(M, K);
        offsets[0] = (size_t)L.a_off;
        offsets[1] = (size_t)L.sa_off;
        offsets[2] = offsets[3] = offsets[4] = 0;
    }
    return MMQ_OK;
}

mmq_status mmq_quantize_act(mmq_atype a, const float* x, int64_t M, int64_t K, int64_t ldx,
                            void* act, void* stream) {
    if (!valid_atype(a) || !sizes_ok(M, 1, K) || K % QK || ldx < K) return MMQ_EINVAL;
    if (!x || !act) return MMQ_EINVAL;
    if (!aligned16(x) || !aligned16(act) || (ldx & 3)) return MMQ_EALIGN;
    hipError_t e = (a == MMQ_ACT_Q8_1) ? launch_quantize_q8_1(x, M, K, ldx, act, as_stream(stream))
                                       : launch_quantize_i8_token(x, M, K, ldx, act, as_stream(stream));
    return from_hip(e);
}

size_t mmq_packed_bytes(mmq_wtype t, int64_t N, int64_t K) {
    if (!valid_wtype(t) || !sizes_ok(1, N, K) || K % k_multiple(t)) return 0;
    return (size_t)packed_layout(t, N, K).bytes;
}

mmq_status mmq_repack_weights(mmq_wtype t, const void* raw, const void* aux, int64_t N,
                              int64_t K, void* packed, void* stream) {
    if (!valid_wtype(t) || !sizes_ok(1, N, K) || K % k_multiple(t)) return MMQ_EINVAL;
    if (!raw || !packed) return MMQ_EINVAL;
    if (needs_aux(t) != (aux != nullptr)) return MMQ_EINVAL;
    if (!aligned16(raw) || !aligned16(packed) || (aux && !aligned16(aux))) return MMQ_EALIGN;
    return from_hip(launch_repack(t, raw, aux, N, K, packed, as_stream(stream)));
}

mmq_status mmq_gemm(mmq_wtype t, const void* packed, const void* act, int64_t M, int64_t N,
                    int64_t K, mmq_otype o, void* out, int64_t ldo, void* stream) {
    if (!valid_wtype(t) || !valid_otype(o) || !sizes_ok(M, N, K) || K % k_multiple(t)) return MMQ_EINVAL;
    if (!packed || !act || !out) return MMQ_EINVAL;
    if (ldo < N) return MMQ_EINVAL;
    if (o == MMQ_OUT_I32_PARTIALS && ldo != N) return MMQ_EINVAL;
    if (t == MMQ_I8_ROW) {
        if (o == MMQ_OUT_F32) return MMQ_EUNSUPPORTED;
        if (K >= MAX_K_I8_ROW) return MMQ_EINVAL;
    } else {
        if (o == MMQ_OUT_BF16) return MMQ_EUNSUPPORTED;
    }
    if (o == MMQ_OUT_I32_PARTIALS &&
        !product_le(M, N, t == MMQ_I8_ROW ? 1 : partials_per_row(t, K), MAX_PARTIALS))
        return MMQ_EINVAL;
    if (!aligned16(packed) || !aligned16(act) || !aligned16(out)) return MMQ_EALIGN;
    t = kernel_format(t);
    // decode batches go to the split-K matrix-vector kernel; the debug partials stay on the
    // prefill kernels
    if (o != MMQ_OUT_I32_PARTIALS && mmvq_dense_ok(M, N))
        return from_hip(launch_mmvq(t, packed, act, M, N, K, out, ldo, as_stream(stream)));
    if (t == MMQ_I8_ROW)
        return from_hip(launch_w8a8_gemm(packed, act, M, N, K, o, out, ldo, as_stream(stream)));
    return from_hip(launch_block_gemm(t, packed, act, M, N, K, o, out, ldo, as_stream(stream)));
}

size_t mmq_gemm_id_workspace_bytes(int64_t E, int64_t T, int64_t top_k) {
    if (E < 1 || T < 1 || top_k < 1 || top_k > E || E > 4096 || T * top_k > MAX_DIM) return 0;
    return gemm_id_workspace_bytes(E, T, top_k);
}

namespace {
// The checks of mmq_gemm_id that do not concern the workspace (MMQ_OK if all pass).
mmq_status gemm_id_args(mmq_wtype t, const void* packed, int64_t E, const void* act,
                        const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                        mmq_otype o, void* out) {
    if (!valid_wtype(t) || !valid_otype(o) || !sizes_ok(T, N, K) || K % k_multiple(t)) return MMQ_EINVAL;
    if (E < 1 || top_k < 1 || top_k > E || E > 4096 || T * top_k > MAX_DIM) return MMQ_EINVAL;
    if (!packed || !act || !ids || !out) return MMQ_EINVAL;
    if (t == MMQ_I8_ROW || o != MMQ_OUT_F32) return MMQ_EUNSUPPORTED;
    if (!aligned16(packed) || !aligned16(act) || !aligned16(ids) || !aligned16(out)) return MMQ_EALIGN;
    const mmq_wtype kt = kernel_format(t);
    if (!mmvq_id_ok(kt, T, top_k, K)) {         // the prefill gather path (decode batches: the
        if (!gather_grid_ok(gemm_id_max_units(E, T * top_k), N) || !gather_regions_ok(kt, T, N, K))
            return MMQ_EINVAL;                  // small-batch kernel, 64-bit addressing)
    }
    return MMQ_OK;
}
}  // namespace

mmq_status mmq_gemm_id(mmq_wtype t, const void* packed, int64_t E, const void* act,
                       const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                       mmq_otype o, void* out, void* workspace, size_t ws_bytes, void* stream) {
    const mmq_status st = gemm_id_args(t, packed, E, act, ids, T, top_k, N, K, o, out);
    if (st != MMQ_OK) return st;
    const size_t need = gemm_id_workspace_bytes(E, T, top_k);
    if (!workspace || ws_bytes < need) return MMQ_EWORKSPACE;
    if (!aligned16(workspace)) return MMQ_EALIGN;
    return from_hip(launch_gemm_id(kernel_format(t), packed, E, act, ids, T, top_k, N, K, out, workspace,
                                   ws_bytes, as_stream(stream)));
}

size_t mmq_gemm_id_noalloc_max_workspace_bytes(void) { return ID_SCRATCH_BYTES; }

mmq_status mmq_gemm_id_noalloc(mmq_wtype t, const void* packed, int64_t E, const void* act,
                               const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                               mmq_otype o, void* out, void* stream) {
    const mmq_status st = gemm_id_args(t, packed, E, act, ids, T, top_k, N, K, o, out);
    if (st != MMQ_OK) return st;
    const size_t need = gemm_id_workspace_bytes(E, T, top_k);
    if (need > ID_SCRATCH_BYTES) return MMQ_EWORKSPACE;
    void* ws = nullptr;
    const hipError_t e = id_scratch(&ws);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(launch_gemm_id(kernel_format(t), packed, E, act, ids, T, top_k, N, K, out, ws,
                                   ID_SCRATCH_BYTES, as_stream(stream)));
}

}  // extern "C"
