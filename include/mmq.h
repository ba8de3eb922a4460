/*
 * mmq.h - C ABI of the MI355X (gfx950) prefill MMQ library, libmmq.so.
 *
 * MMQ ("matrix multiplication with quantized weights") computes
 *
 *     out[m,n] = sum over 32-value k-blocks b of (xs[m,b] * wd[n,b]) * sum_{k in b} xq[m,k] * wq[n,k]
 *
 * with weights kept in their raw block-quantised form, activations quantised once per
 * call to q8_1 (int8 values, one scale and one integer sum per 32 values), every int8 x
 * int8 block dot accumulated exactly in int32, and the f32 block scale applied once per
 * block. Definition: "A Negative Result on int8 Tensor-Core MMQ" (Hanzo paper 07.5),
 * section 2; minfer "08 . R1 - int8 MMQ prefill GEMM", sections 2.1-2.2 and 3.2.
 *
 * Conventions for every entry point
 *  - Pointers marked (device) are device pointers on the current HIP device; (host) are
 *    host pointers. The caller allocates and frees every buffer; the library never
 *    allocates or frees memory and keeps no per-call state.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). All device
 *    work is enqueued asynchronously on it; nothing synchronises.
 *  - Arguments are validated on the host before anything is enqueued. On any error the
 *    call returns a non-zero status and enqueues nothing. A failed kernel launch returns
 *    MMQ_EHIP. Faults inside kernels surface at the caller's next stream synchronisation.
 *  - Every device pointer must be 16-byte aligned (MMQ_EALIGN otherwise).
 *  - Sizes are int64_t: 1 <= M, N <= 2^24 and 32 <= K <= 2^23 for every call (MMQ_EINVAL
 *    otherwise); further limits are stated at the calls they constrain.
 */
#ifndef MMQ_H
#define MMQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MMQ_OK = 0,
    MMQ_EINVAL = 1,        /* a size, stride or enum is out of range */
    MMQ_EUNSUPPORTED = 2,  /* valid enums, but the combination is not implemented */
    MMQ_EALIGN = 3,        /* a pointer or leading dimension breaks the alignment rule */
    MMQ_EWORKSPACE = 4,    /* the workspace is missing or too small */
    MMQ_EHIP = 5           /* the HIP runtime reported an error (launch failure) */
} mmq_status;

/* Raw weight formats (row-major: row n of W is K consecutive values, stored as blocks).
 * Byte layouts (little-endian):
 *  MMQ_Q8_0  34 B per 32 values: f16 d, int8 q[32].                      w = d*q
 *  MMQ_Q4_0  18 B per 32 values: f16 d, u8 qs[16]; value j = qs[j]&15, value j+16 =
 *            qs[j]>>4.                                                   w = d*(nib-8)
 *  MMQ_Q4_K  144 B per 256 values: f16 d, f16 dmin, 6 B of eight 6-bit sub-block scales
 *            sc (LSB-first), 6 B of eight 6-bit mins m, u8 qs[128]; sub-block j uses
 *            qs[16j..16j+15], low nibble = value 32j+i, high = value 32j+16+i.
 *                                                             w = d*sc_j*nib - dmin*m_j
 *            d*sc_j must stay below 65504 and dmin*m_j must be finite in f32 (the repack
 *            splits d*sc_j exactly into two f16; a larger product is not representable there
 *            and the call's output is then undefined - the caller must not pass one).
 *  MMQ_IQ1T  76 B per 256 values (IQ1_M-style ternary): u8 codes[64] (2-bit c = g+1, four
 *            per byte LSB-first, c = 3 invalid), 6 B of sixteen 3-bit sub-scales s (one per
 *            16 values, LSB-first), 4 B of 32 sign bits (one per 8 values, 0 -> +1/8,
 *            1 -> -1/8), f16 d.                                   w = d*(2s+1)*(g+delta)
 *  MMQ_I8_ROW int8 [N][K] plus one f32 scale per row (per-channel W8A8).  w = sw[n]*q
 *  MMQ_IQ1C  56 B per 256 values (the IQ1_M codebook form, 1.75 bits per value): u8 qs[32]
 *            (low 8 bits of each 8-value group's 11-bit grid index), u8 qh[16] (byte j holds
 *            groups 2j and 2j+1 in its low and high nibble: nibble bits 0-2 = index bits
 *            8-10, bit 3 = the group's delta sign, 0 -> +1/8, 1 -> -1/8), 6 B of sixteen
 *            3-bit sub-scales s (LSB-first), f16 d. The grid (passed to the repack) holds
 *            2048 uint16 entries, each eight 2-bit codes c = g+1 (value j of the group at
 *            bits 2j..2j+1; code 3 is invalid).                   w = d*(2s+1)*(g+delta)
 *  MMQ_IQ1S  50 B per 256 values (the IQ1_S codebook form, 1.5625 bits per value): f16 d,
 *            u8 qs[32] (low 8 bits of each 8-value group's 11-bit grid index), uint16 qh[8]
 *            (one per 32-value block: bits 3j..3j+2 = index bits 8-10 of the block's group j,
 *            bits 12-14 = the block's sub-scale s, bit 15 = its delta sign, 0 -> +1/8), with
 *            the same grid as MMQ_IQ1C.                              w = d*(2s+1)*(g+delta)
 *  MMQ_Q6_K  210 B per 256 values: u8 ql[128], u8 qh[64], int8 sc[16] (one per 16 values),
 *            f16 d. In 32-value block j, value 32j+i (i < 16) has its low 4 bits in the low
 *            nibble of ql[16j+i] and value 32j+16+i in the high nibble; the high 2 bits of
 *            value 32j+8t+i (t < 4, i < 8) are bits 2t..2t+1 of qh[8j+i]; q = low | high << 4
 *            in 0..63.                                                   w = d*sc_h*(q-32)
 *            d*|sc| must stay below 65504 (the repack splits d*sc into two f16; a larger
 *            product makes the output undefined - the caller must not pass one).
 * Value formulas: minfer R1 sections 1-2.2 (q8_0, q4_0, Q4_K), 2.2 and 3.3 (q6_K: 6-bit grid
 * moved to the signed domain by -32, a scale per 16 values); llama.cpp PR #304 description
 * (IQ1_M and IQ1_S, the 11-bit grid index per 8 values, IQ1_M's per-16 sub-scales); metainfer "INT8 W8A8
 * GEMM - Prefill" section 1 (per-channel). */
typedef enum {
    MMQ_Q8_0 = 0, MMQ_Q4_0 = 1, MMQ_Q4_K = 2, MMQ_IQ1T = 3, MMQ_I8_ROW = 4, MMQ_IQ1C = 5,
    MMQ_Q6_K = 6, MMQ_IQ1S = 7
} mmq_wtype;

/* Activation formats.
 *  MMQ_ACT_Q8_1     per 32-value block: amax = max|x|; d = amax/127 (f32); di = 1/d in f32,
 *                   except di = 0 if d = 0 and di = FLT_MAX (the largest finite f32) where 1/d
 *                   overflows (amax below ~3.7e-37); q = clamp(round-half-even(x * di), -128,
 *                   127); the stored scale xs = d rounded to f16 (kept as f32); xsum = sum of
 *                   the 32 q (minfer R1 section 3.2 CPU reference; section 2.2 block sum).
 *                   The inputs must be finite.
 *  MMQ_ACT_I8_TOKEN one block per row (the whole of K), the same di rule, scale kept in f32
 *                   (metainfer W8A8 section 1: int8 activations with a per-token f32 scale). */
typedef enum { MMQ_ACT_Q8_1 = 0, MMQ_ACT_I8_TOKEN = 1 } mmq_atype;

/* Output types.
 *  MMQ_OUT_F32          f32 [M][ldo] (block-quantised formats)
 *  MMQ_OUT_BF16         bf16 [M][ldo]: bf16_rne((f32(acc) * sa[m]) * sw[n]), for MMQ_I8_ROW
 *                       with MMQ_ACT_I8_TOKEN only (metainfer section 1: fragment -> scale ->
 *                       bf16, no bias)
 *  MMQ_OUT_I32_PARTIALS debug: block formats: int32 [M][N][K/32] of the exact per-block
 *                       integer dots (Q4_K: sum xq*nib with unsigned nibbles; IQ1T, IQ1C, IQ1S: the folded
 *                       sum_h (2s_h+1) * sum_16 xq*(8g+-1)); MMQ_Q6_K: int32 [M][N][K/16], the
 *                       two half-block dots sum_16 xq*(q-32) of every block (half h of block b
 *                       at index 2b+h); MMQ_I8_ROW: int32 [M][N] of the full-K accumulators.
 *                       ldo must equal N. Same kernels as the scaled outputs, the scale step
 *                       replaced by a store. */
typedef enum { MMQ_OUT_F32 = 0, MMQ_OUT_BF16 = 1, MMQ_OUT_I32_PARTIALS = 2 } mmq_otype;

/* ---------------------------------------------------------------------------------------
 * Activation buffer ("act"). Opaque to most callers, but its layout is fixed so that other
 * producers can fill it. Let Mp = M rounded up to 32, KB = K/32, KBp = KB rounded up to 8.
 *
 * MMQ_ACT_Q8_1 (four regions, each starting on a 256-byte boundary):
 *   region 0  xq   int8, Mp*KBp*32 bytes, tiled for the matrix cores: the 32x32 tile
 *                  (row tile mt = m/32, block b) occupies bytes [(mt*KBp + b)*1024, +1024);
 *                  inside it, row r = m%32 and k' = k%32 sit at ((k'/16)*32 + r)*16 + k'%16.
 *   region 1  xs2  uint32, tile-major: (row m, block b) at ((m/32)*KBp + b)*32 + m%32; the
 *                  scale xs as f16 bits in both 16-bit halves (xs is f16-exact by construction).
 *   region 2  xsx  f32, tile-major like region 1: xs * xsum (exact in f32), xsum the block's
 *                  integer sum of q.
 *   region 3  xg   uint32, (row m, block b, half h) at ((m/32)*KBp + b)*64 + h*32 + m%32: the
 *                  f16 pair (G_2h * 2^-13, G_2h+1 * 2^-13) in its low and high halves, G_j the
 *                  integer sum of the 8 values q of group j (values 8j..8j+7) of the block
 *                  (exact in f16; xsum = G_0 + G_1 + G_2 + G_3).
 *   Rows m >= M and blocks b >= KB hold zeros in every region.
 * MMQ_ACT_I8_TOKEN (two regions, each starting on a 256-byte boundary):
 *   region 0  a    int8, Mp*KBp*32 bytes, tiled exactly like region 0 of MMQ_ACT_Q8_1 (the
 *                  value of row m, column k at ((m/32)*KBp + k/32)*1024 +
 *                  (((k%32)/16)*32 + m%32)*16 + k%16).
 *   region 1  sa   f32 [Mp]: the per-token scale.
 *   Rows m >= M and blocks b >= KB hold zeros in both regions.
 * --------------------------------------------------------------------------------------- */

/* Total bytes of an act buffer; 0 if the arguments are invalid. (host only) */
size_t mmq_act_bytes(mmq_atype a, int64_t M, int64_t K);

/* Byte offsets of the act buffer's regions (MMQ_ACT_Q8_1: regions 0..3; MMQ_ACT_I8_TOKEN:
 * regions 0..1), written to offsets[0..4], unused entries 0 (host). Returns MMQ_EINVAL for
 * invalid arguments. (host only) */
mmq_status mmq_act_region_offsets(mmq_atype a, int64_t M, int64_t K, size_t offsets[5]);

/* Quantise f32 activations x [M][ldx] (device, row stride ldx >= K floats) into `act`
 * (device, mmq_act_bytes(a, M, K) bytes). Deterministic and bit-exact with the definition
 * above. K must be a multiple of 32. (minfer R1 section 3.2 for q8_1; W8A8 section 1 for
 * the per-token form.) */
mmq_status mmq_quantize_act(mmq_atype a, const float* x, int64_t M, int64_t K, int64_t ldx,
                            void* act, void* stream);

/* Bytes of the packed (repacked) weight buffer for one N x K matrix; 0 if invalid. */
size_t mmq_packed_bytes(mmq_wtype t, int64_t N, int64_t K);

/* One-time, untimed repack of raw weights into the library's matrix-core panel layout.
 *  raw       (device) raw rows as described at mmq_wtype; for MMQ_I8_ROW the int8 [N][K]
 *            values.
 *  aux       (device) MMQ_I8_ROW: f32 [N] per-row scales; MMQ_IQ1C, MMQ_IQ1S: the grid,
 *            uint16 [2048]; must be NULL for every other format. Read only during the call's
 *            kernels; not referenced afterwards.
 *  packed    (device) mmq_packed_bytes(t, N, K) bytes; every region is written completely
 *            (padding rows and blocks are zero), the alignment gaps between regions are not
 *            written. Immutable afterwards and safe to reuse across graph replays
 *            (metainfer section 3.2: one-time pack outside the timed region).
 * K must be a multiple of 32 (Q8_0, Q4_0, I8_ROW) or 256 (Q4_K, Q6_K, IQ1T, IQ1C, IQ1S).
 * MMQ_IQ1C and MMQ_IQ1S keep their grid indices: per 16 values one dword with the two
 * 11-bit indices and that half-block's s and delta signs (IQ1S repeats its per-32 s and
 * sign), d per 4-block group, and a copy of the grid (2048 entries, 8 KiB) at the end of the
 * packed buffer, which the GEMMs look up on chip (about 2.1 bits per value instead of the
 * 3 of the expanded MMQ_IQ1T form). The two formats share one kernel form. An invalid code
 * (3, in IQ1T rows or in a grid entry) decodes as 0 - the caller must not pass one. */
mmq_status mmq_repack_weights(mmq_wtype t, const void* raw, const void* aux,
                              int64_t N, int64_t K, void* packed, void* stream);

/* The MMQ contraction out = act x packed^T.
 *  packed (device) from mmq_repack_weights(t, ..., N, K, ...)
 *  act    (device) from mmq_quantize_act (MMQ_ACT_Q8_1 for the block formats,
 *         MMQ_ACT_I8_TOKEN for MMQ_I8_ROW) with the same M and K
 *  out    (device) o = MMQ_OUT_F32: f32 [M][ldo]; MMQ_OUT_BF16: bf16 [M][ldo];
 *         MMQ_OUT_I32_PARTIALS: see mmq_otype (ldo = N). Columns n >= N of each row are
 *         left untouched.
 *  ldo    >= N, in elements.
 * Supported (t, o): block formats with F32 or I32_PARTIALS; I8_ROW with BF16 or
 * I32_PARTIALS.
 * Limits (MMQ_EINVAL before any launch): MMQ_I8_ROW needs K < 131072, so that its int32
 * accumulator over all of K cannot overflow (|q_a * q_w| <= 2^14 per term); the
 * I32_PARTIALS output holds at most 2^31 values. Problems whose packed weights or act
 * buffer reach 2 GiB (e.g. a 262144 x 8192 q8_0 matrix) are run as several launches over
 * ranges of weight and token tiles, with the same results.
 * Dispatch: batches of M <= 16 token rows (F32 / BF16 output) run the small-batch split-K
 * kernel, and so do up to 128 rows as batches of 16 while the batches times the 16-row weight
 * groups, ceil(M/16) * ceil(N/16), stay within 8 times the compute-unit count (such products
 * would leave a prefill grid mostly idle); larger ones run the prefill tiles (a decode batch
 * would leave a prefill tile mostly empty; llama.cpp PR #304, Summary: small batches stay on a
 * matrix-vector kernel). Both compute the same per-block integer dots, with their own f32
 * summation orders; the small-batch kernel may read the zero padding rows M..31 of the
 * activation buffer, so that padding must be zero (mmq_quantize_act writes it so). */
mmq_status mmq_gemm(mmq_wtype t, const void* packed, const void* act, int64_t M, int64_t N,
                    int64_t K, mmq_otype o, void* out, int64_t ldo, void* stream);

/* Workspace bytes needed by mmq_gemm_id for E experts, T tokens, top_k slots. */
size_t mmq_gemm_id_workspace_bytes(int64_t E, int64_t T, int64_t top_k);

/* MUL_MAT_ID (expert-routed MoE, llama.cpp PR #304: MUL_MAT_ID through MMQ):
 *     out[t][j][:] = act[t] x W_{ids[t][j]}^T      for t < T, j < top_k
 *  packed    (device) E packed matrices back to back, each mmq_packed_bytes(t, N, K) bytes
 *            (so every matrix starts on a 256-byte boundary)
 *  E         1..4096 experts; 1 <= top_k <= E
 *  act       (device) MMQ_ACT_Q8_1 act of T rows
 *  ids       (device) int32 [T][top_k]; pair p = t*top_k + j uses expert ids[p]. Pairs with
 *            an id outside [0, E) are skipped (their output rows are left untouched).
 *  out       (device) f32 [T][top_k][N]
 *  workspace (device) >= mmq_gemm_id_workspace_bytes(E, T, top_k) bytes of scratch; its
 *            contents need no initialisation and are overwritten. Two calls that overlap in
 *            time must not share one workspace.
 * The expert grouping (count per expert, scan, scatter of the pairs into expert order) runs
 * on the device with no host round trip, so the call is stream-ordered and capturable; the
 * order of pairs inside one expert is unspecified and does not affect any output value.
 * Decode batches (T <= 10, T*top_k <= 256; past 8 tokens K <= 4096) run the small-batch kernel
 * per expert instead of the prefill tiles (llama.cpp PR #304, Summary: small batches stay on a
 * matrix-vector kernel); the result is the same per-block contraction.
 * Block formats only; o must be MMQ_OUT_F32. MMQ_IQ1C / MMQ_IQ1S: every expert must have
 * been packed with the same grid (the decode-batch kernel reads the first matrix's copy).
 * Limits (MMQ_EINVAL before any launch): T * top_k <= 2^24; outside the decode-batch case,
 * one expert's packed matrix must keep its fragment and scale regions below 2 GiB each
 * (e.g. N * K < 2^31 values of q8_0) and the act buffer's value region below 2 GiB
 * (T * K < 2^31), because the grouped launch addresses them with 32-bit offsets. */
mmq_status mmq_gemm_id(mmq_wtype t, const void* packed, int64_t E, const void* act,
                       const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                       mmq_otype o, void* out, void* workspace, size_t ws_bytes, void* stream);

/* MUL_MAT_ID for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. The same operation, arguments, limits
 * and kernels as mmq_gemm_id, without the workspace argument: the call allocates nothing and
 * takes its workspace from a static device array of the library, one per GPU (held until the
 * process ends), of mmq_gemm_id_noalloc_max_workspace_bytes() bytes (1 MiB).
 *  - If mmq_gemm_id_workspace_bytes(E, T, top_k) exceeds that size the call returns
 *    MMQ_EWORKSPACE and enqueues nothing (1 MiB covers e.g. E = 4096 experts with up to
 *    249,000 (token, slot) pairs).
 *  - Every call on one GPU shares that GPU's array and leaves its contents behind (the next
 *    call needs no clearing: every call writes all of the workspace it reads). Calls that
 *    overlap in time on one GPU (different streams, or different host threads without stream
 *    ordering between them) race on the array and must not be made. */
mmq_status mmq_gemm_id_noalloc(mmq_wtype t, const void* packed, int64_t E, const void* act,
                               const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                               mmq_otype o, void* out, void* stream);

/* Size of mmq_gemm_id_noalloc's static workspace, in bytes (host). */
size_t mmq_gemm_id_noalloc_max_workspace_bytes(void);

/* Static, human-readable name of a status code (host). */
const char* mmq_status_string(mmq_status s);

#ifdef __cplusplus
}
#endif
#endif /* MMQ_H */
