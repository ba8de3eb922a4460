// mmq_internal.h - layouts, constants and device helpers shared by the library's kernels
// and its host-side dispatch. Nothing outside csrc/ includes this file.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mmq.h"

namespace mmq {

constexpr int QK = 32;          // values per quantisation block (one int8 MFMA k-depth)
constexpr int KB_ALIGN = 8;     // activation / packed-weight block counts are padded to this
constexpr int TILE = 32;        // rows per matrix-core tile (v_mfma_*_32x32x*)
constexpr int64_t REGION_ALIGN = 256;

__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ activation layout
// MMQ_ACT_Q8_1: xq tiled [Mp/32][KBp][64 lanes][16 B]; xs, xsum [Mp/32][KBp][32].
struct ActQ81Layout {
    int64_t Mp, MT, KB, KBp;
    int64_t xq_off, xs_off, xsum_off, bytes;
};

inline ActQ81Layout act_q8_1_layout(int64_t M, int64_t K) {
    ActQ81Layout L;
    L.Mp = round_up(M, TILE);
    L.MT = L.Mp / TILE;
    L.KB = K / QK;
    L.KBp = round_up(L.KB, KB_ALIGN);
    L.xq_off = 0;
    int64_t xq_bytes = L.MT * L.KBp * 1024;
    L.xs_off = round_up(xq_bytes, REGION_ALIGN);
    int64_t s_bytes = L.MT * L.KBp * TILE * 4;
    L.xsum_off = L.xs_off + round_up(s_bytes, REGION_ALIGN);
    L.bytes = L.xsum_off + round_up(s_bytes, REGION_ALIGN);
    return L;
}

// MMQ_ACT_I8_TOKEN: a int8 [M][K] row-major, sa f32 [M].
struct ActI8Layout {
    int64_t a_off, sa_off, bytes;
};

inline ActI8Layout act_i8_layout(int64_t M, int64_t K) {
    ActI8Layout L;
    L.a_off = 0;
    L.sa_off = round_up(M * K, REGION_ALIGN);
    L.bytes = L.sa_off + round_up(M * 4, REGION_ALIGN);
    return L;
}

// ------------------------------------------------------------------ packed weight layout
// Weight rows are grouped in 32-row tiles (nt = n/32); within a tile, block b's matrix-core
// fragment holds the A operand of v_mfma_i32_32x32x32_i8 in lane order: lane L = h*32 + r
// carries row r's 16 values k = 16h..16h+15 of the block.
//   Q8_0, I8_ROW: 16 B int8 per lane  -> 1024 B per (nt, b)
//   Q4_0        : 8 B per lane, two dwords X0, X1; the high nibbles of X0 are values
//                 k = 16h+0..3 and its low nibbles k = 16h+4..7 (X1: 8..11 / 12..15), each
//                 stored as the 4-bit two's complement of (nib - 8). Masking a dword with
//                 0xF0F0F0F0 (or shifting it left by 4 first) yields four int8 equal to
//                 16*(nib-8): the matrix core computes 16x the block dot, exactly.
//   Q4_K        : 8 B per lane, unsigned nibbles: X0 & 0x0F0F0F0F = values 16h+0..3,
//                 (X0 >> 4) & 0x0F0F0F0F = 16h+4..7, likewise X1 for 8..15.
// Scales are per (nt, b, r): f16 d for Q8_0 / Q4_0 ([NT][KBp][32], 2 B each); I8_ROW keeps
// one f32 per row [Np].
struct PackedLayout {
    int64_t Np, NT, KB, KBp;
    int64_t frag_bytes;          // bytes per (nt, b) fragment
    int64_t frag_off, scale_off, scale2_off, bytes;
};

inline int frag_bytes_of(mmq_wtype t) {
    switch (t) {
        case MMQ_Q8_0: case MMQ_I8_ROW: return 1024;
        case MMQ_Q4_0: case MMQ_Q4_K: return 512;
        case MMQ_IQ1T: return 256 + 64;   // 16 2-bit codes per lane + one meta byte per lane
    }
    return 0;
}

inline PackedLayout packed_layout(mmq_wtype t, int64_t N, int64_t K) {
    PackedLayout L;
    L.Np = round_up(N, TILE);
    L.NT = L.Np / TILE;
    L.KB = K / QK;
    L.KBp = round_up(L.KB, KB_ALIGN);
    L.frag_bytes = frag_bytes_of(t);
    L.frag_off = 0;
    int64_t fb = L.NT * L.KBp * L.frag_bytes;
    L.scale_off = round_up(fb, REGION_ALIGN);
    int64_t sb = 0, sb2 = 0;
    switch (t) {
        case MMQ_Q8_0: case MMQ_Q4_0: case MMQ_IQ1T: sb = L.NT * L.KBp * TILE * 2; break;  // f16
        case MMQ_Q4_K: sb = L.NT * L.KBp * TILE * 4; sb2 = sb; break;  // f16 hi/lo pairs x2
        case MMQ_I8_ROW: sb = L.Np * 4; break;                         // f32 per row
    }
    L.scale2_off = L.scale_off + round_up(sb, REGION_ALIGN);
    L.bytes = L.scale2_off + round_up(sb2, REGION_ALIGN);
    return L;
}

}  // namespace mmq

// ----------------------------------------------------------------------- device helpers
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// internal launchers (defined in the .hip files, called by api.hip)
namespace mmq {
hipError_t launch_quantize_q8_1(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                hipStream_t s);
hipError_t launch_quantize_i8_token(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                    hipStream_t s);
hipError_t launch_repack(mmq_wtype t, const void* raw, const float* row_scale, int64_t N,
                         int64_t K, void* packed, hipStream_t s);
hipError_t launch_gemm(mmq_wtype t, const void* packed, const void* act, int64_t M, int64_t N,
                       int64_t K, mmq_otype o, void* out, int64_t ldo, hipStream_t s);
hipError_t launch_gemm_id(mmq_wtype t, const void* packed, int64_t E, const void* act,
                          const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                          void* out, void* workspace, size_t ws_bytes, hipStream_t s);
size_t gemm_id_workspace_bytes(int64_t E, int64_t T, int64_t top_k);
}  // namespace mmq
