// mmq_internal.h - layouts, constants and launcher declarations shared by the library's
// kernels and its host-side dispatch. Nothing outside csrc/ includes this file.
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
// MMQ_ACT_Q8_1 (see mmq.h): region 0 xq tiled [Mp/32][KBp][64 lanes][16 B] (lane L = h*32 + r
// holds row r's values 16h..16h+15 of the block: the B operand of v_mfma_i32_32x32x32_i8);
// region 1 xs f32, region 2 xsum int32, region 3 xs as f16 bits, each [Mp/32][KBp][32].
struct ActQ81Layout {
    int64_t Mp, MT, KB, KBp;
    int64_t xq_off, xs_off, xsum_off, xs16_off, bytes;
};

inline ActQ81Layout act_q8_1_layout(int64_t M, int64_t K) {
    ActQ81Layout L;
    L.Mp = round_up(M, TILE);
    L.MT = L.Mp / TILE;
    L.KB = K / QK;
    L.KBp = round_up(L.KB, KB_ALIGN);
    const int64_t tiles = L.MT * L.KBp;
    L.xq_off = 0;
    L.xs_off = round_up(tiles * 1024, REGION_ALIGN);
    L.xsum_off = L.xs_off + round_up(tiles * TILE * 4, REGION_ALIGN);
    L.xs16_off = L.xsum_off + round_up(tiles * TILE * 4, REGION_ALIGN);
    L.bytes = L.xs16_off + round_up(tiles * TILE * 2, REGION_ALIGN);
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
// Weight rows are grouped in 32-row tiles (nt = n/32). Region 0 holds, per (nt, block b), the
// tile's fragment: lane L = h*32 + r carries row r's values k = 16h..16h+15 of the block (the A
// operand of v_mfma_i32_32x32x32_i8; the activations use the same assignment).
//   Q8_0, I8_ROW: 16 B int8 per lane -> 1024 B.
//   Q4_0: 8 B per lane: the high nibbles of dword X0 are k = 16h+0..3 and its low nibbles
//         16h+4..7 (X1: 8..11 / 12..15), each the 4-bit two's complement of nib - 8, so masking
//         with 0xF0F0F0F0 (after a left shift by 4 for the low ones) gives int8 16*(nib-8):
//         the matrix core computes 16x the block dot, exactly -> 512 B.
//   Q4_K: 8 B per lane, unsigned nibbles: X0 & 0x0F0F0F0F = k 16h+0..3, (X0 >> 4) & 0x0F0F0F0F
//         = 16h+4..7, likewise X1 for 8..15 -> 512 B.
//   IQ1T: per lane a dword of 2-bit codes (value 16h + 4q + b at bits 8b + 2q), then 64 meta
//         bytes s | sigma0 << 3 | sigma1 << 4 (the lane's 16-value sub-scale and the sign bits of
//         its two 8-value groups) -> 320 B.
// Region 1 holds the per-(nt, b, row) scales [NT][KBp][32]: f16 d for Q8_0, Q4_0 and IQ1T (the
// super-block's d); f32 pairs (d*sc, -dmin*m) for Q4_K. I8_ROW keeps one f32 per row [Np].
struct PackedLayout {
    int64_t Np, NT, KB, KBp;
    int64_t frag_bytes;          // bytes per (nt, b) fragment
    int64_t scale_bytes;         // bytes per (nt, b, row) scale entry
    int64_t frag_off, scale_off, bytes;
};

inline PackedLayout packed_layout(mmq_wtype t, int64_t N, int64_t K) {
    PackedLayout L;
    L.Np = round_up(N, TILE);
    L.NT = L.Np / TILE;
    L.KB = K / QK;
    L.KBp = round_up(L.KB, KB_ALIGN);
    switch (t) {
        case MMQ_Q8_0: L.frag_bytes = 1024; L.scale_bytes = 2; break;
        case MMQ_Q4_0: L.frag_bytes = 512; L.scale_bytes = 2; break;
        case MMQ_Q4_K: L.frag_bytes = 512; L.scale_bytes = 8; break;
        case MMQ_IQ1T: L.frag_bytes = 320; L.scale_bytes = 2; break;
        default: L.frag_bytes = 1024; L.scale_bytes = 0; break;           // I8_ROW
    }
    L.frag_off = 0;
    L.scale_off = round_up(L.NT * L.KBp * L.frag_bytes, REGION_ALIGN);
    const int64_t sb = (t == MMQ_I8_ROW) ? L.Np * 4 : L.NT * L.KBp * TILE * L.scale_bytes;
    L.bytes = L.scale_off + round_up(sb, REGION_ALIGN);
    return L;
}

}  // namespace mmq

// ----------------------------------------------------------------------- device types
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// internal launchers (defined in the .hip files, called by api.cpp)
namespace mmq {
hipError_t launch_quantize_q8_1(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                hipStream_t s);
hipError_t launch_quantize_i8_token(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                    hipStream_t s);
hipError_t launch_repack(mmq_wtype t, const void* raw, const float* row_scale, int64_t N,
                         int64_t K, void* packed, hipStream_t s);
hipError_t launch_block_gemm(mmq_wtype t, const void* packed, const void* act, int64_t M,
                             int64_t N, int64_t K, mmq_otype o, void* out, int64_t ldo,
                             hipStream_t s);
// Dense grids: false if the launch would exceed the grid limit (checked before any launch).
bool dense_grid_ok(int64_t M, int64_t N);
hipError_t launch_block_gather(mmq_wtype t, const void* packed, int64_t E, const void* act,
                               int64_t T, int64_t top_k, int64_t N, int64_t K,
                               const int32_t* offs, const int32_t* uoff, const int32_t* perm,
                               int max_units, void* out, hipStream_t s);
int gather_unit_tokens();
bool gather_grid_ok(int64_t max_units, int64_t N);
int64_t gemm_id_max_units(int64_t E, int64_t P);
bool w8a8_grid_ok(int64_t M, int64_t N);
hipError_t launch_w8a8_gemm(const void* packed, const void* act, int64_t M, int64_t N, int64_t K,
                            mmq_otype o, void* out, int64_t ldo, hipStream_t s);
hipError_t launch_gemm_id(mmq_wtype t, const void* packed, int64_t E, const void* act,
                          const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                          void* out, void* workspace, size_t ws_bytes, hipStream_t s);
size_t gemm_id_workspace_bytes(int64_t E, int64_t T, int64_t top_k);
}  // namespace mmq
