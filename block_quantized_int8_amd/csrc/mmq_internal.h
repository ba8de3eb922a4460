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
constexpr int64_t GRID_ENTRIES = 2048;   // IQ1C / IQ1S codebook: one 11-bit index per 8 values

__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ activation layout
// MMQ_ACT_Q8_1 (see mmq.h):
//   region 0 xq   int8, tiled [Mp/32][KBp][64 lanes][16 B]: lane L = h*32 + r holds row r's
//                 values 16h..16h+15 of the block (the B operand of v_mfma_i32_32x32x32_i8)
//   region 1 xs2  u32   tile-major [MT][KBp][32]: xs as f16 bits in both halves (the scale-MFMA
//                 operand)
//   region 2 xsx  f32   tile-major [MT][KBp][32]: xs * xsum, exact in f32 (the Q4_K min-term
//                 operand)
//   region 3 xg   u32   tiled [MT][KBp][64 lanes]: lane L = h*32 + r holds the f16 pair
//                 (G_2h * 2^-13, G_2h+1 * 2^-13), G_j the integer sum of row r's 8-value group
//                 j of the block (the IQ1 formats' sign term; xsum = G_0 + G_1 + G_2 + G_3)
// Every region is tile-major so that a stage of a 32-row tile is one contiguous run (the
// global->LDS DMA's cost is per cache line touched) and every quantiser store is a whole line;
// a gathered (MUL_MAT_ID) token row reads one dword per block and region.
struct ActQ81Layout {
    int64_t Mp, MT, KB, KBp;
    int64_t xq_off, xs2_off, xsx_off, xg_off, bytes;
};

inline ActQ81Layout act_q8_1_layout(int64_t M, int64_t K) {
    ActQ81Layout L;
    L.Mp = round_up(M, TILE);
    L.MT = L.Mp / TILE;
    L.KB = K / QK;
    L.KBp = round_up(L.KB, KB_ALIGN);
    const int64_t cells = L.Mp * L.KBp;          // (row, block) entries of a scale region
    L.xq_off = 0;
    L.xs2_off = round_up(L.MT * L.KBp * 1024, REGION_ALIGN);
    L.xsx_off = L.xs2_off + round_up(cells * 4, REGION_ALIGN);
    L.xg_off = L.xsx_off + round_up(cells * 4, REGION_ALIGN);
    L.bytes = L.xg_off + round_up(cells * 8, REGION_ALIGN);
    return L;
}

// MMQ_ACT_I8_TOKEN (see mmq.h):
//   region 0 a    int8, tiled [Mp/32][KBp][64 lanes][16 B] exactly like the q8_1 xq region
//   region 1 sa   f32 [Mp], the per-token scale
// The tiled order lets the GEMM stage 1 KB of whole cache lines per (row tile, block).
struct ActI8Layout {
    int64_t Mp, MT, KB, KBp;
    int64_t a_off, sa_off, bytes;
};

inline ActI8Layout act_i8_layout(int64_t M, int64_t K) {
    ActI8Layout L;
    L.Mp = round_up(M, TILE);
    L.MT = L.Mp / TILE;
    L.KB = K / QK;
    L.KBp = round_up(L.KB, KB_ALIGN);
    L.a_off = 0;
    L.sa_off = round_up(L.MT * L.KBp * 1024, REGION_ALIGN);
    L.bytes = L.sa_off + round_up(L.Mp * 4, REGION_ALIGN);
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
//   IQ1T: 4 B per lane of 2-bit codes (value 16h + 4q + b at bits 8b + 2q) -> 256 B.
//   IQ1C, IQ1S (grid-index panels): 4 B per lane, W = ia << 2 | meta << 13 | ib << 20, with ia, ib
//         the 11-bit grid indices of the lane's 8-value groups 2h and 2h+1 and meta = s |
//         sigma_a << 3 | sigma_b << 4 (the half's sub-scale and the groups' sign bits) -> 256 B.
//   Q6_K: 16 B per lane of int8 q-32, as Q8_0 -> 1024 B.
// Region 1 holds one dword per (row n, block b), tile-major [NT][KBp][32] (row n, block b at
// (n/32 * KBp + b) * 32 + n%32, so a 32-row tile's stage of blocks is one contiguous run):
//   Q8_0, Q4_0: f16 d in the low half, 0 in the high half.
//   IQ1T:       f16 d (the super-block's) | meta0 << 16 | meta1 << 24, meta_h = s | sigma0 << 3 |
//               sigma1 << 4 for the half h = 0, 1 of the block (its 16-value sub-scale and the
//               sign bits of its two 8-value groups).
//   Q4_K:       d*sc split exactly into two f16 (hi | lo << 16), hi + lo = d*sc.
//   Q6_K:       d*sc_0 of the block's first 16 values, split the same way.
//   IQ1C, IQ1S: instead the f16 d of the row's super-block per (row, 4-block group g = b/4),
//               tile-major [NT][KBp/4][32] (a 4-block stage of a 32-row tile is 64 bytes).
// Region 2: Q4_K: f32 -dmin*m per (row, block); Q6_K: the d*sc_1 split of the block's last 16
// values; tile-major like region 1. IQ1C, IQ1S: the grid, 2048 dwords, entry i holding the 8
// codes c = g+1 of index i with value j at bits 8(j%4) + 2(j/4) (so a lane's code dword, in the
// IQ1T order, is entry(ia) | entry(ib) << 4).
// I8_ROW keeps one f32 per row [Np] in region 1.
struct PackedLayout {
    int64_t Np, NT, KB, KBp;
    int64_t frag_bytes;          // bytes per (nt, b) fragment
    int64_t frag_off, scale_off, min_off, bytes;
};

inline PackedLayout packed_layout(mmq_wtype t, int64_t N, int64_t K) {
    PackedLayout L;
    L.Np = round_up(N, TILE);
    L.NT = L.Np / TILE;
    L.KB = K / QK;
    L.KBp = round_up(L.KB, KB_ALIGN);
    switch (t) {
        case MMQ_Q8_0: L.frag_bytes = 1024; break;
        case MMQ_Q4_0: L.frag_bytes = 512; break;
        case MMQ_Q4_K: L.frag_bytes = 512; break;
        case MMQ_IQ1T:
        case MMQ_IQ1C:
        case MMQ_IQ1S: L.frag_bytes = 256; break;
        case MMQ_Q6_K: L.frag_bytes = 1024; break;     // int8 q-32
        default: L.frag_bytes = 1024; break;           // I8_ROW
    }
    const int64_t cells = L.Np * L.KBp;
    L.frag_off = 0;
    L.scale_off = round_up(L.NT * L.KBp * L.frag_bytes, REGION_ALIGN);
    const bool grid = (t == MMQ_IQ1C || t == MMQ_IQ1S);
    const int64_t sb = (t == MMQ_I8_ROW) ? L.Np * 4 : grid ? L.Np * (L.KBp / 4) * 2 : cells * 4;
    L.min_off = L.scale_off + round_up(sb, REGION_ALIGN);
    L.bytes = L.min_off + ((t == MMQ_Q4_K || t == MMQ_Q6_K) ? round_up(cells * 4, REGION_ALIGN)
                           : grid ? GRID_ENTRIES * 4 : 0);
    return L;
}

}  // namespace mmq

// ----------------------------------------------------------------------- device types
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// internal launchers (defined in the .hip files, called by api.cpp)
namespace mmq {
// The packed form the GEMM kernels read: IQ1S is repacked into the IQ1C grid-index panels.
inline mmq_wtype kernel_format(mmq_wtype t) { return t == MMQ_IQ1S ? MMQ_IQ1C : t; }
hipError_t launch_quantize_q8_1(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                hipStream_t s);
hipError_t launch_quantize_i8_token(const float* x, int64_t M, int64_t K, int64_t ldx, void* act,
                                    hipStream_t s);
hipError_t launch_repack(mmq_wtype t, const void* raw, const void* aux, int64_t N,
                         int64_t K, void* packed, hipStream_t s);
hipError_t launch_block_gemm(mmq_wtype t, const void* packed, const void* act, int64_t M,
                             int64_t N, int64_t K, mmq_otype o, void* out, int64_t ldo,
                             hipStream_t s);
// MUL_MAT_ID gather: full units (ufull offsets, up to gather_unit_tokens() pairs) and tail
// units (utail offsets, at most gather_tail_tokens() pairs), each a launch of its own.
hipError_t launch_block_gather(mmq_wtype t, const void* packed, int64_t E, const void* act,
                               int64_t T, int64_t top_k, int64_t N, int64_t K,
                               const int32_t* offs, const int32_t* ufull, const int32_t* utail,
                               const int32_t* perm, int max_full, int max_tail, void* out,
                               hipStream_t s);
int gather_unit_tokens();
int gather_tail_tokens();
bool gather_grid_ok(int64_t max_units, int64_t N);
// false if one expert's packed regions or the T token rows' act regions reach 2 GiB (the
// gather kernel's 32-bit DMA offsets); dense GEMMs split such problems into several launches
bool gather_regions_ok(mmq_wtype t, int64_t T, int64_t N, int64_t K);
int64_t gemm_id_max_units(int64_t E, int64_t P);
hipError_t launch_w8a8_gemm(const void* packed, const void* act, int64_t M, int64_t N, int64_t K,
                            mmq_otype o, void* out, int64_t ldo, hipStream_t s);
// Decode batches (M <= mmvq_max_tokens()): f32 out for the block formats, bf16 for I8_ROW.
int mmvq_max_tokens();
// the decode kernel takes this product (M <= mmvq_max_tokens(), or a few batches of that size)
bool mmvq_dense_ok(int64_t M, int64_t N);
hipError_t launch_mmvq(mmq_wtype t, const void* packed, const void* act, int64_t M, int64_t N,
                       int64_t K, void* out, int64_t ldo, hipStream_t s);
// MUL_MAT_ID with at most 10 tokens (and 256 pairs, K within the staging capacity): the
// decode kernel over (batch of up to 8 of one expert's pairs, 16-row group) units, from the
// route kernel's pair offsets and expert order.
bool mmvq_id_ok(mmq_wtype t, int64_t T, int64_t top_k, int64_t K);
hipError_t launch_mmvq_id(mmq_wtype t, const void* packed, int64_t E, const void* act, int64_t T,
                          int64_t top_k, int64_t N, int64_t K, const int32_t* ids, void* out,
                          hipStream_t s);
hipError_t launch_gemm_id(mmq_wtype t, const void* packed, int64_t E, const void* act,
                          const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                          void* out, void* workspace, size_t ws_bytes, hipStream_t s);
size_t gemm_id_workspace_bytes(int64_t E, int64_t T, int64_t top_k);
// The allocation-free MUL_MAT_ID's workspace: a static device array of ID_SCRATCH_BYTES per GPU;
// id_scratch() gives its device address on the current device.
constexpr size_t ID_SCRATCH_BYTES = size_t(1) << 20;
hipError_t id_scratch(void** ptr);
}  // namespace mmq
