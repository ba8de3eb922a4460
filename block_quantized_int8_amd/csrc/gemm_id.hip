// gemm_id.hip - MUL_MAT_ID (expert-routed MoE) through the block-scaled MMQ kernel.
//
// out[t][j][:] = act[t] x W_{ids[t][j]}^T. The (token, slot) pairs are grouped by expert on the
// device (llama.cpp PR #304 routes MUL_MAT_ID through MMQ instead of one small product per
// expert, which it reports dominates prompt processing otherwise):
//   1. route_kernel (one workgroup): count pairs per expert in LDS, exclusive scan of the
//      counts (pair offsets) and of the per-expert unit counts ceil(count / U) (unit offsets),
//      then scatter the pair ids into expert order.
//   2. the gather-mode MMQ kernel: one workgroup per (unit, 128-row weight tile); a unit is up
//      to U = 64 pairs of one expert (gather_unit_tokens()). It finds its expert by binary
//      search over the unit offsets, reads its tokens' activation rows and writes each pair's
//      own output row.
// No host round trip: the grid is sized for the worst case (P/U + min(E, P) units) and
// workgroups past the actual unit count leave at once.
#include "mmq_internal.h"

namespace mmq {
namespace {

constexpr int ROUTE_THREADS = 1024;
constexpr int MAX_E = 4096;

struct IdWorkspace {
    int64_t offs_w, uoff_w, perm_w, words;
};

IdWorkspace id_workspace(int64_t E, int64_t P) {
    IdWorkspace w;
    w.offs_w = 0;                        // pair offsets [E+1]
    w.uoff_w = E + 1;                    // unit offsets [E+1]
    w.perm_w = round_up(2 * (E + 1), 64);  // pair ids in expert order [P]
    w.words = w.perm_w + P;
    return w;
}

__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                             int U, int32_t* __restrict__ offs,
                                                             int32_t* __restrict__ uoff,
                                                             int32_t* __restrict__ perm) {
    __shared__ int cnt[MAX_E];
    __shared__ int cur[MAX_E];
    __shared__ int wtot[2][ROUTE_THREADS / 64];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += ROUTE_THREADS) cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += ROUTE_THREADS) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();

    // thread t owns experts [t*EPT, t*EPT + EPT)
    const int EPT = (E + ROUTE_THREADS - 1) / ROUTE_THREADS;
    const int e0 = tid * EPT, e1 = min(e0 + EPT, E);
    int sc = 0, su = 0;
    for (int e = e0; e < e1; ++e) {
        sc += cnt[e];
        su += (cnt[e] + U - 1) / U;
    }
    // inclusive scan across the wave, then across the 16 waves
    int ic = sc, iu = su;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int oc = __shfl_up(ic, d, 64), ou = __shfl_up(iu, d, 64);
        if (lane >= d) {
            ic += oc;
            iu += ou;
        }
    }
    if (lane == 63) {
        wtot[0][wave] = ic;
        wtot[1][wave] = iu;
    }
    __syncthreads();
    int bc = 0, bu = 0;
    for (int w = 0; w < wave; ++w) {
        bc += wtot[0][w];
        bu += wtot[1][w];
    }
    int pc = bc + ic - sc, pu = bu + iu - su;      // exclusive prefixes of this thread's range
    for (int e = e0; e < e1; ++e) {
        offs[e] = pc;
        uoff[e] = pu;
        cur[e] = pc;
        pc += cnt[e];
        pu += (cnt[e] + U - 1) / U;
    }
    if (tid == ROUTE_THREADS - 1) {
        offs[E] = pc;
        uoff[E] = pu;
    }
    __syncthreads();
    for (int p = tid; p < P; p += ROUTE_THREADS) {
        const int e = ids[p];
        if (e >= 0 && e < E) perm[atomicAdd(&cur[e], 1)] = p;
    }
}

}  // namespace

int64_t gemm_id_max_units(int64_t E, int64_t P) {
    const int64_t U = gather_unit_tokens();
    return P / U + (E < P ? E : P);
}

size_t gemm_id_workspace_bytes(int64_t E, int64_t T, int64_t top_k) {
    return (size_t)round_up(id_workspace(E, T * top_k).words * 4, REGION_ALIGN);
}

hipError_t launch_gemm_id(mmq_wtype t, const void* packed, int64_t E, const void* act,
                          const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                          void* out, void* workspace, size_t, hipStream_t s) {
    if (E > MAX_E) return hipErrorInvalidValue;
    const int64_t P = T * top_k;
    if (!gather_grid_ok(gemm_id_max_units(E, P), N)) return hipErrorInvalidValue;
    const IdWorkspace w = id_workspace(E, P);
    int32_t* ws = static_cast<int32_t*>(workspace);
    int32_t* offs = ws + w.offs_w;
    int32_t* uoff = ws + w.uoff_w;
    int32_t* perm = ws + w.perm_w;
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(ROUTE_THREADS), 0, s, ids, (int)P, (int)E,
                       gather_unit_tokens(), offs, uoff, perm);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_block_gather(t, packed, E, act, T, top_k, N, K, offs, uoff, perm,
                               (int)gemm_id_max_units(E, P), out, s);
}

}  // namespace mmq
