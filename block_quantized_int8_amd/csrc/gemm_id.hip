// gemm_id.hip - MUL_MAT_ID (expert-routed MoE) through the block-scaled MMQ kernel.
//
// out[t][j][:] = act[t] x W_{ids[t][j]}^T. The (token, slot) pairs are grouped by expert on the
// device (llama.cpp PR #304 routes MUL_MAT_ID through MMQ instead of one small product per
// expert, which it reports dominates prompt processing otherwise):
//   1. route_kernel (one workgroup): count pairs per expert in LDS; split each expert's c pairs
//      into full units of U = gather_unit_tokens() pairs plus, when the remainder is at most
//      R = gather_tail_tokens(), one tail unit (a larger remainder is a last full unit);
//      exclusive scans of the pair counts (pair offsets), full-unit counts and tail-unit counts
//      (unit offsets); then scatter the pair ids into expert order.
//   2. the gather-mode MMQ kernel in one launch: a workgroup per (unit, 256-row weight tile;
//      128 rows for q8_0 and q6_K),
//      the full units (64 token slots) first and the tails (32 slots, one token tile per wave)
//      after them, so tails fill the CUs the last full units leave idle. A workgroup finds its expert by binary search
//      over the unit offsets, reads its tokens' activation rows and writes each pair's own
//      output row.
// No host round trip: the grids are sized for the worst case and workgroups past the actual
// unit counts leave at once. With at most 10 tokens (a decode batch, where the gather tiles
// would be nearly empty) both steps are the decode kernel instead: each of its workgroups
// groups the at most 256 pairs by expert itself (a rank sort in LDS) and runs (batch of up to 8
// of one expert's pairs, 16-row group) units (gemm_mmvq.hip).
#include <mutex>

#include "mmq_internal.h"

namespace mmq {
namespace {

// The allocation-free entry point's workspace: a file-scope device array (one copy per GPU,
// held until the process ends). Host code never passes `scratch` itself to a kernel (in host
// code the name is only a stand-in for the symbol); it passes the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[ID_SCRATCH_BYTES];

constexpr int ROUTE_THREADS = 1024;
constexpr int MAX_E = 4096;

struct IdWorkspace {
    int64_t offs_w, ufull_w, utail_w, perm_w, words;
};

IdWorkspace id_workspace(int64_t E, int64_t P) {
    IdWorkspace w;
    w.offs_w = 0;                          // pair offsets [E+1]
    w.ufull_w = E + 1;                     // full-unit offsets [E+1]
    w.utail_w = 2 * (E + 1);               // tail-unit offsets [E+1]
    w.perm_w = round_up(3 * (E + 1), 64);  // pair ids in expert order [P]
    w.words = w.perm_w + P;
    return w;
}

// full units and tail units of an expert with c pairs (unit size U, tail size at most R < U)
__device__ inline int full_units(int c, int U, int R) { return c / U + (c % U > R ? 1 : 0); }
__device__ inline int tail_units(int c, int U, int R) { const int r = c % U; return (r > 0 && r <= R) ? 1 : 0; }

__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                             int U, int R, int32_t* __restrict__ offs,
                                                             int32_t* __restrict__ ufull,
                                                             int32_t* __restrict__ utail,
                                                             int32_t* __restrict__ perm) {
    __shared__ int cnt[MAX_E];
    __shared__ int cur[MAX_E];
    __shared__ int wtot[3][ROUTE_THREADS / 64];
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
    int sc = 0, sf = 0, st = 0;
    for (int e = e0; e < e1; ++e) {
        sc += cnt[e];
        sf += full_units(cnt[e], U, R);
        st += tail_units(cnt[e], U, R);
    }
    // inclusive scans across the wave, then across the 16 waves
    int ic = sc, jf = sf, jt = st;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int oc = __shfl_up(ic, d, 64), of = __shfl_up(jf, d, 64), ot = __shfl_up(jt, d, 64);
        if (lane >= d) {
            ic += oc;
            jf += of;
            jt += ot;
        }
    }
    if (lane == 63) {
        wtot[0][wave] = ic;
        wtot[1][wave] = jf;
        wtot[2][wave] = jt;
    }
    __syncthreads();
    int bc = 0, bf = 0, bt = 0;
    for (int w = 0; w < wave; ++w) {
        bc += wtot[0][w];
        bf += wtot[1][w];
        bt += wtot[2][w];
    }
    int pc = bc + ic - sc, pf = bf + jf - sf, pt = bt + jt - st;   // exclusive prefixes
    for (int e = e0; e < e1; ++e) {
        offs[e] = pc;
        ufull[e] = pf;
        utail[e] = pt;
        cur[e] = pc;
        pc += cnt[e];
        pf += full_units(cnt[e], U, R);
        pt += tail_units(cnt[e], U, R);
    }
    if (tid == ROUTE_THREADS - 1) {
        offs[E] = pc;
        ufull[E] = pf;
        utail[E] = pt;
    }
    __syncthreads();
    for (int p = tid; p < P; p += ROUTE_THREADS) {
        const int e = ids[p];
        if (e >= 0 && e < E) perm[atomicAdd(&cur[e], 1)] = p;
    }
}

}  // namespace

// Worst-case full units (the tail launch needs at most min(E, P)): sum over experts of
// floor(c/U) + 1 <= P/U + min(E, P).
int64_t gemm_id_max_units(int64_t E, int64_t P) {
    const int64_t U = gather_unit_tokens();
    return P / U + (E < P ? E : P);
}

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
hipError_t id_scratch(void** ptr) {
    static std::mutex mu;
    static void* per_device[64] = {nullptr};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (per_device[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

size_t gemm_id_workspace_bytes(int64_t E, int64_t T, int64_t top_k) {
    return (size_t)round_up(id_workspace(E, T * top_k).words * 4, REGION_ALIGN);
}

hipError_t launch_gemm_id(mmq_wtype t, const void* packed, int64_t E, const void* act,
                          const int32_t* ids, int64_t T, int64_t top_k, int64_t N, int64_t K,
                          void* out, void* workspace, size_t, hipStream_t s) {
    if (E > MAX_E) return hipErrorInvalidValue;
    const int64_t P = T * top_k;
    // a decode batch of a few tokens: the decode kernel, which groups its <= 256 pairs itself
    if (mmvq_id_ok(t, T, top_k, K)) return launch_mmvq_id(t, packed, E, act, T, top_k, N, K, ids, out, s);
    if (!gather_grid_ok(gemm_id_max_units(E, P), N)) return hipErrorInvalidValue;
    const IdWorkspace w = id_workspace(E, P);
    int32_t* ws = static_cast<int32_t*>(workspace);
    int32_t* offs = ws + w.offs_w;
    int32_t* ufull = ws + w.ufull_w;
    int32_t* utail = ws + w.utail_w;
    int32_t* perm = ws + w.perm_w;
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(ROUTE_THREADS), 0, s, ids, (int)P, (int)E,
                       gather_unit_tokens(), gather_tail_tokens(), offs, ufull, utail, perm);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_block_gather(t, packed, E, act, T, top_k, N, K, offs, ufull, utail, perm,
                               (int)gemm_id_max_units(E, P), (int)(E < P ? E : P), out, s);
}

}  // namespace mmq
