// gemm_id.hip - MUL_MAT_ID (expert-routed MoE) on top of the block-scaled MMQ kernel.
#include "mmq_internal.h"

namespace mmq {

size_t gemm_id_workspace_bytes(int64_t E, int64_t T, int64_t top_k) {
    const int64_t pairs = T * top_k;
    // counts[E], offsets[E+1], cursor[E], perm[pairs], unit list 2 x (pairs/32 + E), flags
    const int64_t words = 3 * E + 1 + pairs + 2 * (pairs / 32 + E + 1) + 64;
    return (size_t)round_up(words * 4, REGION_ALIGN);
}

hipError_t launch_gemm_id(mmq_wtype, const void*, int64_t, const void*, const int32_t*, int64_t,
                          int64_t, int64_t, int64_t, void*, void*, size_t, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace mmq
