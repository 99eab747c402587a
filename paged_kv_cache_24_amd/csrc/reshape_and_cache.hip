// Cache write: store each new token's k and v rows in their pool slots.
//
// With the [num_blocks][16][kv_heads][head_dim] layout a token slot is one
// contiguous row of kv_heads * head_dim elements, so the write is a row copy
// from key[t] / value[t] to row slot_mapping[t] ("vLLM-Ascend 原理", §2.3 step
// 3 and §2.4 step 3).  Each lane moves one 16-byte vector; consecutive lanes
// cover consecutive bytes of a row, so loads and stores are fully coalesced.
#include "common.h"
#include "kernels.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ReshapeArgs a) {
    const int64_t vecs_per_token = 2 * (int64_t)a.row_vecs;   // K row then V row
    const int64_t total = a.num_tokens * vecs_per_token;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t t = i / vecs_per_token;
        int64_t v = i - t * vecs_per_token;
        const int64_t slot = a.slot_mapping[t];
        if (slot < 0 || slot >= a.num_slots) continue;   // padding row or outside the pool
        const bool is_v = v >= a.row_vecs;
        v -= is_v ? a.row_vecs : 0;
        const u32x4* src = static_cast<const u32x4*>(is_v ? a.value : a.key) + t * a.row_vecs + v;
        u32x4* dst = static_cast<u32x4*>(is_v ? a.v_cache : a.k_cache) + slot * a.row_vecs + v;
        *dst = __builtin_nontemporal_load(src);   // the new rows are read exactly once
    }
}

hipError_t launch_reshape_and_cache(const ReshapeArgs& a, hipStream_t stream) {
    const int64_t total = a.num_tokens * 2 * (int64_t)a.row_vecs;
    const int64_t want = (total + 255) / 256;
    const int grid = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
