// Block copy: physical block dst becomes a copy of physical block src, K and V,
// all kv heads.  This is the copy behind copy-on-write forks of shared prefixes
// ("vLLM-Ascend 原理", §2.1) and behind swapping ("vLLM学习整理", §三 "Preemption").
// A block is block_size * kv_heads * head_dim contiguous elements, so the copy
// is a plain streaming copy of 16-byte vectors; each workgroup moves 1024
// vectors (4 per lane, issued together) of one pair's K and V.
#include "common.h"
#include "kernels.h"

namespace pa {

typedef uint32_t cb_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
    constexpr int kVecsPerWG = 1024;
    const int64_t pair = blockIdx.x / a.wgs_per_pair;
    const int64_t chunk = blockIdx.x - pair * a.wgs_per_pair;
    if (pair >= a.num_pairs) return;
    const int64_t src = a.block_pairs[2 * pair];
    const int64_t dst = a.block_pairs[2 * pair + 1];
    if (src < 0 || dst < 0 || src >= a.num_blocks || dst >= a.num_blocks || src == dst) return;
    const int64_t v0 = chunk * kVecsPerWG + threadIdx.x;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const cb_u32x4* s = static_cast<const cb_u32x4*>(c == 0 ? a.k_cache : a.v_cache) + src * a.block_vecs;
        cb_u32x4* d = static_cast<cb_u32x4*>(c == 0 ? a.k_cache : a.v_cache) + dst * a.block_vecs;
        cb_u32x4 r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t v = v0 + 256 * i;
            if (v < a.block_vecs) r[i] = __builtin_nontemporal_load(s + v);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t v = v0 + 256 * i;
            if (v < a.block_vecs) d[v] = r[i];
        }
    }
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
    const int64_t wgs = a.num_pairs * a.wgs_per_pair;
    if (wgs == 0) return hipSuccess;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    return launch(copy_blocks_kernel, dim3((unsigned)wgs), dim3(256), stream, a);
}

}  // namespace pa
