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

// ---------------------------------------------------------------------------
// Cache write into an FP8 (OCP E4M3) cache ("vLLM-Ascend 原理", §四 on KV-cache
// quantisation: k and v are quantised when the step writes them).  One row is
// one (token, kv head, K or V): head_dim elements sharing one float32 scale.
// D/8 consecutive lanes own a row, 8 elements each (one 16-byte load): the row
// maximum is a DPP max over those lanes, then
//     s = amax / 448 (s = 1 for an all-zero row),  code = e4m3(clamp(x / s))
// with the quotient rounded once in float32 and the conversion rounding to
// nearest even.  Codes leave as one 8-byte store per lane; the first lane of
// the row stores the scale at [block][head][offset].
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(ReshapeFp8Args a) {
    constexpr int L = D / 8;                       // lanes per row
    const int lane_in_row = threadIdx.x % L;
    const int64_t rows = a.num_tokens * 2 * a.num_kv_heads;
    const int64_t rows_per_grid = (int64_t)gridDim.x * (blockDim.x / L);
    for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / L) + threadIdx.x / L; row < rows;
         row += rows_per_grid) {
        // row = (token * 2 + is_v) * kv_heads + head: consecutive rows of a
        // token are consecutive in memory, so a wave reads whole token rows
        const int64_t th = row / a.num_kv_heads;
        const int h = (int)(row - th * a.num_kv_heads);
        const int64_t t = th >> 1;
        const bool is_v = th & 1;
        const int64_t slot = a.slot_mapping[t];
        if (slot < 0 || slot >= a.num_slots) continue;   // padding row or outside the pool (whole row)
        const uint16_t* src = static_cast<const uint16_t*>(is_v ? a.value : a.key) +
                              (t * a.num_kv_heads + h) * D + 8 * lane_in_row;
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = lo_to_f32<DT>(w[e]);
            x[2 * e + 1] = hi_to_f32<DT>(w[e]);
        }
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
        amax = group_max<L>(amax);
        const float s = amax > 0.f ? amax / 448.f : 1.f;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(x[e] / s, -448.f), 448.f);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
        const int64_t blk = slot / kBlockSize;
        const int off = (int)(slot - blk * kBlockSize);
        uint8_t* cache = is_v ? a.v_cache : a.k_cache;
        *reinterpret_cast<uint2*>(cache + (slot * a.num_kv_heads + h) * D + 8 * lane_in_row) =
            make_uint2((uint32_t)lo, (uint32_t)hi);
        if (lane_in_row == 0)
            (is_v ? a.v_scales : a.k_scales)[(blk * a.num_kv_heads + h) * kBlockSize + off] = s;
    }
}

hipError_t launch_reshape_and_cache_fp8(const ReshapeFp8Args& a, hipStream_t stream) {
    const int64_t rows = a.num_tokens * 2 * a.num_kv_heads;
    const int rows_per_wg = 256 / (a.head_dim / 8);
    const int64_t want = (rows + rows_per_wg - 1) / rows_per_wg;
    const dim3 grid((unsigned)(want < 65536 ? want : 65536));
    if (a.dtype == kF16) {
        if (a.head_dim == 128) hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<kF16, 128>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<kF16, 64>), grid, dim3(256), 0, stream, a);
    } else {
        if (a.head_dim == 128) hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<kBF16, 128>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<kBF16, 64>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace pa
