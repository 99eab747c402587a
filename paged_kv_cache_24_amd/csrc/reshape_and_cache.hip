// Cache write: store each new token's k and v rows in their pool slots.
//
// With the [num_blocks][16][kv_heads][head_dim] layout a token slot is one
// contiguous row of kv_heads * head_dim elements, so the write is a row copy
// from key[t] / value[t] to row slot_mapping[t] ("vLLM-Ascend 原理", §2.3 step
// 3 and §2.4 step 3).  Each lane moves 16-byte vectors; consecutive lanes
// cover consecutive bytes of a row, so loads and stores are fully coalesced.
#include "common.h"
#include "kernels.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per TPW tokens: the slot of each token is one scalar load, and
// the workgroup's threads stream the token's K and V rows (row_vecs 16-byte
// vectors each), so no thread divides a flat index.  Small writes (a decode
// step) take one token per workgroup for parallelism; large ones four.
template <int TPW>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ReshapeArgs a) {
    typedef const __attribute__((address_space(4))) int64_t cslot_t;
    const cslot_t* slots = (const cslot_t*)a.slot_mapping;   // read-only in this kernel: scalar loads
    const int64_t t0 = (int64_t)blockIdx.x * TPW;
    const int row_vecs = a.row_vecs;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        const int64_t t = t0 + k;
        if (t >= a.num_tokens) return;
        int64_t slot;
        if (a.slot_mapping) {
            slot = slots[t];
        } else {   // the newest token of sequence t, through its table row
            const int max_tokens = a.table_stride * a.block_size;
            const int n = min(a.seq_lens[t], max_tokens);
            if (n <= 0) continue;
            const int e = a.block_tables[t * (int64_t)a.table_stride + (n - 1) / a.block_size];
            slot = e < 0 ? -1 : (int64_t)e * a.block_size + (n - 1) % a.block_size;
        }
        if (slot < 0 || slot >= a.num_slots) continue;   // padding row or outside the pool
        const u32x4* ks = static_cast<const u32x4*>(a.key) + t * row_vecs;
        const u32x4* vs = static_cast<const u32x4*>(a.value) + t * row_vecs;
        u32x4* kd = static_cast<u32x4*>(a.k_cache) + slot * row_vecs;
        u32x4* vd = static_cast<u32x4*>(a.v_cache) + slot * row_vecs;
        for (int v = threadIdx.x; v < row_vecs; v += blockDim.x) {
            const u32x4 kx = __builtin_nontemporal_load(ks + v);   // the new rows are read exactly once
            const u32x4 vx = __builtin_nontemporal_load(vs + v);
            kd[v] = kx;
            vd[v] = vx;
        }
    }
}

hipError_t launch_reshape_and_cache(const ReshapeArgs& a, hipStream_t stream) {
    const bool big = a.num_tokens >= 2048;
    const int tpw = big ? 4 : 1;
    const int64_t wgs = (a.num_tokens + tpw - 1) / tpw;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    // a token row is kv_heads * head_dim / 8 vectors: 128 threads cover Hkv = 8 at D = 128
    const int threads = a.row_vecs >= 256 ? 256 : (a.row_vecs >= 128 ? 128 : 64);
    return big ? launch(reshape_and_cache_kernel<4>, dim3((unsigned)wgs), dim3(threads), stream, a)
               : launch(reshape_and_cache_kernel<1>, dim3((unsigned)wgs), dim3(threads), stream, a);
}

// ---------------------------------------------------------------------------
// Cache write into an FP8 (OCP E4M3) cache ("vLLM-Ascend 原理", §四 on KV-cache
// quantisation: k and v are quantised when the step writes them).  One row is
// one (token, kv head, K or V): head_dim elements sharing one float32 scale.
// D/8 consecutive lanes own the K rows and the V rows of two (token, kv head)
// pairs, 8 elements of each (four 16-byte loads in flight): a row maximum is a DPP max
// over those lanes, then
//     s = amax / 448 (s = 1 for an all-zero row),  code = e4m3(clamp(x / s))
// with the quotient rounded once in float32 and the conversion rounding to
// nearest even.  Codes leave as one 8-byte store per lane and row; the first
// lane of the group stores the row scales at [block][head][offset].
// ---------------------------------------------------------------------------
template <int DT, int D>
__device__ __forceinline__ uint2 quantize8(const u32x4& w, float& s_out) {
    constexpr int L = D / 8;
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
    // x / s correctly rounded, from the correctly rounded reciprocal r = 1/s (one
    // IEEE division per row): q = x r is within an ulp of x / s, its residual
    // x - q s is exact in an FMA, and q + residual * r rounded once is the
    // correctly rounded quotient (Markstein's correction; no over- or underflow
    // matters here: |x / s| <= 448, and quotients too small to be normal code
    // to a signed zero whatever their last bits).  The sign is x's, so that
    // -0 stays -0.
    const float r = 1.f / s;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float q = x[e] * r;
        const float q1 = __builtin_copysignf(fmaf(fmaf(-q, s, x[e]), r, q), x[e]);
        y[e] = fminf(fmaxf(q1, -448.f), 448.f);
    }
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
    s_out = s;
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// (token, kv head) pairs number below 2^31 (checked by the caller), so the
// index arithmetic is 32-bit.  Each lane group takes two consecutive pairs and
// issues all four row loads before quantising (a group past the end reloads
// its first pair and stores it once).
template <int DT, int D>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(ReshapeFp8Args a) {
    constexpr int L = D / 8;                       // lanes per (token, head)
    const int lane_in_row = threadIdx.x % L;
    const uint32_t hkv = (uint32_t)a.num_kv_heads;
    const uint32_t pairs = (uint32_t)a.num_tokens * hkv;
    const uint32_t per_grid = 2 * gridDim.x * (blockDim.x / L);
    for (uint32_t p0 = 2 * (blockIdx.x * (blockDim.x / L) + threadIdx.x / L); p0 < pairs; p0 += per_grid) {
        const bool two = p0 + 1 < pairs;
        const uint32_t p1 = two ? p0 + 1 : p0;
        const uint32_t t0 = p0 / hkv, t1 = p1 / hkv;
        const uint32_t h0 = p0 - t0 * hkv, h1 = p1 - t1 * hkv;
        const int64_t slot0 = a.slot_mapping[t0];
        const int64_t slot1 = a.slot_mapping[t1];
        const size_t s0 = (size_t)p0 * D + 8 * lane_in_row, s1 = (size_t)p1 * D + 8 * lane_in_row;
        const u32x4 wk0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.key) + s0));
        const u32x4 wv0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.value) + s0));
        const u32x4 wk1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.key) + s1));
        const u32x4 wv1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.value) + s1));
        float sk0, sv0, sk1, sv1;
        const uint2 ck0 = quantize8<DT, D>(wk0, sk0);
        const uint2 cv0 = quantize8<DT, D>(wv0, sv0);
        const uint2 ck1 = quantize8<DT, D>(wk1, sk1);
        const uint2 cv1 = quantize8<DT, D>(wv1, sv1);
        if (slot0 >= 0 && slot0 < a.num_slots) {
            const int64_t blk = slot0 / kBlockSize;
            const int off = (int)(slot0 - blk * kBlockSize);
            const int64_t dst = (slot0 * hkv + h0) * D + 8 * lane_in_row;
            *reinterpret_cast<uint2*>(a.k_cache + dst) = ck0;
            *reinterpret_cast<uint2*>(a.v_cache + dst) = cv0;
            if (lane_in_row == 0) {
                const int64_t si = (blk * hkv + h0) * kBlockSize + off;
                a.k_scales[si] = sk0;
                a.v_scales[si] = sv0;
            }
        }
        if (two && slot1 >= 0 && slot1 < a.num_slots) {
            const int64_t blk = slot1 / kBlockSize;
            const int off = (int)(slot1 - blk * kBlockSize);
            const int64_t dst = (slot1 * hkv + h1) * D + 8 * lane_in_row;
            *reinterpret_cast<uint2*>(a.k_cache + dst) = ck1;
            *reinterpret_cast<uint2*>(a.v_cache + dst) = cv1;
            if (lane_in_row == 0) {
                const int64_t si = (blk * hkv + h1) * kBlockSize + off;
                a.k_scales[si] = sk1;
                a.v_scales[si] = sv1;
            }
        }
    }
}

hipError_t launch_reshape_and_cache_fp8(const ReshapeFp8Args& a, hipStream_t stream) {
    const int64_t pairs = a.num_tokens * a.num_kv_heads;
    if (pairs > INT32_MAX) return hipErrorInvalidValue;
    const int pairs_per_wg = 2 * 256 / (a.head_dim / 8);
    const int64_t want = (pairs + pairs_per_wg - 1) / pairs_per_wg;
    const dim3 grid((unsigned)(want < 65536 ? want : 65536));
    if (a.dtype == kF16) {
        return a.head_dim == 128 ? launch(reshape_and_cache_fp8_kernel<kF16, 128>, grid, dim3(256), stream, a)
                                 : launch(reshape_and_cache_fp8_kernel<kF16, 64>, grid, dim3(256), stream, a);
    }
    return a.head_dim == 128 ? launch(reshape_and_cache_fp8_kernel<kBF16, 128>, grid, dim3(256), stream, a)
                             : launch(reshape_and_cache_fp8_kernel<kBF16, 64>, grid, dim3(256), stream, a);
}

}  // namespace pa
