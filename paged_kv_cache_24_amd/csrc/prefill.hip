// Causal chunked prefill over the paged KV cache, on gfx950 matrix cores.
//
// What is computed ("vLLM-Ascend 原理", §2.3 step 3 and §2.4 on chunked
// prefill): row i of sequence b sits at position ctx_b + i and attends, with
// a softmax, to keys 0 .. ctx_b + i of that sequence -- the context cached by
// earlier chunks plus this chunk's own tokens, all read through the block
// table.  The L x L score matrix is never stored: key tiles are streamed and
// merged with an online softmax, as fused attention kernels do
// ("vLLM-Ascend 原理", §2.3 step 3 and §四 "ATB 算子").
//
// Mapping.  One workgroup (4 waves) owns 128 query rows of one (sequence, kv
// head): 128/G positions times the G q heads that share the kv head, so every
// K/V tile is staged in LDS once for all of them.  Each wave owns 32 rows.
// For each 64-key tile:
//   S^T[key][row] = K[key][:] . Q[row][:]     (MFMA 16x16x32: A = K from LDS,
//                                              B = Q kept in registers)
//   online softmax per row: the C layout puts one row's keys in the four lanes
//   l, l^16, l^32, l^48, so the row max/sum is an in-lane reduction plus two
//   cross-lane steps;
//   O^T[d][row] += V^T[d][key] . P^T[key][row] (MFMA 16x16x32: B = P^T straight
//   from the softmax registers, A = V^T read from a transposed LDS copy).
// Working on the transposed products keeps each row's statistics in the lanes
// that own the row in both products, so no shuffle of the probabilities or
// of the rescale factors is needed.
#include "common.h"
#include "kernels.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
    if constexpr (DT == kF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
}

constexpr int kPD = 128;            // head_dim
constexpr int kKT = 64;             // keys per tile
constexpr int kRows = 128;          // query rows per workgroup
constexpr int kKRow = kPD + 8;      // LDS K row stride (elements): 272 bytes, staggers banks
constexpr int kVRow = kKT + 4;      // LDS V^T row stride (elements): 136 bytes

template <int DT, int G>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
    constexpr int P = kRows / G;    // positions per workgroup
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKT * kKRow];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kPD * kVRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int lr = lane & 15;       // row (or column) within a 16-wide MFMA tile
    const int lg = lane >> 4;       // lane group 0..3

    // heaviest tiles (last query positions, most keys) are dispatched first
    const int units = a.num_seqs * a.num_kv_heads;
    const int qtiles = (a.max_q_len + P - 1) / P;
    const int id = blockIdx.x;
    const int qtile = qtiles - 1 - id / units;
    const int unit = id % units;
    const int g = unit % a.num_kv_heads;
    const int b = unit / a.num_kv_heads;

    // the row range and context come from device memory: clamp them so a
    // malformed query_start_loc or ctx_lens can never send an access out of bounds
    const int64_t row0 = a.query_start_loc[b];
    const int64_t row1 = min((int64_t)a.query_start_loc[b + 1], a.num_tokens);
    if (row0 < 0 || row1 <= row0) return;
    const int L = (int)min(row1 - row0, (int64_t)a.max_q_len);
    const int max_keys = a.max_blocks_per_seq * kBlockSize;
    const int ctx = min(max(a.ctx_lens[b], 0), max_keys);
    const int pos0 = qtile * P;
    if (qtile < 0 || pos0 >= L) return;
    const int pos_end = min(L, pos0 + P);
    const int n_keys = min(ctx + pos_end, max_keys);
    const int ntiles = (n_keys + kKT - 1) / kKT;
    const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
    const int64_t row_stride = (int64_t)a.num_kv_heads * kPD;

    // ---- this lane's two query rows (one per 16-row tile) and their Q^T fragments
    uint4 qf[2][4];
    int qpos[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int rho = wave * 32 + nt * 16 + lr;
        const int pos = pos0 + rho / G;
        qpos[nt] = ctx + pos;
        const bool ok = pos < L;
        const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                              ((int64_t)(row0 + (ok ? pos : 0)) * a.num_q_heads + g * G + rho % G) * kPD +
                              8 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[nt][kk] = ok ? *reinterpret_cast<const uint4*>(src + 32 * kk) : make_uint4(0, 0, 0, 0);
    }
    const int wave_pos_lo = pos0 + (wave * 32) / G;
    const int wave_pos_hi = min(pos_end - 1, pos0 + (wave * 32 + 31) / G);
    const bool wave_live = wave_pos_lo < pos_end;
    const int wave_q_lo = ctx + wave_pos_lo;
    const int wave_q_hi = ctx + wave_pos_hi;

    f32x4_t o[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) o[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m[2] = {-INFINITY, -INFINITY};
    float lsum[2] = {0.f, 0.f};   // this lane's share of the row sums
    const float cs = a.scale_log2;

    // ---- K/V tile staging: thread t moves 16-byte chunk (t % 16) of key rows t/16 + 16 i
    const int ck = tid & 15;
    auto load_tile = [&](int t, uint4 (&gk)[4], uint4 (&gv)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = t * kKT + (tid >> 4) + 16 * i;
            int pb = -1;
            if (key < n_keys && key < max_keys) pb = table[key / kBlockSize];
            if (pb >= 0 && (int64_t)pb < a.num_blocks) {
                const int64_t off = ((int64_t)pb * kBlockSize + key % kBlockSize) * row_stride +
                                    (int64_t)g * kPD + 8 * ck;
                gk[i] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_cache) + off);
                gv[i] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v_cache) + off);
            } else {
                gk[i] = make_uint4(0, 0, 0, 0);   // past the sequence: zeros, never NaN
                gv[i] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_tile = [&](int buf, const uint4 (&gk)[4], const uint4 (&gv)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kr = (tid >> 4) + 16 * i;
            *reinterpret_cast<uint4*>(&lds_k[buf][kr * kKRow + 8 * ck]) = gk[i];
            const uint32_t w[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lds_v[buf][(8 * ck + 2 * e) * kVRow + kr] = (uint16_t)(w[e] & 0xffffu);
                lds_v[buf][(8 * ck + 2 * e + 1) * kVRow + kr] = (uint16_t)(w[e] >> 16);
            }
        }
    };

    uint4 gk[4], gv[4];
    load_tile(0, gk, gv);
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        store_tile(buf, gk, gv);
        __syncthreads();
        if (t + 1 < ntiles) load_tile(t + 1, gk, gv);
        const int k0 = t * kKT;
        if (!wave_live || k0 > wave_q_hi) continue;   // every key of the tile is in this wave's future

        // ---- S^T = K Q^T for 64 keys x 32 rows
        f32x4_t s[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) s[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const uint4 ka = *reinterpret_cast<const uint4*>(
                    &lds_k[buf][(16 * mt + lr) * kKRow + 32 * kk + 8 * lg]);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) s[mt][nt] = mfma16x16x32<DT>(ka, qf[nt][kk], s[mt][nt]);
            }
        }

        // ---- causal mask (select) and online softmax, per row
        const bool diag = k0 + kKT - 1 > wave_q_lo;
        uint4 pb[2][2];   // P^T fragments [key chunk][row tile]
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float x[4][4];
            float mb = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = s[mt][nt][i] * cs;
                    if (diag) {
                        const int key = k0 + 16 * mt + 4 * lg + i;
                        v = key > qpos[nt] ? -INFINITY : v;
                    }
                    x[mt][i] = v;
                    mb = fmaxf(mb, v);
                }
            mb = fmaxf(mb, __shfl_xor(mb, 16));
            mb = fmaxf(mb, __shfl_xor(mb, 32));
            const float mn = fmaxf(m[nt], mb);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float alpha = fast_exp2(m[nt] - mu);
            m[nt] = mn;
            float ps = 0.f;
            float p[4][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[mt][i] = fast_exp2(x[mt][i] - mu);
                    ps += p[mt][i];
                }
            lsum[nt] = fmaf(lsum[nt], alpha, ps);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) o[mt][nt] *= alpha;
            // key slot 8*lg + i <-> key 32*kc + 4*lg + i; slot 8*lg + 4 + i <-> key 32*kc + 16 + 4*lg + i
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                pb[kc][nt].x = pack2<DT>(p[2 * kc][0], p[2 * kc][1]);
                pb[kc][nt].y = pack2<DT>(p[2 * kc][2], p[2 * kc][3]);
                pb[kc][nt].z = pack2<DT>(p[2 * kc + 1][0], p[2 * kc + 1][1]);
                pb[kc][nt].w = pack2<DT>(p[2 * kc + 1][2], p[2 * kc + 1][3]);
            }
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const uint16_t* vrow = &lds_v[buf][(16 * mt + lr) * kVRow + 32 * kc + 4 * lg];
                const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
                const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
                const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) o[mt][nt] = mfma16x16x32<DT>(va, pb[kc][nt], o[mt][nt]);
            }
        }
    }

    if (!wave_live) return;
    // ---- epilogue: full row sums, normalise, store rows that exist
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        float l = lsum[nt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int rho = wave * 32 + nt * 16 + lr;
        const int pos = pos0 + rho / G;
        if (pos >= L) continue;
        uint16_t* dst = static_cast<uint16_t*>(a.out) +
                        ((int64_t)(row0 + pos) * a.num_q_heads + g * G + rho % G) * kPD + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            uint2 w;
            w.x = pack2<DT>(o[mt][nt][0] * inv, o[mt][nt][1] * inv);
            w.y = pack2<DT>(o[mt][nt][2] * inv, o[mt][nt][3] * inv);
            *reinterpret_cast<uint2*>(dst + 16 * mt) = w;
        }
    }
}

template <int DT>
static void launch_prefill_g(const PrefillArgs& a, hipStream_t s, dim3 grid) {
    switch (a.group) {
        case 1: hipLaunchKernelGGL((prefill_kernel<DT, 1>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<DT, 2>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<DT, 4>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((prefill_kernel<DT, 8>), grid, dim3(256), 0, s, a); break;
    }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    const int positions = kRows / a.group;
    const int64_t qtiles = (a.max_q_len + positions - 1) / positions;
    const int64_t wgs = qtiles * a.num_seqs * a.num_kv_heads;
    if (wgs == 0) return hipSuccess;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    if (a.dtype == kF16) launch_prefill_g<kF16>(a, s, grid);
    else launch_prefill_g<kBF16>(a, s, grid);
    return hipGetLastError();
}

}  // namespace pa
