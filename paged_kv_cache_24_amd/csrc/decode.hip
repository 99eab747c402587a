// Paged decode attention on the vector ALUs of gfx950.
//
// What is computed ("vLLM-Ascend 原理", §2.4 step 3): one new query per
// sequence attends to every cached token of that sequence; the K/V rows are
// read through the block table, one 16-token block at a time, and combined by
// an online softmax ("vLLM-Ascend 原理", §四 "ATB 算子": softmax statistics
// updated on chip, only the result written back; "vLLM 在 CANN 上的推理优化",
// section "CANN 上的 PagedAttention 算子": blocks are not contiguous, so they
// are merged block by block).  With GQA the q heads that share a kv head are
// handled by the same wave, so each K/V tile leaves HBM once.
//
// Work decomposition.  One wave (64 lanes) owns one item = (sequence, kv head,
// q-head chunk, partition of part_blocks blocks).  Partitions make the long
// sequences parallel enough for 256 CUs; their float32 states are merged by
// decode_merge_kernel (the max-rescaled sum of the online softmax).  A
// sequence that fits one partition is finished in place.
//
// Tile mapping.  A K (or V) tile of one block and one kv head is 16 rows of
// head_dim elements, each row contiguous.  Lane (r, c) with c = lane % (D/8)
// and r = lane / (D/8) loads the 16-byte column chunk c of rows r, r + 64/(D/8),
// ...; every wave-wide load instruction therefore reads whole 256-byte (D=128)
// or 128-byte (D=64) rows, fully coalesced.  The tile goes straight into the
// registers of the lanes that consume it, so no LDS round trip is needed:
// QK^T is a per-lane 8-wide dot product (v_dot2 on packed pairs) summed over
// the D/8 lanes of a row with DPP, and PV multiplies each lane's own V chunk
// by the probabilities of its own rows.  Each row group keeps its own
// (max, sum, acc) softmax state; the groups are merged once, at the end.
#include "common.h"
#include "kernels.h"

namespace pa {

template <int DT, int D, int HPW>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeArgs a) {
    constexpr int LPR = D / 8;              // lanes per token row
    constexpr int RPW = kWave / LPR;        // token rows per load instruction
    constexpr int TPL = kBlockSize / RPW;   // token rows per lane per block

    const int lane = threadIdx.x & (kWave - 1);
    const int r = lane / LPR;
    const int c = lane % LPR;

    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.head_chunks;
    const int64_t item = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
    if (item >= units * a.num_parts) return;
    const int part = (int)(item / units);
    int64_t u = item - (int64_t)part * units;
    const int hc = (int)(u % a.head_chunks);
    u /= a.head_chunks;
    const int g = (int)(u % a.num_kv_heads);
    const int b = (int)(u / a.num_kv_heads);

    const int max_tokens = a.max_blocks_per_seq * kBlockSize;
    int n = a.seq_lens[b];
    n = n < 0 ? 0 : (n > max_tokens ? max_tokens : n);
    const int nblk = (n + kBlockSize - 1) / kBlockSize;
    const int nparts = nblk <= a.part_blocks ? 1 : (nblk + a.part_blocks - 1) / a.part_blocks;
    if (part >= nparts) return;
    const int j0 = part * a.part_blocks;
    const int j1 = min(nblk, j0 + a.part_blocks);

    const int hbase = hc * HPW;
    const int hcount = min(HPW, a.group - hbase);
    const int64_t q_row0 = (int64_t)b * a.num_q_heads + (int64_t)g * a.group + hbase;

    uint4 qv[HPW];
    {
        const uint16_t* q = static_cast<const uint16_t*>(a.q) + q_row0 * D + 8 * c;
#pragma unroll
        for (int h = 0; h < HPW; ++h)
            qv[h] = h < hcount ? *reinterpret_cast<const uint4*>(q + (int64_t)h * D)
                               : make_uint4(0, 0, 0, 0);
    }

    float m[HPW], l[HPW], acc[HPW][8];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    const int64_t row_stride = (int64_t)a.num_kv_heads * D;   // elements between token rows
    const int64_t lane_off = (int64_t)g * D + 8 * c + (int64_t)r * row_stride;
    const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + lane_off;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + lane_off;
    const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
    const float cs = a.scale_log2;

    auto load = [&](int j, uint4 (&kr)[TPL], uint4 (&vr)[TPL]) -> bool {
        const int pb = table[j];
        const bool ok = pb >= 0 && (int64_t)pb < a.num_blocks;
        const int64_t off = (int64_t)(ok ? pb : 0) * kBlockSize * row_stride;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            kr[i] = *reinterpret_cast<const uint4*>(kbase + off + (int64_t)i * RPW * row_stride);
            vr[i] = *reinterpret_cast<const uint4*>(vbase + off + (int64_t)i * RPW * row_stride);
        }
        return ok;
    };

    auto process = [&](const uint4 (&kr)[TPL], const uint4 (&vr)[TPL], bool ok, int j) {
        float s[HPW][TPL];
#pragma unroll
        for (int h = 0; h < HPW; ++h)
#pragma unroll
            for (int i = 0; i < TPL; ++i) s[h][i] = group_sum<LPR>(dot8<DT>(qv[h], kr[i])) * cs;

        float vf[TPL][8];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vf[i][2 * e] = lo_to_f32<DT>(w[e]);
                vf[i][2 * e + 1] = hi_to_f32<DT>(w[e]);
            }
        }
        // rows past the sequence end (tail block) or in a bad block: score -inf,
        // value 0 (a select, so NaN bits there cannot leak into the sums)
        if (!(ok && (j + 1) * kBlockSize <= n)) {
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const bool valid = ok && (j * kBlockSize + i * RPW + r < n);
#pragma unroll
                for (int h = 0; h < HPW; ++h) s[h][i] = valid ? s[h][i] : -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) vf[i][e] = valid ? vf[i][e] : 0.f;
            }
        }
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            float mb = s[h][0];
#pragma unroll
            for (int i = 1; i < TPL; ++i) mb = fmaxf(mb, s[h][i]);
            const float mn = fmaxf(m[h], mb);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float alpha = fast_exp2(m[h] - mu);
            float p[TPL];
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                p[i] = fast_exp2(s[h][i] - mu);
                ps += p[i];
            }
            l[h] = fmaf(l[h], alpha, ps);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = acc[h][e] * alpha;
#pragma unroll
                for (int i = 0; i < TPL; ++i) x = fmaf(p[i], vf[i][e], x);
                acc[h][e] = x;
            }
            m[h] = mn;
        }
    };

    if (j0 < j1) {
        uint4 ka[TPL], va[TPL], kb[TPL], vb[TPL];
        bool oka = load(j0, ka, va);
        bool okb = false;
        for (int j = j0; j < j1; j += 2) {
            if (j + 1 < j1) okb = load(j + 1, kb, vb);
            process(ka, va, oka, j);
            if (j + 1 >= j1) break;
            if (j + 2 < j1) oka = load(j + 2, ka, va);
            process(kb, vb, okb, j + 1);
        }
    }

    // merge the row groups' states: rescale to the common max, then sum
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        float big = m[h];
#pragma unroll
        for (int off = LPR; off < kWave; off <<= 1) big = fmaxf(big, __shfl_xor(big, off));
        const float w = m[h] == -INFINITY ? 0.f : fast_exp2(m[h] - big);
        float lt = l[h] * w;
#pragma unroll
        for (int off = LPR; off < kWave; off <<= 1) lt += __shfl_xor(lt, off);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[h][e] * w;
#pragma unroll
            for (int off = LPR; off < kWave; off <<= 1) x += __shfl_xor(x, off);
            acc[h][e] = x;
        }
        m[h] = big;
        l[h] = lt;
    }

    if (r != 0) return;
    if (nparts == 1) {
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            if (h >= hcount) break;
            const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
            uint4 o;
            o.x = pack2<DT>(acc[h][0] * inv, acc[h][1] * inv);
            o.y = pack2<DT>(acc[h][2] * inv, acc[h][3] * inv);
            o.z = pack2<DT>(acc[h][4] * inv, acc[h][5] * inv);
            o.w = pack2<DT>(acc[h][6] * inv, acc[h][7] * inv);
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (q_row0 + h) * D + 8 * c) = o;
        }
    } else {
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            if (h >= hcount) break;
            const int64_t idx = (q_row0 + h) * a.num_parts + part;
            float4* dst = reinterpret_cast<float4*>(a.ws_acc + idx * D + 8 * c);
            dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
            dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
            if (c == 0) a.ws_ml[idx] = make_float2(m[h], l[h]);
        }
    }
}

// Combine the partition states of one (sequence, q head):
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p with M = max_p m_p.
template <int DT, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int EPL = D / kWave;   // output elements per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
    if (item >= (int64_t)a.num_seqs * a.num_q_heads) return;
    const int b = (int)(item / a.num_q_heads);

    const int max_tokens = a.max_blocks_per_seq * kBlockSize;
    int n = a.seq_lens[b];
    n = n < 0 ? 0 : (n > max_tokens ? max_tokens : n);
    const int nblk = (n + kBlockSize - 1) / kBlockSize;
    const int nparts = nblk <= a.part_blocks ? 1 : (nblk + a.part_blocks - 1) / a.part_blocks;
    if (nparts <= 1) return;   // finished by the partition kernel

    const int64_t base = item * a.num_parts;
    float big = -INFINITY;
    for (int i = 0; i < nparts; ++i) big = fmaxf(big, a.ws_ml[base + i].x);
    float den = 0.f;
    float num[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] = 0.f;
    for (int i = 0; i < nparts; ++i) {
        const float2 ml = a.ws_ml[base + i];
        const float w = ml.x == -INFINITY ? 0.f : fast_exp2(ml.x - big);
        den = fmaf(w, ml.y, den);
        const float* src = a.ws_acc + (base + i) * D + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) num[e] = fmaf(w, src[e], num[e]);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    uint16_t* dst = static_cast<uint16_t*>(a.out) + item * D + lane * EPL;
    if constexpr (EPL == 2) {
        *reinterpret_cast<uint32_t*>(dst) = pack2<DT>(num[0] * inv, num[1] * inv);
    } else {
        *dst = f32_to_bits<DT>(num[0] * inv);
    }
}

template <int DT, int D>
static hipError_t launch_partitions_d(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    switch (a.heads_per_wave) {
        case 1: hipLaunchKernelGGL((decode_partition_kernel<DT, D, 1>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_partition_kernel<DT, D, 2>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_partition_kernel<DT, D, 4>), grid, dim3(256), 0, s, a); break;
        case 8: hipLaunchKernelGGL((decode_partition_kernel<DT, D, 8>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t s) {
    const int64_t items = (int64_t)a.num_seqs * a.num_kv_heads * a.head_chunks * a.num_parts;
    if (items == 0) return hipSuccess;
    const int64_t wgs = (items + 3) / 4;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    if (a.dtype == kF16) {
        return a.head_dim == 128 ? launch_partitions_d<kF16, 128>(a, s, grid)
                                 : launch_partitions_d<kF16, 64>(a, s, grid);
    }
    return a.head_dim == 128 ? launch_partitions_d<kBF16, 128>(a, s, grid)
                             : launch_partitions_d<kBF16, 64>(a, s, grid);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s) {
    const int64_t items = (int64_t)a.num_seqs * a.num_q_heads;
    if (items == 0 || a.num_parts <= 1) return hipSuccess;
    const int64_t wgs = (items + 3) / 4;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    if (a.dtype == kF16) {
        if (a.head_dim == 128) hipLaunchKernelGGL((decode_merge_kernel<kF16, 128>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((decode_merge_kernel<kF16, 64>), grid, dim3(256), 0, s, a);
    } else {
        if (a.head_dim == 128) hipLaunchKernelGGL((decode_merge_kernel<kBF16, 128>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((decode_merge_kernel<kBF16, 64>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace pa
