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

// Blocks j0 .. j1-1 of unit (b, g, hc) -- sequence b, kv head g, q-head chunk
// hc, n tokens -- for one wave: the online softmax over them, then the final
// output (final_out) or the partial state, in slot qrow * num_parts + slot
// (fixed partitions: slot = partition) or slot * state_heads + h (balanced
// split, slot from balanced_walk).
// MQ: several queries per sequence (see decode_gqa_kernel); the columns of a
// kv head are (query, q head) pairs and each sees keys up to its own position.
template <int DT, int D, int HPW, bool NT, bool MQ, bool BAL>
__device__ __forceinline__ void vector_segment(const DecodeArgs& a, int b, int g, int hc, int n,
                                               int j0, int j1, bool final_out, int64_t slot) {
    constexpr int LPR = D / 8;              // lanes per token row
    constexpr int RPW = kWave / LPR;        // token rows per load instruction
    constexpr int TPL = kBlockSize / RPW;   // token rows per lane per block

    const int lane = threadIdx.x & (kWave - 1);
    const int r = lane / LPR;
    const int c = lane % LPR;

    const int hbase = hc * HPW;
    const int hcount = min(HPW, (MQ ? a.cols : a.group) - hbase);
    const int64_t q_row0 = (int64_t)b * a.num_q_heads + (int64_t)g * a.group + hbase;
    // the step's cache write (new_k set, single query): the newest token, at
    // position n - 1, is not read from the pool (nm = n - 1 keys come from it);
    // the wave whose segment ends the sequence scores it from new_k / new_v in one
    // more step and, for the first head chunk, stores it to its slot
    const bool fused = !MQ && a.new_k != nullptr && n > 0;
    int nm = fused ? n - 1 : n;
    // q / out row of column h; with MQ also the keys it may see
    int64_t qrow[HPW];
    int lim[HPW];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        if constexpr (MQ) {
            const int col = hbase + h;
            const int jq = col / a.group;
            qrow[h] = ((int64_t)b * a.q_per_seq + jq) * a.num_q_heads + (int64_t)g * a.group + col % a.group;
            lim[h] = n - a.q_per_seq + 1 + jq;
        } else {
            qrow[h] = q_row0 + h;
            lim[h] = nm;
        }
    }
    int lim_min = MQ ? n - a.q_per_seq + 1 : nm;   // keys every column sees

    uint4 qv[HPW];
    {
        const uint16_t* q = static_cast<const uint16_t*>(a.q) + 8 * c;
#pragma unroll
        for (int h = 0; h < HPW; ++h)
            qv[h] = h < hcount ? *reinterpret_cast<const uint4*>(q + qrow[h] * D)
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
    const int32_t* table = a.block_tables + (int64_t)b * a.table_stride;
    const float cs = a.scale_log2;

    auto load = [&](int j, uint4 (&kr)[TPL], uint4 (&vr)[TPL]) -> bool {
        const int pb = sub_block(table[j >> a.block_shift], j, a.block_shift);
        const bool ok = pb >= 0 && (int64_t)pb < a.num_blocks;
        const int64_t off = (int64_t)(ok ? pb : 0) * kBlockSize * row_stride;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            kr[i] = load_kv<NT>(kbase + off + (int64_t)i * RPW * row_stride);
            vr[i] = load_kv<NT>(vbase + off + (int64_t)i * RPW * row_stride);
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
        // value 0 (a select, so NaN bits there cannot leak into the sums); with
        // MQ a column also masks the keys past its own position
        if (!(ok && (j + 1) * kBlockSize <= lim_min)) {
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int tok = j * kBlockSize + i * RPW + r;
                const bool valid = ok && (tok < nm);
#pragma unroll
                for (int h = 0; h < HPW; ++h) s[h][i] = (ok && tok < lim[h]) ? s[h][i] : -INFINITY;
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

    // three register buffers: while one block is computed, the next two are in flight
    if (j0 < j1) {
        uint4 ka[TPL], va[TPL], kb[TPL], vb[TPL], kc[TPL], vc[TPL];
        bool oka = load(j0, ka, va);
        bool okb = false, okc = false;
        if (j0 + 1 < j1) okb = load(j0 + 1, kb, vb);
        for (int j = j0; j < j1; j += 3) {
            if (j + 2 < j1) okc = load(j + 2, kc, vc);
            process(ka, va, oka, j);
            if (j + 1 >= j1) break;
            if (j + 3 < j1) oka = load(j + 3, ka, va);
            process(kb, vb, okb, j + 1);
            if (j + 2 >= j1) break;
            if (j + 4 < j1) okb = load(j + 4, kb, vb);
            process(kc, vc, okc, j + 2);
        }
    }
    if (fused && j1 == ceil_blocks(n)) {   // the newest token: row 0 of one more step
        const int64_t new_off = ((int64_t)b * a.num_kv_heads + g) * D + 8 * c;
        uint4 kx[TPL], vx[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) kx[i] = vx[i] = make_uint4(0, 0, 0, 0);
        if (r == 0) {
            kx[0] = load_kv<true>(static_cast<const uint16_t*>(a.new_k) + new_off);
            vx[0] = load_kv<true>(static_cast<const uint16_t*>(a.new_v) + new_off);
        }
        // a block outside the pool: the token is masked and not written, as the
        // separate cache write would skip its slot and the decode the block
        const int jn = (n - 1) / kBlockSize;
        const int pb = sub_block(table[jn >> a.block_shift], jn, a.block_shift);
        const bool okn = pb >= 0 && (int64_t)pb < a.num_blocks;
        nm = 1;
        lim_min = 1;
#pragma unroll
        for (int h = 0; h < HPW; ++h) lim[h] = 1;
        process(kx, vx, okn, 0);
        if (hc == 0 && r == 0 && okn) {
            const int64_t dst = ((int64_t)pb * kBlockSize + (n - 1) % kBlockSize) * row_stride;
            // the pools are written here only (the step's cache write)
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(const_cast<void*>(a.k_cache)) + lane_off + dst) = kx[0];
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(const_cast<void*>(a.v_cache)) + lane_off + dst) = vx[0];
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
    if (final_out) {
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            if (h >= hcount) break;
            const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
            uint4 o;
            o.x = pack2<DT>(acc[h][0] * inv, acc[h][1] * inv);
            o.y = pack2<DT>(acc[h][2] * inv, acc[h][3] * inv);
            o.z = pack2<DT>(acc[h][4] * inv, acc[h][5] * inv);
            o.w = pack2<DT>(acc[h][6] * inv, acc[h][7] * inv);
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + qrow[h] * D + 8 * c) = o;
        }
    } else {
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            if (h >= hcount) break;
            const int64_t idx = BAL ? slot * a.state_heads + h : qrow[h] * a.num_parts + slot;
            float4* dst = reinterpret_cast<float4*>(a.ws_acc + idx * D + 8 * c);
            dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
            dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
            if (c == 0) a.ws_ml[idx] = make_float2(m[h], l[h]);
        }
    }
}

// Fixed partitions: one wave per (partition, unit) item.
template <int DT, int D, int HPW, bool NT, bool MQ>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeArgs a) {
    DecodeItem it;
    if (!decode_item<NT>(a, uniform(threadIdx.x >> 6), it)) return;
    const int n = seq_tokens(a, it.b);
    const int nblk = ceil_blocks(n);
    const int nparts = nblk <= a.part_blocks ? 1 : (nblk + a.part_blocks - 1) / a.part_blocks;
    if (it.part >= nparts) return;
    const int j0 = it.part * a.part_blocks;
    vector_segment<DT, D, HPW, NT, MQ, false>(a, it.b, it.g, it.hc, n, j0, min(nblk, j0 + a.part_blocks),
                                              nparts == 1, it.part);
}

// Balanced split: each wave an equal stretch of the stream of all units' blocks.
template <int DT, int D, int HPW, bool NT>
__global__ __launch_bounds__(256) void decode_balanced_kernel(DecodeArgs a) {
    balanced_walk<NT>(a, uniform(threadIdx.x >> 6),
                      [&](int b, int g, int hc, int n, int j0, int j1, bool whole, int64_t slot) {
                          vector_segment<DT, D, HPW, NT, false, true>(a, b, g, hc, n, j0, j1, whole, slot);
                      });
}

// ---------------------------------------------------------------------------
// GQA decode (head_dim 128, 3..16 q heads per kv head): both products on
// matrix cores.
//
// With G q heads sharing a kv head, one block's S = K Q^T ([16 tokens x 128] .
// [128 x G]) and O += P V ([G x 16] . [16 x 128]) are real small contractions
// shared by G heads; on the vector ALUs their cost grows with G until it, not
// HBM, bounds the kernel (measured on the 64K-token long-context workload, 8 q
// heads per kv head: the vector kernel 0.666 ms, 40% of HBM peak; this one
// 0.327 ms, 80%).  Here:
//   S^T tile  = MFMA 16x16x32 x 4:  A = K rows (lane l: token pi(l%16),
//               elements 32*kk + 8*(l/16) .. +8), B = Q^T (lane l: head l%16);
//               pi(m) = 4*(m%4) + m/4, so lane l receives the scores of
//               tokens 4*i + l/16 (i = 0..3) for head l%16;
//   O^T      += MFMA 16x16x16 x 8:  A = V^T (16 elements of head_dim x the 16
//               tokens), B = P^T -- exactly the probabilities lane l already
//               holds, in the same token order, so they never move.
// V^T comes from a per-wave LDS copy of the V tile: each lane writes its
// row-coalesced 16-byte chunks, and ds_read_b64_tr_b16 returns the transposed
// 4 x 16-bit fragments in one instruction per 16 columns.  Softmax state is
// per head (lanes l, l^16, l^32, l^48 share it), so the rescale of O^T, whose
// column is also the head, stays in-lane.
// ---------------------------------------------------------------------------
typedef __bf16 dbf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 dbf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 df16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 df16x4_t __attribute__((ext_vector_type(4)));
typedef float df32x4_t __attribute__((ext_vector_type(4)));
typedef short ds16x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ df32x4_t mfma_16x16x32(const uint4& a, const uint4& b, df32x4_t c) {
    if constexpr (DT == kF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(df16x8_t, a),
                                                      __builtin_bit_cast(df16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dbf16x8_t, a),
                                                       __builtin_bit_cast(dbf16x8_t, b), c, 0, 0, 0);
    }
}
template <int DT>
__device__ __forceinline__ df32x4_t mfma_16x16x16(const uint2& a, const uint2& b, df32x4_t c) {
    if constexpr (DT == kF16) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(df16x4_t, a),
                                                     __builtin_bit_cast(df16x4_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(dbf16x4_t, a),
                                                         __builtin_bit_cast(dbf16x4_t, b), c, 0, 0, 0);
    }
}

constexpr int kVRow = 144;   // LDS row stride of the V tile (elements): 288 B staggers banks

// MQ: several queries per sequence, as speculative decoding verifies its draft
// tokens ("vLLM-Ascend 原理", §四 on speculative decoding: all draft tokens are
// checked in one pass).  Column c of the kv head is query c / group and q head
// c % group; query jq sits at position n - Q + jq and sees keys up to it, so
// each K/V tile is read once for every query of the sequence.
//
// gqa_segment: blocks j0 .. j1-1 of unit (b, g, hc) for one wave, `vt` its V
// tile in LDS; the final output (final_out) or the partial state of column lr
// in slot my_row * num_parts + slot (fixed partitions) or
// slot * state_heads + lr (balanced split).
template <int DT, bool NT, bool MQ, bool BAL>
__device__ __forceinline__ void gqa_segment(const DecodeArgs& a, uint16_t* vt, int b, int g, int hc, int n,
                                            int j0, int j1, bool final_out, int64_t slot) {
    constexpr int D = 128;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;    // MFMA column = q head; V column chunk; V^T row
    const int lg = lane >> 4;    // token group: tokens 4*i + lg of each block
    const int hcount = min(16, (MQ ? a.cols : a.group) - hc * 16);
    const bool head_live = lr < hcount;
    // q / out row of this lane's column, and (MQ) the keys the column may see
    int64_t my_row;
    int lim;
    if constexpr (MQ) {
        const int col = hc * 16 + (head_live ? lr : 0);
        const int jq = col / a.group;
        my_row = ((int64_t)b * a.q_per_seq + jq) * a.num_q_heads + (int64_t)g * a.group + col % a.group;
        lim = n - a.q_per_seq + 1 + jq;
    } else {
        my_row = (int64_t)b * a.num_q_heads + (int64_t)g * a.group + hc * 16 + (head_live ? lr : 0);
        lim = n;
    }

    uint4 qf[4];
    {
        const uint16_t* q = static_cast<const uint16_t*>(a.q) + my_row * D + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[kk] = head_live ? *reinterpret_cast<const uint4*>(q + 32 * kk) : make_uint4(0, 0, 0, 0);
    }

    float m = -INFINITY;   // running max of head lr (same in lanes l, l^16, l^32, l^48)
    float l = 0.f;         // this lane's share of the running sum
    df32x4_t o[8];         // O^T: lane holds elements 16*mt + 4*lg + i of head lr
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = df32x4_t{0.f, 0.f, 0.f, 0.f};

    const int64_t row_stride = (int64_t)a.num_kv_heads * D;
    const int tk = (lr & 3) * 4 + (lr >> 2);
    const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)g * D + 8 * lg +
                            (int64_t)tk * row_stride;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + (int64_t)g * D + 8 * lr +
                            (int64_t)lg * row_stride;
    const int32_t* table = a.block_tables + (int64_t)b * a.table_stride;
    const float cs = a.scale_log2;
    // transposed-read address of this lane: row 4*(lr/4) + lg, column 4*(lr%4) (+16 per tile)
    const uint16_t* vtr = vt + (4 * (lr >> 2) + lg) * kVRow + 4 * (lr & 3);
    // the step's cache write (new_k set, single query): as in vector_segment, the
    // newest token is left out of the pool's keys (nm = n - 1) and scored from
    // new_k / new_v in one more step by the wave whose segment ends the sequence
    const bool fused = !MQ && a.new_k != nullptr && n > 0;
    int nm = fused ? n - 1 : n;

    auto load = [&](int j, uint4 (&kr)[4], uint4 (&vr)[4]) -> bool {
        const int pb = sub_block(table[j >> a.block_shift], j, a.block_shift);
        const bool ok = pb >= 0 && (int64_t)pb < a.num_blocks;
        const int64_t off = (int64_t)(ok ? pb : 0) * kBlockSize * row_stride;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kr[i] = load_kv<NT>(kbase + off + 32 * i);
            vr[i] = load_kv<NT>(vbase + off + (int64_t)4 * i * row_stride);
        }
        return ok;
    };

    auto process = [&](const uint4 (&kr)[4], const uint4 (&vr)[4], bool ok, int j) {
        df32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) sacc = mfma_16x16x32<DT>(kr[kk], qf[kk], sacc);
        const bool full = ok && (j + 1) * kBlockSize <= nm;
        bool valid[4];
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            valid[i] = full || (ok && (j * kBlockSize + 4 * i + lg < nm));
            // MQ: the score of column lr also ends at the column's own position
            const bool seen = MQ ? (ok && j * kBlockSize + 4 * i + lg < lim) : valid[i];
            x[i] = seen ? sacc[i] * cs : -INFINITY;
        }
        float mb = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]),
                                                 __builtin_elementwise_maximum(x[2], x[3]));
        mb = xor32_max(xor16_max(mb));   // lanes l, l^16, l^32, l^48: VALU lane swaps
        // raise the running max only when this block beats it by more than 2^8:
        // otherwise keep it (p <= 256, exact algebra) and skip the rescale of O^T
        const bool raise = mb > m + 8.f;   // also true on the first live block
        const float mn = raise ? mb : m;
        if (__any(raise)) {
            const float alpha = raise ? fast_exp2(m - mn) : 1.f;   // exp2(-inf) = 0
            l *= alpha;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
        }
        m = mn;
        const float mu = mn == -INFINITY ? 0.f : mn;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - mu);
        // P^T enters the PV product as 16-bit values; the row sum adds those same
        // rounded values, so the weights that multiply V sum to exactly l
        uint2 pb;
        pb.x = pack2<DT>(p[0], p[1]);
        pb.y = pack2<DT>(p[2], p[3]);
        l = dot2<DT>(pb.y, kOnes2<DT>, dot2<DT>(pb.x, kOnes2<DT>, l));
        // V tile to LDS, rows past the sequence end as zeros (MFMA would turn 0 x NaN into NaN)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(vt + (4 * i + lg) * kVRow + 8 * lr) =
                valid[i] ? vr[i] : make_uint4(0, 0, 0, 0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const ds16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (ds16x4_t __attribute__((address_space(3)))*)(vtr + 16 * mt));
            o[mt] = mfma_16x16x16<DT>(__builtin_bit_cast(uint2, va), pb, o[mt]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    if (j0 < j1) {
        uint4 kc[4], vc[4];
        bool okc = load(j0, kc, vc);
        for (int j = j0; j < j1; ++j) {
            uint4 kn[4], vn[4];
            bool okn = false;
            if (j + 1 < j1) okn = load(j + 1, kn, vn);   // next block in flight
            process(kc, vc, okc, j);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kc[i] = kn[i];
                vc[i] = vn[i];
            }
            okc = okn;
        }
    }
    if (fused && j1 == ceil_blocks(n)) {   // the newest token: key 0 of one more step
        const int64_t new_row = ((int64_t)b * a.num_kv_heads + g) * D;
        uint4 kx[4], vx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kx[i] = vx[i] = make_uint4(0, 0, 0, 0);
        if (tk == 0) {   // K row 0: lanes lr = 0, elements 8*lg + 32*i
#pragma unroll
            for (int i = 0; i < 4; ++i)
                kx[i] = load_kv<true>(static_cast<const uint16_t*>(a.new_k) + new_row + 8 * lg + 32 * i);
        }
        if (lg == 0) vx[0] = load_kv<true>(static_cast<const uint16_t*>(a.new_v) + new_row + 8 * lr);   // V row 0
        // a block outside the pool: the token is masked and not written (as in vector_segment)
        const int jn = (n - 1) / kBlockSize;
        const int pb = sub_block(table[jn >> a.block_shift], jn, a.block_shift);
        const bool okn = pb >= 0 && (int64_t)pb < a.num_blocks;
        nm = 1;
        process(kx, vx, okn, 0);
        if (hc == 0 && okn) {
            // the pools are written here only (the step's cache write)
            const int64_t dst = ((int64_t)pb * kBlockSize + (n - 1) % kBlockSize) * row_stride + (int64_t)g * D;
            uint16_t* kp = static_cast<uint16_t*>(const_cast<void*>(a.k_cache)) + dst;
            uint16_t* vp = static_cast<uint16_t*>(const_cast<void*>(a.v_cache)) + dst;
            if (tk == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(kp + 8 * lg + 32 * i) = kx[i];
            }
            if (lg == 0) *reinterpret_cast<uint4*>(vp + 8 * lr) = vx[0];
        }
    }

    const float lt = xor32_sum(xor16_sum(l));
    if (!head_live) return;
    if (final_out) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        uint16_t* dst = static_cast<uint16_t*>(a.out) + my_row * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            uint2 w;
            w.x = pack2<DT>(o[mt][0] * inv, o[mt][1] * inv);
            w.y = pack2<DT>(o[mt][2] * inv, o[mt][3] * inv);
            *reinterpret_cast<uint2*>(dst + 16 * mt) = w;
        }
    } else {
        const int64_t idx = BAL ? slot * a.state_heads + lr : my_row * a.num_parts + slot;
        float* dst = a.ws_acc + idx * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            *reinterpret_cast<float4*>(dst + 16 * mt) = make_float4(o[mt][0], o[mt][1], o[mt][2], o[mt][3]);
        if (lg == 0) a.ws_ml[idx] = make_float2(m, lt);
    }
}

template <int DT, bool NT, bool MQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void decode_gqa_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t vlds[4][kBlockSize * kVRow];
    const int wave = uniform(threadIdx.x >> 6);
    DecodeItem it;
    if (!decode_item<NT>(a, wave, it)) return;
    const int n = seq_tokens(a, it.b);
    const int nblk = ceil_blocks(n);
    const int nparts = nblk <= a.part_blocks ? 1 : (nblk + a.part_blocks - 1) / a.part_blocks;
    if (it.part >= nparts) return;
    const int j0 = it.part * a.part_blocks;
    gqa_segment<DT, NT, MQ, false>(a, vlds[wave], it.b, it.g, it.hc, n, j0, min(nblk, j0 + a.part_blocks),
                                   nparts == 1, it.part);
}

// MQ: several queries per sequence (their (query, head) columns share each block)
template <int DT, bool NT, bool MQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void decode_gqa_balanced_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t vlds[4][kBlockSize * kVRow];
    const int wave = uniform(threadIdx.x >> 6);
    balanced_walk<NT>(a, wave, [&](int b, int g, int hc, int n, int j0, int j1, bool whole, int64_t slot) {
        gqa_segment<DT, NT, MQ, true>(a, vlds[wave], b, g, hc, n, j0, j1, whole, slot);
    });
}

// ---------------------------------------------------------------------------
// Sequence groups (PA_DECODE_SHARED_PREFIX).  Sequences that share a prefix
// point at the same physical blocks ("vLLM-Ascend 原理", §2.1; "vLLM学习整理",
// §三 on prefix caching).  With G q heads per kv head a matrix-core wave has 16
// columns but fills G of them; here one wave carries the heads of S = 16 / G
// consecutive sequences, a group (column c: member c / G, head c % G).  The
// group's leading blocks, up to the first block at which fewer than two
// members are still in play or those in play name different blocks, are its
// shared blocks: each is read once and scored for every member still in play.
//
// The balanced split runs over a stream of owners, group after group: the
// group's cp shared blocks, then each member's blocks past them.  A stretch's
// segment of a shared run scores all 16 columns; a segment of a member's own
// blocks scores that member's G columns (the others see -inf).  Slots stay
// unique as in the one-sequence split (owners appear in stream order): a
// member's segment writes its G heads' states at ((b + stretch) * Hkv + g) * G
// + head, a shared segment its 16 columns' at shared_base + ((group + stretch)
// * Hkv + g) * 16 + column.  A row is finished in place when one segment saw
// all of its blocks.

// The plan: one wave per group finds the shared run cp of its members' tables
// (lane i tests block base + i; the scan ends by the longest member's last
// block, where no member is in play) and writes the group's owner counts.
__global__ __launch_bounds__(256) void decode_group_plan_kernel(DecodeArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int S = a.seqs_per_wave;
    const int64_t grp = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
    if (grp * S >= a.num_seqs) return;
    const int b0 = (int)grp * S;
    int nb[kMaxGroupSeqs];
#pragma unroll
    for (int s = 0; s < kMaxGroupSeqs; ++s) nb[s] = s < S && b0 + s < a.num_seqs ? ceil_blocks(seq_tokens(a, b0 + s)) : 0;
    int cp = 0;
    for (int base = 0;; base += kWave) {
        const int j = base + lane;
        // every member row's entry j is inside its row (j < max_blocks_per_seq): the
        // loads need not wait for the lengths
        int e[kMaxGroupSeqs];
#pragma unroll
        for (int s = 0; s < kMaxGroupSeqs; ++s)
            e[s] = s < S && b0 + s < a.num_seqs && j < a.max_blocks_per_seq
                       ? a.block_tables[(int64_t)(b0 + s) * a.table_stride + (j >> a.block_shift)]
                       : -1;
        int in_play = 0, e0 = 0;
        bool same = true;
#pragma unroll
        for (int s = 0; s < kMaxGroupSeqs; ++s) {
            if (j < nb[s]) {
                const int sb = sub_block(e[s], j, a.block_shift);
                if (in_play == 0) e0 = sb;
                same = same && sb == e0;
                ++in_play;
            }
        }
        const unsigned long long stop = __ballot(in_play < 2 || !same);
        if (stop) {
            cp = uniform(base + __ffsll(stop) - 1);
            break;
        }
    }
    // lane 0: the shared run; lane 1 + s: member s's blocks past it
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < kMaxGroupSeqs; ++s)
        if (lane == 1 + s) cnt = nb[s] - min(cp, nb[s]);
    if (lane == 0) cnt = cp;
    if (lane <= S) a.owner_blocks[grp * (S + 1) + lane] = cnt;
}

// One segment of a stretch: blocks [j0, j1) of owner (group grp, member sel;
// sel < 0: the group's shared run) among its cnt blocks, for kv head g.
template <int DT, bool NT>
__device__ __forceinline__ void grouped_segment(const DecodeArgs& a, uint16_t* vt, int grp, int g, int sel, int j0,
                                                int j1, int cnt, int64_t st) {
    constexpr int D = 128;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;                   // MFMA column
    const int lg = lane >> 4;
    const int S = a.seqs_per_wave;
    const int b0 = grp * S;
    const int s_col = lr / a.group;             // this column's member
    const int h_col = lr - s_col * a.group;
    const bool col_live = s_col < S && b0 + s_col < a.num_seqs;
    const int n_col = col_live ? seq_tokens(a, b0 + s_col) : 0;
    const int64_t my_row = (int64_t)(col_live ? b0 + s_col : b0) * a.num_q_heads + (int64_t)g * a.group + h_col;

    int nt[kMaxGroupSeqs], nb[kMaxGroupSeqs];   // members' lengths and block counts (uniform)
    int nmax = 0;
#pragma unroll
    for (int s = 0; s < kMaxGroupSeqs; ++s) {
        nt[s] = s < S && b0 + s < a.num_seqs ? seq_tokens(a, b0 + s) : 0;
        nb[s] = ceil_blocks(nt[s]);
        nmax = max(nmax, nt[s]);
    }
    // a member's own blocks follow the shared run: offset them by it
    int off = 0, nsel = 0;
#pragma unroll
    for (int s = 0; s < kMaxGroupSeqs; ++s)
        if (s == sel) {
            off = nb[s] - cnt;
            nsel = nt[s];
        }
    if (sel >= 0) nmax = nsel;   // V rows past it hold no token of this member
    const bool on = sel < 0 ? col_live : s_col == sel;

    uint4 qf[4];
    {
        const uint16_t* q = static_cast<const uint16_t*>(a.q) + my_row * D + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[kk] = on ? *reinterpret_cast<const uint4*>(q + 32 * kk) : make_uint4(0, 0, 0, 0);
    }
    float m = -INFINITY;
    float l = 0.f;
    df32x4_t o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = df32x4_t{0.f, 0.f, 0.f, 0.f};

    const int64_t row_stride = (int64_t)a.num_kv_heads * D;
    const int tk = (lr & 3) * 4 + (lr >> 2);
    const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)g * D + 8 * lg +
                            (int64_t)tk * row_stride;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + (int64_t)g * D + 8 * lr +
                            (int64_t)lg * row_stride;
    const float cs = a.scale_log2;
    const uint16_t* vtr = vt + (4 * (lr >> 2) + lg) * kVRow + 4 * (lr & 3);
    const int32_t* tables = a.block_tables + (int64_t)b0 * a.table_stride;

    // block j of the owner: its own, or the one every member in play names
    auto load = [&](int j, uint4 (&kr)[4], uint4 (&vr)[4]) __attribute__((always_inline)) -> bool {
        int who = sel;
        if (sel < 0) {
            who = 0;
#pragma unroll
            for (int s = kMaxGroupSeqs - 1; s >= 0; --s)
                if (j < nb[s]) who = s;
        }
        const int pb = sub_block(tables[(int64_t)who * a.table_stride + (j >> a.block_shift)], j, a.block_shift);
        const bool ok = pb >= 0 && (int64_t)pb < a.num_blocks;
        const int64_t boff = (int64_t)(ok ? pb : 0) * kBlockSize * row_stride;
        // a member's own blocks are read once in the call: stream them; the
        // shared run is read by every group of its sharers: keep it cacheable
        if (sel >= 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kr[i] = load_kv<true>(kbase + boff + 32 * i);
                vr[i] = load_kv<true>(vbase + boff + (int64_t)4 * i * row_stride);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kr[i] = load_kv<NT>(kbase + boff + 32 * i);
                vr[i] = load_kv<NT>(vbase + boff + (int64_t)4 * i * row_stride);
            }
        }
        return ok;
    };

    auto process = [&](const uint4 (&kr)[4], const uint4 (&vr)[4], bool ok, int j) __attribute__((always_inline)) {
        df32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) sacc = mfma_16x16x32<DT>(kr[kk], qf[kk], sacc);
        bool vrow[4];
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = j * kBlockSize + 4 * i + lg;
            vrow[i] = ok && key < nmax;
            x[i] = ok && on && key < n_col ? sacc[i] * cs : -INFINITY;
        }
        float mb = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]),
                                                 __builtin_elementwise_maximum(x[2], x[3]));
        mb = xor32_max(xor16_max(mb));
        const bool raise = mb > m + 8.f;
        const float mn = raise ? mb : m;
        if (__any(raise)) {
            const float alpha = raise ? fast_exp2(m - mn) : 1.f;
            l *= alpha;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
        }
        m = mn;
        const float mu = mn == -INFINITY ? 0.f : mn;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - mu);
        uint2 pb;
        pb.x = pack2<DT>(p[0], p[1]);
        pb.y = pack2<DT>(p[2], p[3]);
        l = dot2<DT>(pb.y, kOnes2<DT>, dot2<DT>(pb.x, kOnes2<DT>, l));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(vt + (4 * i + lg) * kVRow + 8 * lr) = vrow[i] ? vr[i] : make_uint4(0, 0, 0, 0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const ds16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (ds16x4_t __attribute__((address_space(3)))*)(vtr + 16 * mt));
            o[mt] = mfma_16x16x16<DT>(__builtin_bit_cast(uint2, va), pb, o[mt]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    const int ja = off + j0, jb = off + j1;
    {
        uint4 kc[4], vc[4];
        bool okc = load(ja, kc, vc);
        for (int j = ja; j < jb; ++j) {
            uint4 kn[4], vn[4];
            bool okn = false;
            if (j + 1 < jb) okn = load(j + 1, kn, vn);   // next block in flight
            process(kc, vc, okc, j);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kc[i] = kn[i];
                vc[i] = vn[i];
            }
            okc = okn;
        }
    }

    const float lt = xor32_sum(xor16_sum(l));
    if (!on) return;
    // the column's row is finished here when this segment saw all of its blocks
    const bool all = j0 == 0 && j1 == cnt;
    bool final_out;
    int64_t idx;
    if (sel < 0) {
        if (min(cnt, ceil_blocks(n_col)) == 0) return;   // an empty member: the merge writes its zeros
        final_out = all && a.owner_blocks[(int64_t)grp * (S + 1) + 1 + s_col] == 0;
        idx = a.shared_base + (((int64_t)grp + st) * a.num_kv_heads + g) * 16 + lr;
    } else {
        final_out = all && off == 0;
        idx = (((int64_t)b0 + sel + st) * a.num_kv_heads + g) * a.group + h_col;
    }
    if (final_out) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        uint16_t* dst = static_cast<uint16_t*>(a.out) + my_row * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            uint2 w;
            w.x = pack2<DT>(o[mt][0] * inv, o[mt][1] * inv);
            w.y = pack2<DT>(o[mt][2] * inv, o[mt][3] * inv);
            *reinterpret_cast<uint2*>(dst + 16 * mt) = w;
        }
    } else {
        float* dst = a.ws_acc + idx * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            *reinterpret_cast<float4*>(dst + 16 * mt) = make_float4(o[mt][0], o[mt][1], o[mt][2], o[mt][3]);
        if (lg == 0) a.ws_ml[idx] = make_float2(m, lt);
    }
}

// The balanced split over the owner stream: stretch st, kv head g per wave.
template <int DT, bool NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void decode_gqa_grouped_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t vlds[4][kBlockSize * kVRow];
    const int wave = uniform(threadIdx.x >> 6);
    grouped_walk<NT>(a, wave, [&](int grp, int g, int sel, int j0, int j1, int cnt, int64_t st) {
        grouped_segment<DT, NT>(a, vlds[wave], grp, g, sel, j0, j1, cnt, st);
    });
}

// Combine the partial states of one (sequence, q head):
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p with M = max_p m_p.
// One wave per output row (sequence, query, q head); lane i owns elements
// D/64 * i ..: the max and the denominator are wave reductions over the
// partial states' (m, l), the numerator one pass over the partial rows -- no
// LDS, no barrier, so the merge costs little more than reading the partials.
// Fixed partitions: the row's states are slots row * num_parts + p.  Balanced
// split: sequence b covers stream blocks [P, P + nblk), so stretches
// s0 = P / C .. s1 = (P + nblk - 1) / C left the state of the row's unit ui in
// slots ((b + s) * upb + ui) * state_heads + h; a row whose sequence one stretch
// covered whole was finished there, and a row of an empty sequence, which no
// stretch covers, gets its zeros here.  With sequence groups the stretches of
// the group's shared run come first, then those of the member's own blocks.
template <int DT, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int EPL = D / kWave;   // elements per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);   // q / out row
    if (item >= (int64_t)a.num_seqs * a.q_per_seq * a.num_q_heads) return;
    const int b = (int)(item / ((int64_t)a.q_per_seq * a.num_q_heads));
    uint16_t* dst = static_cast<uint16_t*>(a.out) + item * D + EPL * lane;

    const int n = seq_tokens(a, b);
    const int nblk = ceil_blocks(n);
    int64_t base = 0, shared = 0;
    int stride = 0, count = 0, nsh = 0, sh_stride = 0;
    if (a.balanced) {
        if (nblk == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) dst[e] = 0;
            return;
        }
        const int head = (int)(item % a.num_q_heads);
        const int g = head / a.group;
        if (a.owner_blocks) {   // sequence groups: the shared run's stretches, then the member's own
            const int S = a.seqs_per_wave;
            const int grp = b / S;
            const int mem = b - grp * S;
            const int hh = head - g * a.group;
            const int og = grp * (S + 1);
            const int cp = a.owner_blocks[og];
            const int priv = a.owner_blocks[og + 1 + mem];
            const BlockCounts counts = owner_counts(a);
            const int pg = counts.prefix(og);
            const int stretch = balanced_stretch(a, counts.total());
            if (priv < nblk) {
                const int t0 = pg / stretch;
                const int t1 = (pg + cp - 1) / stretch;
                if (priv == 0 && t0 == t1) return;   // one stretch covered the whole row
                nsh = t1 - t0 + 1;
                shared = a.shared_base + (((int64_t)grp + t0) * a.num_kv_heads + g) * 16 + mem * a.group + hh;
                sh_stride = a.num_kv_heads * 16;
            }
            if (priv > 0) {
                int pb = pg + cp;
                for (int r = 0; r < mem; ++r) pb += a.owner_blocks[og + 1 + r];
                const int s0 = pb / stretch;
                const int s1 = (pb + priv - 1) / stretch;
                if (nsh == 0 && s0 == s1) return;   // one stretch covered the whole row
                base = (((int64_t)b + s0) * a.num_kv_heads + g) * a.group + hh;
                stride = a.num_kv_heads * a.group;
                count = s1 - s0 + 1;
            }
        } else {
            // the row's column of its kv head: (query, head) = jq * group + head % group
            const int jq = (int)((item / a.num_q_heads) % a.q_per_seq);
            const int col = jq * a.group + head - g * a.group;
            const int hc = col / a.heads_per_wave;
            const int h = col - hc * a.heads_per_wave;
            const int upb = a.num_kv_heads * a.head_chunks;
            const BlockCounts counts = sequence_blocks(a);
            const int before = counts.prefix(b);
            const int stretch = balanced_stretch(a, counts.total());
            const int s0 = before / stretch;
            const int s1 = (before + nblk - 1) / stretch;
            if (s0 == s1) return;   // one stretch covered the whole sequence
            base = (((int64_t)b + s0) * upb + g * a.head_chunks + hc) * a.state_heads + h;
            stride = upb * a.state_heads;
            count = s1 - s0 + 1;
        }
    } else {
        const int nparts = nblk <= a.part_blocks ? 1 : (nblk + a.part_blocks - 1) / a.part_blocks;
        if (nparts <= 1) return;   // finished by the partition kernel
        base = item * a.num_parts;
        stride = 1;
        count = nparts;
    }

    // state p: the shared run's (p < nsh), else the row's own
    auto slot = [&](int p) -> int64_t {
        return p < nsh ? shared + (int64_t)p * sh_stride : base + (int64_t)(p - nsh) * stride;
    };
    const int states = nsh + count;
    float big = -INFINITY;
    for (int p = lane; p < states; p += kWave) big = fmaxf(big, a.ws_ml[slot(p)].x);
    big = xor32_max(xor16_max(group_max<16>(big)));
    float den = 0.f;
    for (int p = lane; p < states; p += kWave) {
        const float2 ml = a.ws_ml[slot(p)];
        den = fmaf(ml.x == -INFINITY ? 0.f : fast_exp2(ml.x - big), ml.y, den);
    }
    den = xor32_sum(xor16_sum(group_sum<16>(den)));

    float num[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] = 0.f;
    const float* acc = a.ws_acc + EPL * lane;
#pragma unroll 4
    for (int p = 0; p < states; ++p) {
        const int64_t sl = slot(p);
        const float mp = a.ws_ml[sl].x;   // the same address in every lane
        const float w = mp == -INFINITY ? 0.f : fast_exp2(mp - big);
#pragma unroll
        for (int e = 0; e < EPL; ++e) num[e] = fmaf(w, acc[sl * D + e], num[e]);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = f32_to_bits<DT>(num[e] * inv);
}

template <int DT, int D, bool NT, bool MQ>
static hipError_t launch_partitions_d(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    switch (a.heads_per_wave) {
        case 1: return launch(decode_partition_kernel<DT, D, 1, NT, MQ>, grid, dim3(256), s, a);
        case 2: return launch(decode_partition_kernel<DT, D, 2, NT, MQ>, grid, dim3(256), s, a);
        case 4: return launch(decode_partition_kernel<DT, D, 4, NT, MQ>, grid, dim3(256), s, a);
        case 8: return launch(decode_partition_kernel<DT, D, 8, NT, MQ>, grid, dim3(256), s, a);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, bool NT, bool MQ>
static hipError_t launch_partitions_t(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    if (a.gqa_mfma) return launch(decode_gqa_kernel<DT, NT, MQ>, grid, dim3(256), s, a);
    return a.head_dim == 128 ? launch_partitions_d<DT, 128, NT, MQ>(a, s, grid)
                             : launch_partitions_d<DT, 64, NT, MQ>(a, s, grid);
}

template <bool MQ>
static hipError_t launch_partitions_mq(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    if (a.dtype == kF16) {
        return a.stream_kv ? launch_partitions_t<kF16, true, MQ>(a, s, grid)
                           : launch_partitions_t<kF16, false, MQ>(a, s, grid);
    }
    return a.stream_kv ? launch_partitions_t<kBF16, true, MQ>(a, s, grid)
                       : launch_partitions_t<kBF16, false, MQ>(a, s, grid);
}

template <int DT, int D, bool NT>
static hipError_t launch_balanced_d(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    switch (a.heads_per_wave) {
        case 1: return launch(decode_balanced_kernel<DT, D, 1, NT>, grid, dim3(256), s, a);
        case 2: return launch(decode_balanced_kernel<DT, D, 2, NT>, grid, dim3(256), s, a);
        case 4: return launch(decode_balanced_kernel<DT, D, 4, NT>, grid, dim3(256), s, a);
        case 8: return launch(decode_balanced_kernel<DT, D, 8, NT>, grid, dim3(256), s, a);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, bool NT>
static hipError_t launch_balanced_t(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    if (a.gqa_mfma)
        return a.q_per_seq > 1 ? launch(decode_gqa_balanced_kernel<DT, NT, true>, grid, dim3(256), s, a)
                               : launch(decode_gqa_balanced_kernel<DT, NT, false>, grid, dim3(256), s, a);
    return a.head_dim == 128 ? launch_balanced_d<DT, 128, NT>(a, s, grid)
                             : launch_balanced_d<DT, 64, NT>(a, s, grid);
}

hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t s) {
    if (a.balanced) {
        // several queries per sequence: on matrix cores only
        if ((a.q_per_seq != 1 && !a.gqa_mfma) || a.num_items <= 0 || a.num_seqs > kScanItems)
            return hipErrorInvalidValue;
        const dim3 grid((unsigned)((a.num_items + 3) / 4));
        if (a.dtype == kF16)
            return a.stream_kv ? launch_balanced_t<kF16, true>(a, s, grid) : launch_balanced_t<kF16, false>(a, s, grid);
        return a.stream_kv ? launch_balanced_t<kBF16, true>(a, s, grid) : launch_balanced_t<kBF16, false>(a, s, grid);
    }
    const int64_t items = (int64_t)a.num_seqs * a.num_kv_heads * a.head_chunks * a.num_parts;
    if (items == 0) return hipSuccess;
    const int64_t wgs = (items + 3) / 4;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    return a.q_per_seq > 1 ? launch_partitions_mq<true>(a, s, grid) : launch_partitions_mq<false>(a, s, grid);
}

hipError_t launch_group_plan(const DecodeArgs& a, hipStream_t s) {
    if (a.seqs_per_wave < 2 || a.seqs_per_wave > kMaxGroupSeqs || !a.owner_blocks || a.num_seqs <= 0)
        return hipErrorInvalidValue;
    const int64_t groups = (a.num_seqs + a.seqs_per_wave - 1) / a.seqs_per_wave;
    if (groups * (a.seqs_per_wave + 1) > kScanItems) return hipErrorInvalidValue;
    return launch(decode_group_plan_kernel, dim3((unsigned)((groups + 3) / 4)), dim3(256), s, a);
}

hipError_t launch_decode_grouped(const DecodeArgs& a, hipStream_t s) {
    if (!a.gqa_mfma || a.head_dim != 128 || a.q_per_seq != 1 || !a.balanced || a.head_chunks != 1 ||
        a.seqs_per_wave < 2 || a.seqs_per_wave > kMaxGroupSeqs || a.seqs_per_wave * a.group > 16 ||
        !a.owner_blocks || !a.ws_acc || a.num_items <= 0 || a.num_items % a.num_kv_heads != 0)
        return hipErrorInvalidValue;
    hipError_t e = launch_group_plan(a, s);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((a.num_items + 3) / 4));
    if (a.dtype == kF16)
        return a.stream_kv ? launch(decode_gqa_grouped_kernel<kF16, true>, grid, dim3(256), s, a)
                           : launch(decode_gqa_grouped_kernel<kF16, false>, grid, dim3(256), s, a);
    return a.stream_kv ? launch(decode_gqa_grouped_kernel<kBF16, true>, grid, dim3(256), s, a)
                       : launch(decode_gqa_grouped_kernel<kBF16, false>, grid, dim3(256), s, a);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s) {
    const int64_t items = (int64_t)a.num_seqs * a.q_per_seq * a.num_q_heads;
    if (items == 0 || (!a.balanced && a.num_parts <= 1)) return hipSuccess;
    if (a.balanced && a.num_seqs > kScanItems) return hipErrorInvalidValue;
    const int64_t wgs = (items + 3) / 4;   // one wave per row
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    if (a.dtype == kF16) {
        return a.head_dim == 128 ? launch(decode_merge_kernel<kF16, 128>, grid, dim3(256), s, a)
                                 : launch(decode_merge_kernel<kF16, 64>, grid, dim3(256), s, a);
    }
    return a.head_dim == 128 ? launch(decode_merge_kernel<kBF16, 128>, grid, dim3(256), s, a)
                             : launch(decode_merge_kernel<kBF16, 64>, grid, dim3(256), s, a);
}

}  // namespace pa
