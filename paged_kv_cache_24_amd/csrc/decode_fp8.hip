// Paged decode attention over an FP8 (OCP E4M3) KV cache on gfx950.
//
// What is computed ("vLLM-Ascend 原理", §四 on KV-cache quantisation, with
// §2.4 step 3 for decode): the K/V rows are fetched through the block table as
// 8-bit codes, dequantised on chip with their per-(token, kv head) float32
// scale, and attended to exactly as in the 16-bit kernels of decode.hip:
//     score_t = scale * k_scale_t * (q . code_k_t)
//     out     = sum_t p_t * v_scale_t * code_v_t / sum_t p_t
// The partition / merge structure, the softmax state and the workspace format
// are those of the 16-bit kernels (the merge kernel is shared).  Half the
// bytes per token leave HBM, so the same bandwidth carries twice the tokens.
#include "common.h"
#include "kernels.h"

namespace pa {

typedef uint32_t u32x4_f8 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint8_t* p) {
    if constexpr (NT) {
        const u32x4_f8 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_f8*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

// 16 codes -> 8 packed 16-bit pairs, exact (scale 1)
template <int DT>
__device__ __forceinline__ void codes16_to_16bit(const uint4& c, uint4& lo, uint4& hi) {
    const uint2 a = fp8x4_to_16<DT>(c.x, 1.f), b = fp8x4_to_16<DT>(c.y, 1.f);
    const uint2 d = fp8x4_to_16<DT>(c.z, 1.f), e = fp8x4_to_16<DT>(c.w, 1.f);
    lo = make_uint4(a.x, a.y, b.x, b.y);
    hi = make_uint4(d.x, d.y, e.x, e.y);
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel (group <= 2, or head_dim 64).
//
// One wave owns one (sequence, kv head, q-head chunk, partition) item.  A
// token row of one kv head is D bytes of codes; LPR = D/16 lanes each load
// 16 of them with one 16-byte load, so a load instruction covers 64/LPR whole
// rows.  Lane (r, c) owns the TPL consecutive tokens r*TPL .. r*TPL+TPL-1 of
// every block: their scales are TPL consecutive floats, one small load.
// QK^T: the codes become 16-bit pairs (exact) for v_dot2 against q, summed
// over the row's lanes with DPP, then scaled by k_scale.  PV: codes become
// float32 and meet p * v_scale in float32 FMAs.
// ---------------------------------------------------------------------------
//
// fp8_vector_segment: blocks j0 .. j1-1 of unit (b, g, hc) for one wave; the
// final output (final_out) or the partial state in slot row * num_parts + slot
// (fixed partitions) or slot * state_heads + h (balanced split), as in decode.hip.
template <int DT, int D, int HPW, bool NT, bool BAL>
__device__ __forceinline__ void fp8_vector_segment(const DecodeArgs& a, int b, int g, int hc, int n,
                                                   int j0, int j1, bool final_out, int64_t slot) {
    constexpr int LPR = D / 16;             // lanes per token row
    constexpr int RPW = kWave / LPR;        // token rows per load instruction
    constexpr int TPL = kBlockSize / RPW;   // tokens per lane per block
    constexpr int NBUF = 4;                 // blocks in registers: one computed, three in flight
    constexpr float kLazyMax = 8.f;         // log2 margin before the reference max is raised
    static_assert(TPL == 1 || TPL == 2, "head_dim 64 or 128");

    const int lane = threadIdx.x & (kWave - 1);
    const int r = lane / LPR;
    const int c = lane % LPR;

    const int hbase = hc * HPW;
    const int hcount = min(HPW, a.group - hbase);
    const int64_t q_row0 = (int64_t)b * a.num_q_heads + (int64_t)g * a.group + hbase;

    uint4 qv[HPW][2];   // q elements 16c .. 16c+15 of each head
    {
        const uint16_t* q = static_cast<const uint16_t*>(a.q) + q_row0 * D + 16 * c;
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            const bool live = h < hcount;
            qv[h][0] = live ? *reinterpret_cast<const uint4*>(q + (int64_t)h * D) : make_uint4(0, 0, 0, 0);
            qv[h][1] = live ? *reinterpret_cast<const uint4*>(q + (int64_t)h * D + 8) : make_uint4(0, 0, 0, 0);
        }
    }

    float m[HPW], l[HPW], acc[HPW][16];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
    }

    const int64_t row_stride = (int64_t)a.num_kv_heads * D;   // bytes between token rows
    const int64_t lane_off = (int64_t)g * D + 16 * c + (int64_t)(r * TPL) * row_stride;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache) + lane_off;
    const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache) + lane_off;
    const float* ksb = a.k_scales + (int64_t)g * kBlockSize + r * TPL;
    const float* vsb = a.v_scales + (int64_t)g * kBlockSize + r * TPL;
    const int64_t scale_block_stride = (int64_t)a.num_kv_heads * kBlockSize;
    const int32_t* table = a.block_tables + (int64_t)b * a.table_stride;   // FP8 caches: 16-token blocks
    const float cs = a.scale_log2;

    struct Buf {
        uint4 k[TPL], v[TPL];
        float ks[TPL], vs[TPL];
        bool ok;
    };

    auto load = [&](int j, Buf& buf) {
        const int pb = table[j];
        buf.ok = pb >= 0 && (int64_t)pb < a.num_blocks;
        const int64_t blk = buf.ok ? pb : 0;
        const int64_t off = blk * kBlockSize * row_stride;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            buf.k[i] = load16<NT>(kbase + off + (int64_t)i * row_stride);
            buf.v[i] = load16<NT>(vbase + off + (int64_t)i * row_stride);
        }
        if constexpr (TPL == 2) {
            const float2 ks = *reinterpret_cast<const float2*>(ksb + blk * scale_block_stride);
            const float2 vs = *reinterpret_cast<const float2*>(vsb + blk * scale_block_stride);
            buf.ks[0] = ks.x; buf.ks[1] = ks.y;
            buf.vs[0] = vs.x; buf.vs[1] = vs.y;
        } else {
            buf.ks[0] = ksb[blk * scale_block_stride];
            buf.vs[0] = vsb[blk * scale_block_stride];
        }
    };

    auto process = [&](const Buf& buf, int j) {
        const bool full = buf.ok && (j + 1) * kBlockSize <= n;   // uniform
        float s[HPW][TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            uint4 k0, k1;
            codes16_to_16bit<DT>(buf.k[i], k0, k1);
            const float ksc = buf.ks[i] * cs;
#pragma unroll
            for (int h = 0; h < HPW; ++h) {
                const float d = dot8<DT>(qv[h][0], k0) + dot8<DT>(qv[h][1], k1);
                float t;
                if constexpr (LPR == 8) t = group_sum<8>(d);
                else t = quad_sum(d);
                s[h][i] = t * ksc;
            }
        }
        float vf[TPL][16];
        float vsc[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const uint32_t w[4] = {buf.v[i].x, buf.v[i].y, buf.v[i].z, buf.v[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f32x2_t lo = fp8x2_to_f32<false>(w[e]);
                const f32x2_t hi = fp8x2_to_f32<true>(w[e]);
                vf[i][4 * e] = lo.x;
                vf[i][4 * e + 1] = lo.y;
                vf[i][4 * e + 2] = hi.x;
                vf[i][4 * e + 3] = hi.y;
            }
            vsc[i] = buf.vs[i];
        }
        if (!full) {
            // the sequence's last block, or a block outside the pool: rows past the
            // end score -inf and weigh 0 (selects, so NaN codes or scales there
            // cannot leak into the sums)
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const bool valid = buf.ok && j * kBlockSize + r * TPL + i < n;
#pragma unroll
                for (int h = 0; h < HPW; ++h) s[h][i] = valid ? s[h][i] : -INFINITY;
#pragma unroll
                for (int e = 0; e < 16; ++e) vf[i][e] = valid ? vf[i][e] : 0.f;
                vsc[i] = valid ? vsc[i] : 0.f;
            }
        }
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            float mb = s[h][0];
#pragma unroll
            for (int i = 1; i < TPL; ++i) mb = fmaxf(mb, s[h][i]);
            // The lane's reference max m is raised only when a score passes it by
            // more than 2^8 (log2 domain), so probabilities stay below 256 and the
            // state is rescaled once per raise, not once per block; the result is
            // the same algebra.  While m = -inf any finite score raises it.
            if (mb > m[h] + kLazyMax) {
                const float alpha = fast_exp2(m[h] - mb);   // 0 while m = -inf
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[h][e] *= alpha;
                m[h] = mb;
            }
            const float mu = m[h] == -INFINITY ? 0.f : m[h];
            float pv[TPL];
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const float p = fast_exp2(s[h][i] - mu);
                ps += p;
                pv[i] = p * vsc[i];
            }
            l[h] += ps;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float x = acc[h][e];
#pragma unroll
                for (int i = 0; i < TPL; ++i) x = fmaf(pv[i], vf[i][e], x);
                acc[h][e] = x;
            }
        }
    };
    // NBUF register buffers: while one block is computed, NBUF-1 are in flight
    if (j0 < j1) {
        Buf buf[NBUF];
#pragma unroll
        for (int s = 0; s < NBUF - 1; ++s)
            if (j0 + s < j1) load(j0 + s, buf[s]);
        for (int j = j0; j < j1; j += NBUF) {
#pragma unroll
            for (int s = 0; s < NBUF; ++s) {
                if (j + s >= j1) break;
                if (j + s + NBUF - 1 < j1) load(j + s + NBUF - 1, buf[(s + NBUF - 1) % NBUF]);
                process(buf[s], j + s);
            }
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
        for (int e = 0; e < 16; ++e) {
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
            uint4 o0, o1;
            o0.x = pack2<DT>(acc[h][0] * inv, acc[h][1] * inv);
            o0.y = pack2<DT>(acc[h][2] * inv, acc[h][3] * inv);
            o0.z = pack2<DT>(acc[h][4] * inv, acc[h][5] * inv);
            o0.w = pack2<DT>(acc[h][6] * inv, acc[h][7] * inv);
            o1.x = pack2<DT>(acc[h][8] * inv, acc[h][9] * inv);
            o1.y = pack2<DT>(acc[h][10] * inv, acc[h][11] * inv);
            o1.z = pack2<DT>(acc[h][12] * inv, acc[h][13] * inv);
            o1.w = pack2<DT>(acc[h][14] * inv, acc[h][15] * inv);
            uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (q_row0 + h) * D + 16 * c);
            dst[0] = o0;
            dst[1] = o1;
        }
    } else {
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            if (h >= hcount) break;
            const int64_t idx = BAL ? slot * a.state_heads + h : (q_row0 + h) * a.num_parts + slot;
            float4* dst = reinterpret_cast<float4*>(a.ws_acc + idx * D + 16 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[e] = make_float4(acc[h][4 * e], acc[h][4 * e + 1], acc[h][4 * e + 2], acc[h][4 * e + 3]);
            if (c == 0) a.ws_ml[idx] = make_float2(m[h], l[h]);
        }
    }
}

template <int DT, int D, int HPW, bool NT>
__global__ __launch_bounds__(256) void decode_fp8_partition_kernel(DecodeArgs a) {
    DecodeItem it;
    if (!decode_item<NT>(a, uniform(threadIdx.x >> 6), it)) return;
    const int n = seq_tokens(a, it.b);
    const int nblk = ceil_blocks(n);
    const int nparts = nblk <= a.part_blocks ? 1 : (nblk + a.part_blocks - 1) / a.part_blocks;
    if (it.part >= nparts) return;
    const int j0 = it.part * a.part_blocks;
    fp8_vector_segment<DT, D, HPW, NT, false>(a, it.b, it.g, it.hc, n, j0, min(nblk, j0 + a.part_blocks),
                                              nparts == 1, it.part);
}

template <int DT, int D, int HPW, bool NT>
__global__ __launch_bounds__(256) void decode_fp8_balanced_kernel(DecodeArgs a) {
    balanced_walk<NT>(a, uniform(threadIdx.x >> 6),
                      [&](int b, int g, int hc, int n, int j0, int j1, bool whole, int64_t slot) {
                          fp8_vector_segment<DT, D, HPW, NT, true>(a, b, g, hc, n, j0, j1, whole, slot);
                      });
}

// ---------------------------------------------------------------------------
// GQA kernel (head_dim 128, 3..16 q heads per kv head): both products on
// matrix cores, as in decode.hip, with the codes widened on the way in.  A
// step takes TWO blocks (32 tokens): one softmax update, one max reduction and
// one LDS hand-off per 32 tokens, and P V contracts over all 32 at once.
//   S^T = K Q^T, per block: MFMA 16x16x32 x 4.  Lane (lr, lg) feeds token lr of
//        the block and head_dim elements 32*lg + 8*kk .. +8 for step kk (the
//        order of the head_dim sum is free as long as Q uses the same one): two
//        16-byte loads of 16 codes, widened exactly to 16-bit.  Lane l then
//        holds the scores of tokens 4*lg + i (i = 0..3) of each block for head
//        lr, so their k/v scales are one 16-byte load per block.
//   O^T += V^T P^T: MFMA 16x16x32 x 8 per step.  Contraction index
//        k = 8*lg + j stands for token 4*lg + j of the first block (j < 4) and
//        token 4*lg + j - 4 of the second (j >= 4): exactly the probabilities
//        lane (lr, lg) already holds, so P never moves.  V^T comes from one
//        per-wave LDS tile per block: the transposed read (ds_read_b64_tr_b16)
//        at row 4*lg + lr/4, column 4*(lr%4) hands lane (lr, lg) tokens
//        4*lg .. 4*lg+3 of head_dim element lr; one read per tile fills the
//        eight A elements.  The V codes are widened times 2^e (e = exponent of
//        the token's v_scale, exact in 16 bits) and the mantissa factor in
//        [1, 2) of v_scale multiplies the probabilities, so P never meets a
//        tiny scale in 16-bit precision; P times the factor enters rounded
//        once to 16 bits, and the row sum adds each rounded weight times
//        1/factor, so the weights stay consistent with the sum.
//        Lane (lr, lg) loads tokens 4*lg + (lr/8) and 4*lg + 2 + (lr/8) of a
//        block, codes 16*(lr%8) .. +16: tokens among its own four.
// ---------------------------------------------------------------------------
typedef __bf16 f8bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f8f16x8_t __attribute__((ext_vector_type(8)));
typedef float f8f32x4_t __attribute__((ext_vector_type(4)));
typedef short f8s16x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f8f32x4_t f8_mfma_16x16x32(const uint4& a, const uint4& b, f8f32x4_t c) {
    if constexpr (DT == kF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f8f16x8_t, a),
                                                      __builtin_bit_cast(f8f16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(f8bf16x8_t, a),
                                                       __builtin_bit_cast(f8bf16x8_t, b), c, 0, 0, 0);
    }
}

__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (f8s16x4_t __attribute__((address_space(3)))*)(p)));
}

constexpr int kVRowF8 = 144;   // LDS row stride of a widened V tile (16-bit elements)
// Register ring depth, in block pairs.  Measured on MI355X: a deeper ring
// (one or two pairs in flight while a pair is computed) needs more registers
// than 3 waves per SIMD allow, or drops to 2 waves, and was no faster than one
// pair at a time with 4 resident waves (122 registers) hiding each other's loads.
constexpr int kGqaFp8Pairs = 1;

//
// fp8_gqa_segment: blocks j0 .. j1-1 of unit (b, g, hc) for one wave, `vt` its
// two V tiles in LDS; the final output (final_out) or the partial state of
// column lr in slot row * num_parts + slot (fixed partitions) or
// slot * state_heads + lr (balanced split).
constexpr int kFp8Tile = kBlockSize * kVRowF8;

template <int DT, bool NT, int NBUF, bool BAL>
__device__ __forceinline__ void fp8_gqa_segment(const DecodeArgs& a, uint16_t* vt, int b, int g, int hc, int n,
                                                int j0, int j1, bool final_out, int64_t slot) {
    constexpr int D = 128;
    constexpr int kTile = kFp8Tile;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;    // MFMA column = q head; token of the K rows; V^T row
    const int lg = lane >> 4;    // tokens 4*lg .. 4*lg+3 of each block
    const int hcount = min(16, a.group - hc * 16);
    const int64_t q_row0 = (int64_t)b * a.num_q_heads + (int64_t)g * a.group + hc * 16;
    const bool head_live = lr < hcount;

    uint4 qf[4];   // head lr, elements 32*lg + 8*kk .. +8
    {
        const uint16_t* q = static_cast<const uint16_t*>(a.q) + (q_row0 + (head_live ? lr : 0)) * D + 32 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[kk] = head_live ? *reinterpret_cast<const uint4*>(q + 8 * kk) : make_uint4(0, 0, 0, 0);
    }

    float m = -INFINITY;   // running max of head lr (same in lanes l, l^16, l^32, l^48)
    float l = 0.f;         // this lane's share of the running sum
    f8f32x4_t o[8];        // O^T: lane holds elements 16*mt + 4*lg + i of head lr
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f8f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int64_t row_stride = (int64_t)a.num_kv_heads * D;   // bytes
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache) + (int64_t)g * D + 32 * lg +
                           (int64_t)lr * row_stride;
    const int vrow0 = 4 * lg + (lr >> 3);      // V rows of this lane: vrow0 and vrow0 + 2
    const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache) + (int64_t)g * D + 16 * (lr & 7) +
                           (int64_t)vrow0 * row_stride;
    // scales of tokens 4*lg .. 4*lg+3: lanes lr < 8 load the k scales, lanes
    // lr >= 8 the v scales (half the registers per buffer); a DPP rotation by
    // 8 lanes hands each lane the other half when the block is computed
    const bool k_half = lr < 8;
    const float* scb = (k_half ? a.k_scales : a.v_scales) + (int64_t)g * kBlockSize + 4 * lg;
    const int64_t scale_block_stride = (int64_t)a.num_kv_heads * kBlockSize;
    const int32_t* table = a.block_tables + (int64_t)b * a.table_stride;   // FP8 caches: 16-token blocks
    const float cs = a.scale_log2;
    const int tr_off = (4 * lg + (lr >> 2)) * kVRowF8 + 4 * (lr & 3);

    struct Blk {
        uint4 k[2], v[2];
        float4 sc;
        bool ok;
    };
    struct Pair {
        Blk x[2];
    };

    auto load_blk = [&](int j, Blk& blk_regs) {
        if (j >= j1) {   // the odd block after the last one: nothing to read, every row masked
            blk_regs.ok = false;
            blk_regs.k[0] = blk_regs.k[1] = blk_regs.v[0] = blk_regs.v[1] = make_uint4(0, 0, 0, 0);
            blk_regs.sc = make_float4(1.f, 1.f, 1.f, 1.f);
            return;
        }
        const int pb = table[j];
        blk_regs.ok = pb >= 0 && (int64_t)pb < a.num_blocks;
        const int64_t blk = blk_regs.ok ? pb : 0;
        const int64_t off = blk * kBlockSize * row_stride;
        blk_regs.k[0] = load16<NT>(kbase + off);
        blk_regs.k[1] = load16<NT>(kbase + off + 16);
        blk_regs.v[0] = load16<NT>(vbase + off);
        blk_regs.v[1] = load16<NT>(vbase + off + 2 * row_stride);
        blk_regs.sc = *reinterpret_cast<const float4*>(scb + blk * scale_block_stride);
    };
    auto load = [&](int j, Pair& pr) {
        load_blk(j, pr.x[0]);
        load_blk(j + 1, pr.x[1]);
    };

    auto process = [&](const Pair& pr, int j) {
        f8f32x4_t sacc[2];
        float ks[2][4], vs[2][4];
        bool valid[2][4];
        float x[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const Blk& bk = pr.x[h];
            sacc[h] = f8f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint4& w = bk.k[kk >> 1];
                const uint32_t w0 = (kk & 1) ? w.z : w.x;
                const uint32_t w1 = (kk & 1) ? w.w : w.y;
                const uint2 e0 = fp8x4_to_16<DT>(w0, 1.f), e1 = fp8x4_to_16<DT>(w1, 1.f);
                sacc[h] = f8_mfma_16x16x32<DT>(make_uint4(e0.x, e0.y, e1.x, e1.y), qf[kk], sacc[h]);
            }
            const float mine[4] = {bk.sc.x, bk.sc.y, bk.sc.z, bk.sc.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float other = dpp<kDppRowRor8>(mine[i]);
                ks[h][i] = k_half ? mine[i] : other;
                vs[h][i] = k_half ? other : mine[i];
            }
            const int t0 = (j + h) * kBlockSize;
            const bool full = bk.ok && t0 + kBlockSize <= n;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                valid[h][i] = full || (bk.ok && (t0 + 4 * lg + i < n));
                x[h][i] = valid[h][i] ? sacc[h][i] * (ks[h][i] * cs) : -INFINITY;
            }
        }
        float mb = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                         fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
        mb = xor32_max(xor16_max(mb));
        // raise the running max only when this step beats it by more than 2^8:
        // otherwise keep it (p <= 256, exact algebra) and skip the rescale of O^T
        const bool raise = mb > m + 8.f;   // also true on the first live step
        const float mn = raise ? mb : m;
        if (__any(raise)) {
            const float alpha = raise ? fast_exp2(m - mn) : 1.f;   // exp2(-inf) = 0
            l *= alpha;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
        }
        m = mn;
        const float mu = mn == -INFINITY ? 0.f : mn;
        // P times the mantissa factor of each key's v scale (V holds code * 2^e)
        // enters PV rounded once to 16 bits; the row sum adds each rounded weight
        // times 1/factor, the probability the product used, so the weights that
        // multiply V stay consistent with the sum
        float pm[2][4], imu[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(x[h][i] - mu);
                const float f = scale_mantissa(vs[h][i]);
                pm[h][i] = valid[h][i] ? p * f : 0.f;
                imu[h][i] = __builtin_amdgcn_rcpf(f);
            }
        // V tiles to LDS, widened times 2^exponent(v_scale); rows past the
        // sequence end as zeros (MFMA would turn 0 x NaN into NaN)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const Blk& bk = pr.x[h];
            const int t0 = (j + h) * kBlockSize;
            const bool full = bk.ok && t0 + kBlockSize <= n;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int row = vrow0 + 2 * k;
                const int sel = (lr >> 3) + 2 * k;
                const float vsr = sel == 0 ? vs[h][0] : sel == 1 ? vs[h][1] : sel == 2 ? vs[h][2] : vs[h][3];
                const bool ok = full || (bk.ok && (t0 + row < n));
                const uint4& w = bk.v[k];
                const uint2 e0 = fp8x4_to_16<DT>(w.x, vsr), e1 = fp8x4_to_16<DT>(w.y, vsr);
                const uint2 e2 = fp8x4_to_16<DT>(w.z, vsr), e3 = fp8x4_to_16<DT>(w.w, vsr);
                uint4* dst = reinterpret_cast<uint4*>(vt + h * kTile + row * kVRowF8 + 16 * (lr & 7));
                dst[0] = ok ? make_uint4(e0.x, e0.y, e1.x, e1.y) : make_uint4(0, 0, 0, 0);
                dst[1] = ok ? make_uint4(e2.x, e2.y, e3.x, e3.y) : make_uint4(0, 0, 0, 0);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint4 ph;
        ph.x = pack2<DT>(pm[0][0], pm[0][1]);
        ph.y = pack2<DT>(pm[0][2], pm[0][3]);
        ph.z = pack2<DT>(pm[1][0], pm[1][1]);
        ph.w = pack2<DT>(pm[1][2], pm[1][3]);
        l = fmaf(lo_to_f32<DT>(ph.x), imu[0][0], l);
        l = fmaf(hi_to_f32<DT>(ph.x), imu[0][1], l);
        l = fmaf(lo_to_f32<DT>(ph.y), imu[0][2], l);
        l = fmaf(hi_to_f32<DT>(ph.y), imu[0][3], l);
        l = fmaf(lo_to_f32<DT>(ph.z), imu[1][0], l);
        l = fmaf(hi_to_f32<DT>(ph.z), imu[1][1], l);
        l = fmaf(lo_to_f32<DT>(ph.w), imu[1][2], l);
        l = fmaf(hi_to_f32<DT>(ph.w), imu[1][3], l);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const uint2 v0 = lds_read_tr16(vt + tr_off + 16 * mt);
            const uint2 v1 = lds_read_tr16(vt + kTile + tr_off + 16 * mt);
            const uint4 va = make_uint4(v0.x, v0.y, v1.x, v1.y);
            o[mt] = f8_mfma_16x16x32<DT>(va, ph, o[mt]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // NBUF register buffers of block pairs: while one pair is computed,
    // NBUF-1 are in flight
    if (j0 < j1) {
        Pair buf[NBUF];
#pragma unroll
        for (int s = 0; s < NBUF - 1; ++s)
            if (j0 + 2 * s < j1) load(j0 + 2 * s, buf[s]);
        for (int j = j0; j < j1; j += 2 * NBUF) {
#pragma unroll
            for (int s = 0; s < NBUF; ++s) {
                const int jj = j + 2 * s;
                if (jj >= j1) break;
                if (jj + 2 * (NBUF - 1) < j1) load(jj + 2 * (NBUF - 1), buf[(s + NBUF - 1) % NBUF]);
                process(buf[s], jj);
            }
        }
    }

    const float lt = xor32_sum(xor16_sum(l));
    if (!head_live) return;
    if (final_out) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        uint16_t* dst = static_cast<uint16_t*>(a.out) + (q_row0 + lr) * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            uint2 w;
            w.x = pack2<DT>(o[mt][0] * inv, o[mt][1] * inv);
            w.y = pack2<DT>(o[mt][2] * inv, o[mt][3] * inv);
            *reinterpret_cast<uint2*>(dst + 16 * mt) = w;
        }
    } else {
        const int64_t idx = BAL ? slot * a.state_heads + lr : (q_row0 + lr) * a.num_parts + slot;
        float* dst = a.ws_acc + idx * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            *reinterpret_cast<float4*>(dst + 16 * mt) = make_float4(o[mt][0], o[mt][1], o[mt][2], o[mt][3]);
        if (lg == 0) a.ws_ml[idx] = make_float2(m, lt);
    }
}

template <int DT, bool NT, int NBUF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_fp8_gqa_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t vlds[4][2 * kFp8Tile];
    const int wave = uniform(threadIdx.x >> 6);
    DecodeItem it;
    if (!decode_item<NT>(a, wave, it)) return;
    const int n = seq_tokens(a, it.b);
    const int nblk = ceil_blocks(n);
    const int nparts = nblk <= a.part_blocks ? 1 : (nblk + a.part_blocks - 1) / a.part_blocks;
    if (it.part >= nparts) return;
    const int j0 = it.part * a.part_blocks;
    fp8_gqa_segment<DT, NT, NBUF, false>(a, vlds[wave], it.b, it.g, it.hc, n, j0,
                                         min(nblk, j0 + a.part_blocks), nparts == 1, it.part);
}

template <int DT, bool NT, int NBUF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_fp8_gqa_balanced_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t vlds[4][2 * kFp8Tile];
    const int wave = uniform(threadIdx.x >> 6);
    balanced_walk<NT>(a, wave, [&](int b, int g, int hc, int n, int j0, int j1, bool whole, int64_t slot) {
        fp8_gqa_segment<DT, NT, NBUF, true>(a, vlds[wave], b, g, hc, n, j0, j1, whole, slot);
    });
}

// ---------------------------------------------------------------------------
// Sequence groups over the FP8 cache (PA_DECODE_SHARED_PREFIX): the owner
// stream, plan and state slots of the 16-bit grouped decode (decode.hip), with
// this file's block-pair step.  Column c carries member c / G, head c % G; a
// shared run's pair scores every member still in play, a member's own pair its
// G columns.  Own blocks stream (read once in the call), shared runs stay
// cacheable.
template <int DT, bool NT>
__device__ __forceinline__ void fp8_grouped_segment(const DecodeArgs& a, uint16_t* vt, int grp, int g, int sel,
                                                    int j0, int j1, int cnt, int64_t st) {
    constexpr int D = 128;
    constexpr int kTile = kFp8Tile;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;    // MFMA column; token of the K rows; V^T row
    const int lg = lane >> 4;    // tokens 4*lg .. 4*lg+3 of each block
    const int S = a.seqs_per_wave;
    const int b0 = grp * S;
    const int s_col = lr / a.group;
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
    int off = 0, nsel = 0;
#pragma unroll
    for (int s = 0; s < kMaxGroupSeqs; ++s)
        if (s == sel) {
            off = nb[s] - cnt;
            nsel = nt[s];
        }
    if (sel >= 0) nmax = nsel;   // V rows past it hold no token of this member
    const bool on = sel < 0 ? col_live : s_col == sel;

    uint4 qf[4];   // column lr, elements 32*lg + 8*kk .. +8
    {
        const uint16_t* q = static_cast<const uint16_t*>(a.q) + my_row * D + 32 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[kk] = on ? *reinterpret_cast<const uint4*>(q + 8 * kk) : make_uint4(0, 0, 0, 0);
    }
    float m = -INFINITY;
    float l = 0.f;
    f8f32x4_t o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f8f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int64_t row_stride = (int64_t)a.num_kv_heads * D;   // bytes
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache) + (int64_t)g * D + 32 * lg +
                           (int64_t)lr * row_stride;
    const int vrow0 = 4 * lg + (lr >> 3);
    const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache) + (int64_t)g * D + 16 * (lr & 7) +
                           (int64_t)vrow0 * row_stride;
    const bool k_half = lr < 8;
    const float* scb = (k_half ? a.k_scales : a.v_scales) + (int64_t)g * kBlockSize + 4 * lg;
    const int64_t scale_block_stride = (int64_t)a.num_kv_heads * kBlockSize;
    const int32_t* tables = a.block_tables + (int64_t)b0 * a.table_stride;   // 16-token blocks
    const float cs = a.scale_log2;
    const int tr_off = (4 * lg + (lr >> 2)) * kVRowF8 + 4 * (lr & 3);
    const int ja = off + j0, jb = off + j1;

    struct Blk {
        uint4 k[2], v[2];
        float4 sc;
        bool ok;
    };
    auto load_blk = [&](int j, Blk& r) {
        if (j >= jb) {   // the odd block after the last one: nothing to read, every row masked
            r.ok = false;
            r.k[0] = r.k[1] = r.v[0] = r.v[1] = make_uint4(0, 0, 0, 0);
            r.sc = make_float4(1.f, 1.f, 1.f, 1.f);
            return;
        }
        int who = sel;
        if (sel < 0) {   // the block every member in play names
            who = 0;
#pragma unroll
            for (int s = kMaxGroupSeqs - 1; s >= 0; --s)
                if (j < nb[s]) who = s;
        }
        const int pb = tables[(int64_t)who * a.table_stride + j];
        r.ok = pb >= 0 && (int64_t)pb < a.num_blocks;
        const int64_t blk = r.ok ? pb : 0;
        const int64_t boff = blk * kBlockSize * row_stride;
        if (sel >= 0) {
            r.k[0] = load16<true>(kbase + boff);
            r.k[1] = load16<true>(kbase + boff + 16);
            r.v[0] = load16<true>(vbase + boff);
            r.v[1] = load16<true>(vbase + boff + 2 * row_stride);
        } else {
            r.k[0] = load16<NT>(kbase + boff);
            r.k[1] = load16<NT>(kbase + boff + 16);
            r.v[0] = load16<NT>(vbase + boff);
            r.v[1] = load16<NT>(vbase + boff + 2 * row_stride);
        }
        r.sc = *reinterpret_cast<const float4*>(scb + blk * scale_block_stride);
    };

    for (int j = ja; j < jb; j += 2) {
        Blk pr[2];
        load_blk(j, pr[0]);
        load_blk(j + 1, pr[1]);
        f8f32x4_t sacc[2];
        float vs[2][4];
        bool valid[2][4];
        float x[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const Blk& bk = pr[h];
            sacc[h] = f8f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint4& w = bk.k[kk >> 1];
                const uint32_t w0 = (kk & 1) ? w.z : w.x;
                const uint32_t w1 = (kk & 1) ? w.w : w.y;
                const uint2 e0 = fp8x4_to_16<DT>(w0, 1.f), e1 = fp8x4_to_16<DT>(w1, 1.f);
                sacc[h] = f8_mfma_16x16x32<DT>(make_uint4(e0.x, e0.y, e1.x, e1.y), qf[kk], sacc[h]);
            }
            const float mine[4] = {bk.sc.x, bk.sc.y, bk.sc.z, bk.sc.w};
            float ks[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float other = dpp<kDppRowRor8>(mine[i]);
                ks[i] = k_half ? mine[i] : other;
                vs[h][i] = k_half ? other : mine[i];
            }
            const int t0 = (j + h) * kBlockSize;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                valid[h][i] = bk.ok && on && t0 + 4 * lg + i < n_col;
                x[h][i] = valid[h][i] ? sacc[h][i] * (ks[i] * cs) : -INFINITY;
            }
        }
        float mb = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                         fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
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
        float pm[2][4], imu[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(x[h][i] - mu);
                const float f = scale_mantissa(vs[h][i]);
                pm[h][i] = valid[h][i] ? p * f : 0.f;
                imu[h][i] = __builtin_amdgcn_rcpf(f);
            }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const Blk& bk = pr[h];
            const int t0 = (j + h) * kBlockSize;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int row = vrow0 + 2 * k;
                const int sv = (lr >> 3) + 2 * k;
                const float vsr = sv == 0 ? vs[h][0] : sv == 1 ? vs[h][1] : sv == 2 ? vs[h][2] : vs[h][3];
                const bool ok = bk.ok && t0 + row < nmax;
                const uint4& w = bk.v[k];
                const uint2 e0 = fp8x4_to_16<DT>(w.x, vsr), e1 = fp8x4_to_16<DT>(w.y, vsr);
                const uint2 e2 = fp8x4_to_16<DT>(w.z, vsr), e3 = fp8x4_to_16<DT>(w.w, vsr);
                uint4* dst = reinterpret_cast<uint4*>(vt + h * kTile + row * kVRowF8 + 16 * (lr & 7));
                dst[0] = ok ? make_uint4(e0.x, e0.y, e1.x, e1.y) : make_uint4(0, 0, 0, 0);
                dst[1] = ok ? make_uint4(e2.x, e2.y, e3.x, e3.y) : make_uint4(0, 0, 0, 0);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint4 ph;
        ph.x = pack2<DT>(pm[0][0], pm[0][1]);
        ph.y = pack2<DT>(pm[0][2], pm[0][3]);
        ph.z = pack2<DT>(pm[1][0], pm[1][1]);
        ph.w = pack2<DT>(pm[1][2], pm[1][3]);
        l = fmaf(lo_to_f32<DT>(ph.x), imu[0][0], l);
        l = fmaf(hi_to_f32<DT>(ph.x), imu[0][1], l);
        l = fmaf(lo_to_f32<DT>(ph.y), imu[0][2], l);
        l = fmaf(hi_to_f32<DT>(ph.y), imu[0][3], l);
        l = fmaf(lo_to_f32<DT>(ph.z), imu[1][0], l);
        l = fmaf(hi_to_f32<DT>(ph.z), imu[1][1], l);
        l = fmaf(lo_to_f32<DT>(ph.w), imu[1][2], l);
        l = fmaf(hi_to_f32<DT>(ph.w), imu[1][3], l);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const uint2 v0 = lds_read_tr16(vt + tr_off + 16 * mt);
            const uint2 v1 = lds_read_tr16(vt + kTile + tr_off + 16 * mt);
            o[mt] = f8_mfma_16x16x32<DT>(make_uint4(v0.x, v0.y, v1.x, v1.y), ph, o[mt]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    const float lt = xor32_sum(xor16_sum(l));
    if (!on) return;
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

// 3 waves per SIMD hold the balanced split's 3072 waves in one round (at 4 the
// segment's registers spill)
template <int DT, bool NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void decode_fp8_gqa_grouped_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t vlds[4][2 * kFp8Tile];
    const int wave = uniform(threadIdx.x >> 6);
    grouped_walk<NT>(a, wave, [&](int grp, int g, int sel, int j0, int j1, int cnt, int64_t st) {
        fp8_grouped_segment<DT, NT>(a, vlds[wave], grp, g, sel, j0, j1, cnt, st);
    });
}

template <int DT, int D, bool NT>
static hipError_t launch_fp8_balanced_vector(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    switch (a.heads_per_wave) {
        case 1: return launch(decode_fp8_balanced_kernel<DT, D, 1, NT>, grid, dim3(256), s, a);
        case 2: return launch(decode_fp8_balanced_kernel<DT, D, 2, NT>, grid, dim3(256), s, a);
        case 4: return launch(decode_fp8_balanced_kernel<DT, D, 4, NT>, grid, dim3(256), s, a);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, bool NT>
static hipError_t launch_fp8_balanced_t(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    if (a.gqa_mfma) return launch(decode_fp8_gqa_balanced_kernel<DT, NT, kGqaFp8Pairs>, grid, dim3(256), s, a);
    return a.head_dim == 128 ? launch_fp8_balanced_vector<DT, 128, NT>(a, s, grid)
                             : launch_fp8_balanced_vector<DT, 64, NT>(a, s, grid);
}

template <int DT, int D, bool NT>
static hipError_t launch_fp8_vector(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    switch (a.heads_per_wave) {
        case 1: return launch(decode_fp8_partition_kernel<DT, D, 1, NT>, grid, dim3(256), s, a);
        case 2: return launch(decode_fp8_partition_kernel<DT, D, 2, NT>, grid, dim3(256), s, a);
        case 4: return launch(decode_fp8_partition_kernel<DT, D, 4, NT>, grid, dim3(256), s, a);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, bool NT>
static hipError_t launch_fp8_t(const DecodeArgs& a, hipStream_t s, dim3 grid) {
    if (a.gqa_mfma) return launch(decode_fp8_gqa_kernel<DT, NT, kGqaFp8Pairs>, grid, dim3(256), s, a);
    return a.head_dim == 128 ? launch_fp8_vector<DT, 128, NT>(a, s, grid)
                             : launch_fp8_vector<DT, 64, NT>(a, s, grid);
}

hipError_t launch_decode_grouped_fp8(const DecodeArgs& a, hipStream_t s) {
    if (!a.gqa_mfma || a.head_dim != 128 || a.q_per_seq != 1 || !a.balanced || a.head_chunks != 1 ||
        a.block_shift != 0 || a.seqs_per_wave < 2 || a.seqs_per_wave > kMaxGroupSeqs ||
        a.seqs_per_wave * a.group > 16 || !a.owner_blocks || !a.ws_acc || !a.k_scales || !a.v_scales ||
        a.num_items <= 0 || a.num_items % a.num_kv_heads != 0)
        return hipErrorInvalidValue;
    hipError_t e = launch_group_plan(a, s);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((a.num_items + 3) / 4));
    if (a.dtype == kF16)
        return a.stream_kv ? launch(decode_fp8_gqa_grouped_kernel<kF16, true>, grid, dim3(256), s, a)
                           : launch(decode_fp8_gqa_grouped_kernel<kF16, false>, grid, dim3(256), s, a);
    return a.stream_kv ? launch(decode_fp8_gqa_grouped_kernel<kBF16, true>, grid, dim3(256), s, a)
                       : launch(decode_fp8_gqa_grouped_kernel<kBF16, false>, grid, dim3(256), s, a);
}

hipError_t launch_decode_partitions_fp8(const DecodeArgs& a, hipStream_t s) {
    if (a.balanced) {
        if (a.q_per_seq != 1 || a.num_items <= 0 || a.num_seqs > kScanItems) return hipErrorInvalidValue;
        const dim3 grid((unsigned)((a.num_items + 3) / 4));
        if (a.dtype == kF16)
            return a.stream_kv ? launch_fp8_balanced_t<kF16, true>(a, s, grid)
                               : launch_fp8_balanced_t<kF16, false>(a, s, grid);
        return a.stream_kv ? launch_fp8_balanced_t<kBF16, true>(a, s, grid)
                           : launch_fp8_balanced_t<kBF16, false>(a, s, grid);
    }
    const int64_t items = (int64_t)a.num_seqs * a.num_kv_heads * a.head_chunks * a.num_parts;
    if (items == 0) return hipSuccess;
    const int64_t wgs = (items + 3) / 4;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    if (a.dtype == kF16) {
        return a.stream_kv ? launch_fp8_t<kF16, true>(a, s, grid) : launch_fp8_t<kF16, false>(a, s, grid);
    }
    return a.stream_kv ? launch_fp8_t<kBF16, true>(a, s, grid) : launch_fp8_t<kBF16, false>(a, s, grid);
}

}  // namespace pa
