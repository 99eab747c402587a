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
// Mapping.  One workgroup (8 waves) owns 128 query rows of one (sequence, kv
// head): 128/G positions times the G q heads that share the kv head, so every
// K/V tile is staged in LDS once for all of them.  Each wave owns 16 rows, which
// keeps it at ~128 VGPRs so four waves share each SIMD (two workgroups per CU):
// the softmax of one wave overlaps the matrix work of the others.
// For each 64-key tile:
//   S^T[key][row] = K[key][:] . Q[row][:]     (MFMA 16x16x32: A = K from LDS,
//                                              B = Q kept in registers)
//   online softmax per row: the C layout puts one row's keys in the four lanes
//   l, l^16, l^32, l^48, so the row max/sum is an in-lane reduction plus two
//   cross-lane steps;
//   O^T[d][row] += V^T[d][key] . P^T[key][row] (MFMA 16x16x32: B = P^T straight
//   from the softmax registers, A = V^T fragments produced by ds_read_b64_tr_b16
//   from the row-major V tile in LDS).
// Working on the transposed products keeps each row's statistics in the lanes
// that own the row in both products, so no shuffle of the probabilities or
// of the rescale factors is needed.  The next tile's K/V rows are loaded into
// registers while the current tile is computed and stored to the other LDS
// buffer afterwards (one barrier per tile).
//
// FP8 cache (F8): the same kernel over E4M3 codes with per-(token, kv head)
// float32 scales ("vLLM-Ascend 原理", §四 on KV-cache quantisation: dequantised
// after the block-table lookup, inside the operator).  Each thread stages 16
// codes of one key row; K enters LDS as exact 16-bit codes and its scale
// multiplies the scores, V enters as codes times 2^e (e = exponent of its
// scale, exact) and the scale's mantissa factor in [1, 2) multiplies P, which
// goes to the matrix cores as a 16-bit head and tail so the factor adds no
// rounding.  The per-key factors sit in two small LDS arrays beside the tiles.
#include <type_traits>

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
constexpr int kRows = 128;          // query rows per workgroup (8 waves x 16)
constexpr int kVRow = kPD + 16;     // LDS V row stride (elements): 288 bytes, conflict-free transposed reads

typedef short ps16x4_t __attribute__((ext_vector_type(4)));

constexpr int kKRow = kPD + 8;      // LDS K row stride (elements): 272 bytes, so the 16 rows of
                                    // an MFMA A fragment start 4 banks apart (conflict-free)

template <int DT, int G, bool F8>
__global__ __launch_bounds__(512, 4) void prefill_kernel(PrefillArgs a) {
    constexpr int P = kRows / G;    // positions per workgroup
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKT * kKRow];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kKT * kVRow];
    // FP8 only: per-key k scale and v-scale mantissa factor of each staged tile
    __shared__ __attribute__((aligned(16))) float lds_ks[F8 ? 2 : 1][F8 ? kKT : 4];
    __shared__ __attribute__((aligned(16))) float lds_mu[F8 ? 2 : 1][F8 ? kKT : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);   // 0..7: rows 16*wave .. 16*wave+15
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

    // ---- this lane's query row and its Q^T fragments
    uint4 qf[4];
    const int rho = wave * 16 + lr;
    const int qpos = ctx + pos0 + rho / G;
    {
        const int pos = pos0 + rho / G;
        const bool ok = pos < L;
        const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                              ((row0 + (ok ? pos : 0)) * a.num_q_heads + g * G + rho % G) * kPD + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[kk] = ok ? *reinterpret_cast<const uint4*>(src + 32 * kk) : make_uint4(0, 0, 0, 0);
    }
    const int wave_pos_lo = pos0 + (wave * 16) / G;
    const int wave_pos_hi = min(pos_end - 1, pos0 + (wave * 16 + 15) / G);
    const bool wave_live = wave_pos_lo < pos_end;
    const int wave_q_lo = ctx + wave_pos_lo;
    const int wave_q_hi = ctx + wave_pos_hi;

    f32x4_t o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    float lsum = 0.f;   // this lane's share of the row sum
    const float cs = a.scale_log2;

    // ---- K/V tile staging.  The block ids of a tile are read through the
    // constant address space (the kernel never writes the table), so they are
    // scalar loads, fetched one tile ahead.  Each thread's rows are arranged so
    // that its block is the same for the whole wave: the block's base address
    // is scalar and every load is base + a loop-invariant 32-bit lane offset.
    typedef const __attribute__((address_space(4))) int32_t ctab_t;
    const ctab_t* ctab = (const ctab_t*)table;
    auto tile_blocks = [&](int tt, int (&pb)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int blk = tt * 4 + q;
            pb[q] = blk * kBlockSize < n_keys ? ctab[blk] : -1;
        }
    };
    // 16-bit: thread t moves 16-byte chunk t % 16 of row (t / 16) % 16 of blocks
    // 2 i + t / 256 (i = 0, 1) of the tile: a wave's two blocks are uniform.
    const int ck = tid & 15;
    const int rr = (tid >> 4) & 15;
    const int half = uniform(tid >> 8);
    const uint32_t lane_off = (uint32_t)(rr * row_stride + g * kPD + 8 * ck) * 2u;   // bytes
    auto load_tile = [&](int tt, const int (&pb)[4], uint4 (&gk)[2], uint4 (&gv)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = 2 * i + half;
            const int pbq = half ? pb[2 * i + 1] : pb[2 * i];
            const bool ok = pbq >= 0 && (int64_t)pbq < a.num_blocks;
            const int64_t base = (int64_t)(ok ? pbq : 0) * (kBlockSize * row_stride * 2);
            const uint4 k4 = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_cache) + base + lane_off);
            const uint4 v4 = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_cache) + base + lane_off);
            // rows past the keys or in a bad block: V must be zeros (MFMA would turn
            // 0 x NaN into NaN); K there only meets masked scores
            const bool full = ok && tt * kKT + 16 * (q + 1) <= n_keys;   // uniform
            const bool valid = full || (ok && tt * kKT + 16 * q + rr < n_keys);
            gk[i] = k4;
            gv[i] = valid ? v4 : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&](int buf, const uint4 (&gk)[2], const uint4 (&gv)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int kr = 16 * (2 * i + half) + rr;
            *reinterpret_cast<uint4*>(&lds_k[buf][kr * kKRow + 8 * ck]) = gk[i];
            *reinterpret_cast<uint4*>(&lds_v[buf][kr * kVRow + 8 * ck]) = gv[i];
        }
    };
    // ---- FP8 staging: thread t moves the 16 codes 16*(t % 8) .. +16 of key row
    // t / 8 (block t / 128: uniform per wave) and that row's two scales.  Invalid
    // rows stage zeros with k scale 0 and v scale 1, so NaN bits in unused slots
    // never reach the products.
    const int c8 = tid & 7;
    const int kr8 = tid >> 3;       // 0..63
    const int q8 = uniform(tid >> 7);
    const uint32_t lane_off8 = (uint32_t)((kr8 & 15) * row_stride + g * kPD + 16 * c8);   // bytes
    const uint32_t lane_soff = (uint32_t)(g * kBlockSize + (kr8 & 15));                  // floats
    auto load_tile8 = [&](int tt, const int (&pb)[4], uint4& ck8, uint4& cv8, float& ksc, float& vsc) {
        const int pbq = q8 == 0 ? pb[0] : q8 == 1 ? pb[1] : q8 == 2 ? pb[2] : pb[3];
        const bool ok = pbq >= 0 && (int64_t)pbq < a.num_blocks;
        const int64_t pblk = ok ? pbq : 0;
        const int64_t base = pblk * (kBlockSize * row_stride);
        const int64_t sbase = pblk * a.num_kv_heads * kBlockSize;
        const uint4 k4 = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.k_cache) + base + lane_off8);
        const uint4 v4 = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.v_cache) + base + lane_off8);
        const float ks = a.k_scales[sbase + lane_soff];
        const float vs = a.v_scales[sbase + lane_soff];
        const bool valid = ok && tt * kKT + kr8 < n_keys;
        ck8 = valid ? k4 : make_uint4(0, 0, 0, 0);
        cv8 = valid ? v4 : make_uint4(0, 0, 0, 0);
        ksc = valid ? ks : 0.f;
        vsc = valid ? vs : 1.f;
    };
    auto store_tile8 = [&](int buf, const uint4& ck8, const uint4& cv8, float ksc, float vsc) {
        const uint32_t kw[4] = {ck8.x, ck8.y, ck8.z, ck8.w};
        const uint32_t vw[4] = {cv8.x, cv8.y, cv8.z, cv8.w};
        uint2 ke[4], ve[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ke[e] = fp8x4_to_16<DT>(kw[e], 1.f);
            ve[e] = fp8x4_to_16<DT>(vw[e], vsc);
        }
        uint4* kd = reinterpret_cast<uint4*>(&lds_k[buf][kr8 * kKRow + 16 * c8]);
        uint4* vd = reinterpret_cast<uint4*>(&lds_v[buf][kr8 * kVRow + 16 * c8]);
        kd[0] = make_uint4(ke[0].x, ke[0].y, ke[1].x, ke[1].y);
        kd[1] = make_uint4(ke[2].x, ke[2].y, ke[3].x, ke[3].y);
        vd[0] = make_uint4(ve[0].x, ve[0].y, ve[1].x, ve[1].y);
        vd[1] = make_uint4(ve[2].x, ve[2].y, ve[3].x, ve[3].y);
        if (c8 == 0) {
            lds_ks[buf][kr8] = ksc;
            lds_mu[buf][kr8] = scale_mantissa(vsc);
        }
    };
    // transposed V^T fragment address of this lane: row 4*lg + lr/4 (+16), column 4*(lr%4) (+16 mt)
    const int v_tr_off = (4 * lg + (lr >> 2)) * kVRow + 4 * (lr & 3);

    uint4 gk[2], gv[2];
    uint4 ck8, cv8;
    float ksc = 0.f, vsc = 1.f;
    int pbn[4];                     // block ids of the next tile to stage
    tile_blocks(0, pbn);
    if constexpr (F8) {
        load_tile8(0, pbn, ck8, cv8, ksc, vsc);
        store_tile8(0, ck8, cv8, ksc, vsc);
    } else {
        load_tile(0, pbn, gk, gv);
        store_tile(0, gk, gv);
    }
    if (ntiles > 1) tile_blocks(1, pbn);
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        __syncthreads();   // tile t is in LDS; everybody is done with tile t-1's buffer
        const bool more = t + 1 < ntiles;
        if (more) {   // in flight while this tile is computed
            if constexpr (F8) load_tile8(t + 1, pbn, ck8, cv8, ksc, vsc);
            else load_tile(t + 1, pbn, gk, gv);
            if (t + 2 < ntiles) tile_blocks(t + 2, pbn);
        }
        const int k0 = t * kKT;
        if (wave_live && k0 <= wave_q_hi) {
            // ---- S^T = K Q^T for 64 keys x 16 rows
            f32x4_t s[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) s[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const uint4 ka = *reinterpret_cast<const uint4*>(
                        &lds_k[buf][(16 * mt + lr) * kKRow + 32 * kk + 8 * lg]);
                    s[mt] = mfma16x16x32<DT>(ka, qf[kk], s[mt]);
                }
            }
            if constexpr (F8) {   // k scale of each key (keys 16*mt + 4*lg + i)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const float4 ks4 = *reinterpret_cast<const float4*>(&lds_ks[buf][16 * mt + 4 * lg]);
                    s[mt][0] *= ks4.x;
                    s[mt][1] *= ks4.y;
                    s[mt][2] *= ks4.z;
                    s[mt][3] *= ks4.w;
                }
            }

            // ---- online softmax of this lane's row (P overwrites S).  The scale is folded
            // into the exponent (scale > 0, so the max commutes with it).  The running max
            // is raised only when a tile beats it by more than 2^8: otherwise the old max
            // is kept, p <= 256 (exact algebra, no overflow in the 16-bit P), and the
            // rescale of O^T is skipped for the whole wave.
            if (k0 + kKT - 1 > wave_q_lo) {   // diagonal tile: causal mask by select
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (k0 + 16 * mt + 4 * lg + i > qpos) s[mt][i] = -INFINITY;
            }
            float mb = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
            for (int mt = 1; mt < 4; ++mt)
                mb = fmaxf(mb, fmaxf(fmaxf(s[mt][0], s[mt][1]), fmaxf(s[mt][2], s[mt][3])));
            mb = xor32_max(xor16_max(mb));
            const float mbs = mb * cs;
            const bool raise = mbs > m + 8.f;   // also true on the first live tile
            const float mn = raise ? mbs : m;
            if (__any(raise)) {
                const float alpha = raise ? fast_exp2(m - mn) : 1.f;   // exp2(-inf) = 0
                lsum *= alpha;
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
            }
            m = mn;
            const float nmu = mn == -INFINITY ? 0.f : -mn;
            float ps = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = fast_exp2(fmaf(s[mt][i], cs, nmu));
                    s[mt][i] = pv;
                    ps += pv;
                }
            lsum += ps;
            if constexpr (F8) {   // times the v-scale mantissa factor of each key
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const float4 mu4 = *reinterpret_cast<const float4*>(&lds_mu[buf][16 * mt + 4 * lg]);
                    s[mt][0] *= mu4.x;
                    s[mt][1] *= mu4.y;
                    s[mt][2] *= mu4.z;
                    s[mt][3] *= mu4.w;
                }
            }
            // key slot 8*lg + i <-> key 32*kc + 4*lg + i; slot 8*lg + 4 + i <-> key 32*kc + 16 + 4*lg + i
            uint4 pb[2], pt[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                pb[kc].x = pack2<DT>(s[2 * kc][0], s[2 * kc][1]);
                pb[kc].y = pack2<DT>(s[2 * kc][2], s[2 * kc][3]);
                pb[kc].z = pack2<DT>(s[2 * kc + 1][0], s[2 * kc + 1][1]);
                pb[kc].w = pack2<DT>(s[2 * kc + 1][2], s[2 * kc + 1][3]);
                if constexpr (F8) {   // the 16-bit tail of P: what the head's rounding lost
                    pt[kc].x = pack2<DT>(s[2 * kc][0] - lo_to_f32<DT>(pb[kc].x), s[2 * kc][1] - hi_to_f32<DT>(pb[kc].x));
                    pt[kc].y = pack2<DT>(s[2 * kc][2] - lo_to_f32<DT>(pb[kc].y), s[2 * kc][3] - hi_to_f32<DT>(pb[kc].y));
                    pt[kc].z = pack2<DT>(s[2 * kc + 1][0] - lo_to_f32<DT>(pb[kc].z), s[2 * kc + 1][1] - hi_to_f32<DT>(pb[kc].z));
                    pt[kc].w = pack2<DT>(s[2 * kc + 1][2] - lo_to_f32<DT>(pb[kc].w), s[2 * kc + 1][3] - hi_to_f32<DT>(pb[kc].w));
                }
            }

            // ---- O^T += V^T P^T; V^T fragments by transposed LDS reads of the row-major V tile
            const uint16_t* vbuf = lds_v[buf] + v_tr_off;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    const ps16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (ps16x4_t __attribute__((address_space(3)))*)(vbuf + 32 * kc * kVRow + 16 * mt));
                    const ps16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (ps16x4_t __attribute__((address_space(3)))*)(vbuf + (32 * kc + 16) * kVRow + 16 * mt));
                    const uint2 l2 = __builtin_bit_cast(uint2, lo);
                    const uint2 h2 = __builtin_bit_cast(uint2, hi);
                    const uint4 va = make_uint4(l2.x, l2.y, h2.x, h2.y);
                    o[mt] = mfma16x16x32<DT>(va, pb[kc], o[mt]);
                    if constexpr (F8) o[mt] = mfma16x16x32<DT>(va, pt[kc], o[mt]);
                }
            }
        }
        if (more) {
            if constexpr (F8) store_tile8(buf ^ 1, ck8, cv8, ksc, vsc);
            else store_tile(buf ^ 1, gk, gv);
        }
    }

    if (!wave_live) return;
    // ---- epilogue: full row sum, normalise, store the row if it exists
    const float l = xor32_sum(xor16_sum(lsum));
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int pos = pos0 + rho / G;
    if (pos >= L) return;
    uint16_t* dst = static_cast<uint16_t*>(a.out) +
                    ((row0 + pos) * a.num_q_heads + g * G + rho % G) * kPD + 4 * lg;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        uint2 w;
        w.x = pack2<DT>(o[mt][0] * inv, o[mt][1] * inv);
        w.y = pack2<DT>(o[mt][2] * inv, o[mt][3] * inv);
        *reinterpret_cast<uint2*>(dst + 16 * mt) = w;
    }
}

template <int DT, bool F8>
static void launch_prefill_g(const PrefillArgs& a, hipStream_t s, dim3 grid) {
    switch (a.group) {
        case 1: hipLaunchKernelGGL((prefill_kernel<DT, 1, F8>), grid, dim3(512), 0, s, a); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<DT, 2, F8>), grid, dim3(512), 0, s, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<DT, 4, F8>), grid, dim3(512), 0, s, a); break;
        default: hipLaunchKernelGGL((prefill_kernel<DT, 8, F8>), grid, dim3(512), 0, s, a); break;
    }
}

template <bool F8>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
    const int positions = kRows / a.group;
    const int64_t qtiles = (a.max_q_len + positions - 1) / positions;
    const int64_t wgs = qtiles * a.num_seqs * a.num_kv_heads;
    if (wgs == 0) return hipSuccess;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    if (a.dtype == kF16) launch_prefill_g<kF16, F8>(a, s, grid);
    else launch_prefill_g<kBF16, F8>(a, s, grid);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) { return launch_prefill_t<false>(a, s); }
hipError_t launch_prefill_fp8(const PrefillArgs& a, hipStream_t s) { return launch_prefill_t<true>(a, s); }

}  // namespace pa
