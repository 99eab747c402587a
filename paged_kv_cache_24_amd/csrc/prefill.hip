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
// Two kernels:
//  * prefill16_kernel (head_dim 128): 32x32x16 matrix-core products, S(t+1) =
//    K Q^T overlapped with the softmax of tile t; described at the kernel.  Over
//    the 16-bit cache K/V tiles go from HBM straight into LDS; over the FP8
//    cache the codes pass through registers and are widened to 16 bits on the
//    way into LDS.
//  * prefill_kernel<.., F8, D> (head_dim 64, either cache): 16x16x32 products
//    over tiles staged through registers, as follows.
//
// Both take the q-head group G at run time: a workgroup's rows are floor(R/G)
// positions times the G q heads that share the kv head (R = 128 or 256 rows),
// so every K/V tile is staged in LDS once for all of them; when G does not
// divide R the last R mod G rows are idle (no q, no store).  Both walk the
// cache in 16-token blocks; a cache of 32-token blocks (template argument
// SH = 1) is read as two 16-token halves per table entry (sub_block).
//
// prefill_kernel.  One workgroup (8 waves) owns 128 query rows of one
// (sequence, kv head).  Each wave
// owns 16 rows (~128 VGPRs, four waves per SIMD).  For each 64-key tile:
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
// Over the FP8 cache (in both kernels), each thread stages 16 or 32 codes of
// one key row ("vLLM-Ascend 原理", §四 on KV-cache quantisation: dequantised
// after the block-table lookup, inside the operator); K enters LDS as exact 16-bit codes
// and its scale multiplies the scores, V enters as codes times 2^e (e = exponent
// of its scale, exact) and the scale's mantissa factor mu in [1, 2) multiplies
// P, which goes to the matrix cores rounded once to 16 bits; the row sum adds
// each rounded weight times 1/mu, the probability the product used, so the
// weights stay consistent with the sum as on the 16-bit cache.  The per-key
// factors (k scale, mu, 1/mu) sit in small LDS arrays beside the tiles.
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

constexpr int kPD = 128;            // head_dim of the 32x32x16 kernel
constexpr int kKT = 64;             // keys per tile
constexpr int kRows = 128;          // query rows per workgroup (8 waves x 16)

typedef short ps16x4_t __attribute__((ext_vector_type(4)));

// Work order.  A workgroup's cost is its number of key tiles, which grows with
// the sequence's cached context and with the q tile's position, so neither the
// q-tile index nor the sequence index orders the work.  Workgroup x takes kv
// head x % Hkv and the (x / Hkv)-th costliest (sequence, q tile) item -- ties
// broken by sequence, then by later q tile first -- so the grid runs
// longest-first and the last wave of workgroups is short.  The workgroup finds
// its item from the lengths in device memory: a search over the tile count t
// for the largest t with more than x / Hkv items of at least t tiles (a
// closed-form count per sequence), in which the eight waves test eight
// candidates per step, then a prefix count over the sequences whose items tie.
struct SeqLens {
    int ctx, len, nq;
    int r0;   // first packed row of the sequence
};

__device__ __forceinline__ SeqLens prefill_seq(const PrefillArgs& a, int b, int P, int max_keys) {
    const int64_t r0 = a.query_start_loc[b];
    const int64_t r1 = min((int64_t)a.query_start_loc[b + 1], a.num_tokens);
    SeqLens s;
    s.len = (r0 < 0 || r1 <= r0) ? 0 : (int)min(r1 - r0, (int64_t)a.max_q_len);
    s.ctx = min(max(a.ctx_lens[b], 0), max_keys);
    s.nq = (s.len + P - 1) / P;
    s.r0 = (int)r0;
    return s;
}

// items of one sequence with at least t key tiles: q tile q has
// min(ctx + min((q + 1) P, len), max_keys) keys
__device__ __forceinline__ int items_with_tiles(const SeqLens& s, int t, int P, int max_keys) {
    if (s.nq == 0) return 0;
    const int w = kKT * (t - 1) + 1;          // tiles >= t  <=>  keys >= w
    if (w > max_keys) return 0;
    const int d = w - s.ctx;
    if (d <= 0) return s.nq;
    if (d > s.len) return 0;
    return s.nq - (d + P - 1) / P + 1;
}

// sum over the wave on the vector ALUs (DPP within 16 lanes, then lane swaps);
// the counts summed here stay far below 2^24, so float adds are exact
__device__ __forceinline__ int wave_sum_i32(int x) {
    return (int)xor32_sum(xor16_sum(group_sum<16>((float)x)));
}

// inclusive prefix sum over the wave's 64 lanes (DPP row shifts, then the
// row broadcasts of lanes 15 and 31)
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return x;
}

// (sequence, q tile) of rank j in the cost order; false if there are fewer
// items.  Called by all waves of the workgroup together (it holds barriers);
// flags is 2 x kSearchWaves ints of LDS that nothing else uses meanwhile.
// The lengths of up to 256 sequences stay in registers (4 per lane); the
// lengths of any further sequences are read again at each step.
constexpr int kSearchWaves = 8;
__device__ __forceinline__ bool prefill_item(const PrefillArgs& a, int P, int64_t j, int& b_out, int& qt_out,
                                             SeqLens& seq_out, int* flags) {
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int max_keys = a.max_blocks_per_seq * kBlockSize;
    constexpr int kHeld = 4;
    SeqLens held[kHeld];
#pragma unroll
    for (int i = 0; i < kHeld; ++i) {
        const int b = lane + 64 * i;
        held[i] = b < a.num_seqs ? prefill_seq(a, b, P, max_keys) : SeqLens{0, 0, 0, 0};
    }
    auto seq_at = [&](int i) -> SeqLens {   // sequence lane + 64 i
        if (i < kHeld) {
            SeqLens s = held[0];
#pragma unroll
            for (int k = 1; k < kHeld; ++k) s = i == k ? held[k] : s;
            return s;
        }
        const int b = lane + 64 * i;
        return b < a.num_seqs ? prefill_seq(a, b, P, max_keys) : SeqLens{0, 0, 0, 0};
    };
    const int chunks = (a.num_seqs + 63) / 64;
    auto count = [&](int t) -> int {   // items with at least t tiles (the same in every lane)
        int c = 0;
#pragma unroll
        for (int i = 0; i < kHeld; ++i) c += items_with_tiles(held[i], t, P, max_keys);
        for (int i = kHeld; i < chunks; ++i) c += items_with_tiles(seq_at(i), t, P, max_keys);
        return wave_sum_i32(c);
    };
    // largest t with count(t) > j: invariant count(lo) > j >= count(hi), with
    // lo = 0 standing for "none yet" (count(0) = all items).  Each step wave w
    // tests candidate lo + 1 + w (hi - lo - 1) / 8; counts fall as t grows, so
    // the passing candidates are a prefix.  Flags alternate between two slots,
    // so one barrier per step suffices.
    int lo = 0, hi = (max_keys + kKT - 1) / kKT + 1;   // count(hi) = 0
    for (int step = 0; hi - lo > 1; ++step) {
        const int c = lo + 1 + (wave * (hi - lo - 1)) / kSearchWaves;   // lo < c < hi
        const bool pass = count(c) > (int)j;
        int* slot = flags + (step & 1) * kSearchWaves;
        if (lane == 0) slot[wave] = pass ? c : -c;
        __syncthreads();
        int nlo = lo, nhi = hi;
#pragma unroll
        for (int w = 0; w < kSearchWaves; ++w) {
            const int v = slot[w];
            nlo = v > 0 ? max(nlo, v) : nlo;
            nhi = v > 0 ? nhi : min(nhi, -v);
        }
        lo = uniform(nlo);
        hi = uniform(nhi);
    }
    if (lo == 0) return false;   // j >= number of items
    int rank = (int)j - count(lo + 1);                  // among the items with exactly lo tiles
    for (int i = 0; i < chunks; ++i) {
        const SeqLens sl = seq_at(i);
        const int above = items_with_tiles(sl, lo + 1, P, max_keys);
        const int eq = items_with_tiles(sl, lo, P, max_keys) - above;
        const int incl = wave_incl_scan(eq);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (rank < total) {
            const uint64_t hit = __ballot(incl > rank && incl - eq <= rank);
            const int src = uniform(__builtin_ctzll(hit));
            b_out = 64 * i + src;
            const int excl = __builtin_amdgcn_readlane(incl - eq, src);
            qt_out = __builtin_amdgcn_readlane(sl.nq - 1 - above, src) - (rank - excl);
            seq_out.ctx = __builtin_amdgcn_readlane(sl.ctx, src);
            seq_out.len = __builtin_amdgcn_readlane(sl.len, src);
            seq_out.nq = __builtin_amdgcn_readlane(sl.nq, src);
            seq_out.r0 = __builtin_amdgcn_readlane(sl.r0, src);
            return true;
        }
        rank -= total;
    }
    return false;
}

static_assert(kRows / 16 == kSearchWaves, "the work-order search takes one candidate per wave");

template <int DT, bool F8, int D, int SH>
__global__ __launch_bounds__(512, 4) void prefill_kernel(PrefillArgs a) {
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    const int G = a.group;          // q heads per kv head, 1 .. kRows
    const int P = kRows / G;        // positions per workgroup; rows P G .. kRows-1 idle
    constexpr int KR = D + 8;       // LDS K row stride (elements): rows 4 banks apart
    constexpr int VR = D + 16;      // LDS V row stride (elements): rows 8 banks apart
    constexpr int KK = D / 32;      // 32-element steps of QK^T
    constexpr int MT = D / 16;      // 16-row blocks of O^T
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKT * KR];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kKT * VR];
    // FP8 only: per-key k scale and v-scale mantissa factor of each staged tile
    __shared__ __attribute__((aligned(16))) float lds_ks[F8 ? 2 : 1][F8 ? kKT : 4];
    __shared__ __attribute__((aligned(16))) float lds_mu[F8 ? 2 : 1][F8 ? kKT : 4];
    __shared__ __attribute__((aligned(16))) float lds_imu[F8 ? 2 : 1][F8 ? kKT : 4];   // 1 / mu

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);   // 0..7: rows 16*wave .. 16*wave+15
    const int lr = lane & 15;       // row (or column) within a 16-wide MFMA tile
    const int lg = lane >> 4;       // lane group 0..3

    // costliest (sequence, q tile) items first
    const int g = blockIdx.x % a.num_kv_heads;
    int b, qtile;
    SeqLens picked;
    __shared__ int search_flags[2 * kSearchWaves];
    if (!prefill_item(a, P, blockIdx.x / a.num_kv_heads, b, qtile, picked, search_flags)) return;   // uniform
    b = uniform(b);
    qtile = uniform(qtile);

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
    // (16-token tables: the stride is max_blocks_per_seq, already in a register)
    const int32_t* table = a.block_tables + (int64_t)b * (SH == 0 ? a.max_blocks_per_seq : a.table_stride);
    const int64_t row_stride = (int64_t)a.num_kv_heads * D;

    // ---- this lane's query row and its Q^T fragments
    uint4 qf[KK];
    const int rho = wave * 16 + lr;
    const bool row_live = rho < P * G;   // a row of this workgroup's positions
    const int qpos = ctx + pos0 + rho / G;
    {
        const int pos = pos0 + rho / G;
        const bool ok = row_live && pos < L;
        const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                              ((row0 + (ok ? pos : 0)) * a.num_q_heads + g * G + rho % G) * D + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qf[kk] = ok ? *reinterpret_cast<const uint4*>(src + 32 * kk) : make_uint4(0, 0, 0, 0);
    }
    const int wave_pos_lo = pos0 + (wave * 16) / G;
    const int wave_pos_hi = min(pos_end - 1, pos0 + (wave * 16 + 15) / G);
    const bool wave_live = wave_pos_lo < pos_end;
    const int wave_q_lo = ctx + wave_pos_lo;
    const int wave_q_hi = ctx + wave_pos_hi;

    f32x4_t o[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
            pb[q] = blk * kBlockSize < n_keys ? sub_block<SH>(ctab[blk >> SH], blk) : -1;
        }
    };
    // 16-bit: a row is CPR 16-byte chunks; thread t moves chunk t % CPR of row
    // (t / CPR) % 16 of blocks QPP i + t / (16 CPR) (i < NI) of the tile, so a
    // wave's blocks are uniform.
    constexpr int CPR = D / 8;
    constexpr int QPP = 32 / CPR;   // blocks per pass of the 512 threads
    constexpr int NI = 4 / QPP;     // passes per tile
    const int ck = tid % CPR;
    const int rr = (tid / CPR) & 15;
    const int part = uniform(tid / (16 * CPR));
    const uint32_t lane_off = (uint32_t)(rr * row_stride + g * D + 8 * ck) * 2u;   // bytes
    auto load_tile = [&](int tt, const int (&pb)[4], uint4 (&gk)[NI], uint4 (&gv)[NI]) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int q = QPP * i + part;   // uniform
            const int pbq = q == 0 ? pb[0] : q == 1 ? pb[1] : q == 2 ? pb[2] : pb[3];
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
    auto store_tile = [&](int buf, const uint4 (&gk)[NI], const uint4 (&gv)[NI]) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int kr = 16 * (QPP * i + part) + rr;
            *reinterpret_cast<uint4*>(&lds_k[buf][kr * KR + 8 * ck]) = gk[i];
            *reinterpret_cast<uint4*>(&lds_v[buf][kr * VR + 8 * ck]) = gv[i];
        }
    };
    // ---- FP8 staging: a key row is TPR8 runs of 16 codes; thread t < 64 TPR8
    // moves the codes 16*(t % TPR8) .. +16 of key row t / TPR8 (block t / (16
    // TPR8): uniform per wave) and that row's two scales; at D = 64 waves 4..7
    // stage nothing.  Invalid rows stage zeros with k scale 0 and v scale 1, so
    // NaN bits in unused slots never reach the products.
    constexpr int TPR8 = D / 16;
    const bool stage8 = TPR8 == kSearchWaves || wave < TPR8;   // whole waves: 8 at D = 128, 4 at 64
    const int c8 = tid % TPR8;
    const int kr8 = (tid / TPR8) & 63;     // key row 0..63 (a copy for the idle waves)
    const int q8 = uniform(kr8 >> 4);
    const uint32_t lane_off8 = (uint32_t)((kr8 & 15) * row_stride + g * D + 16 * c8);   // bytes
    const uint32_t lane_soff = (uint32_t)(g * kBlockSize + (kr8 & 15));                  // floats
    auto load_tile8 = [&](int tt, const int (&pb)[4], uint4& ck8, uint4& cv8, float& ksc, float& vsc) {
        if (!stage8) return;
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
        if (!stage8) return;
        const uint32_t kw[4] = {ck8.x, ck8.y, ck8.z, ck8.w};
        const uint32_t vw[4] = {cv8.x, cv8.y, cv8.z, cv8.w};
        uint2 ke[4], ve[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ke[e] = fp8x4_to_16<DT>(kw[e], 1.f);
            ve[e] = fp8x4_to_16<DT>(vw[e], vsc);
        }
        uint4* kd = reinterpret_cast<uint4*>(&lds_k[buf][kr8 * KR + 16 * c8]);
        uint4* vd = reinterpret_cast<uint4*>(&lds_v[buf][kr8 * VR + 16 * c8]);
        kd[0] = make_uint4(ke[0].x, ke[0].y, ke[1].x, ke[1].y);
        kd[1] = make_uint4(ke[2].x, ke[2].y, ke[3].x, ke[3].y);
        vd[0] = make_uint4(ve[0].x, ve[0].y, ve[1].x, ve[1].y);
        vd[1] = make_uint4(ve[2].x, ve[2].y, ve[3].x, ve[3].y);
        if (c8 == 0) {
            const float mu = scale_mantissa(vsc);
            lds_ks[buf][kr8] = ksc;
            lds_mu[buf][kr8] = mu;
            lds_imu[buf][kr8] = 1.f / mu;
        }
    };
    // transposed V^T fragment address of this lane: row 4*lg + lr/4 (+16), column 4*(lr%4) (+16 mt)
    const int v_tr_off = (4 * lg + (lr >> 2)) * VR + 4 * (lr & 3);

    uint4 gk[NI], gv[NI];
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
            // ---- S^T = K Q^T for 64 keys x 16 rows (the product phases run at a
            // raised wave priority: a ready product goes ahead of other waves'
            // vector instructions)
            __builtin_amdgcn_s_setprio(2);
            f32x4_t s[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) s[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const uint4 ka = *reinterpret_cast<const uint4*>(
                        &lds_k[buf][(16 * mt + lr) * KR + 32 * kk + 8 * lg]);
                    s[mt] = mfma16x16x32<DT>(ka, qf[kk], s[mt]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
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
                for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
            }
            m = mn;
            const float nmu = mn == -INFINITY ? 0.f : -mn;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = fast_exp2(fmaf(s[mt][i], cs, nmu));
                    s[mt][i] = pv;
                }
            // P enters PV as one 16-bit value per key, and the row sum adds the
            // probabilities those values stand for, so the weights that multiply V
            // sum to exactly l: with a 16-bit cache P itself; over FP8, P times the
            // mantissa mu of the key's v scale (V holds code * 2^e), whose rounded
            // value times 1/mu is the probability the product used.
            float imu[4][4];
            if constexpr (F8) {   // times the v-scale mantissa factor of each key
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const float4 mu4 = *reinterpret_cast<const float4*>(&lds_mu[buf][16 * mt + 4 * lg]);
                    const float4 imu4 = *reinterpret_cast<const float4*>(&lds_imu[buf][16 * mt + 4 * lg]);
                    s[mt][0] *= mu4.x;
                    s[mt][1] *= mu4.y;
                    s[mt][2] *= mu4.z;
                    s[mt][3] *= mu4.w;
                    imu[mt][0] = imu4.x;
                    imu[mt][1] = imu4.y;
                    imu[mt][2] = imu4.z;
                    imu[mt][3] = imu4.w;
                }
            }
            // key slot 8*lg + i <-> key 32*kc + 4*lg + i; slot 8*lg + 4 + i <-> key 32*kc + 16 + 4*lg + i
            uint4 pb[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                pb[kc].x = pack2<DT>(s[2 * kc][0], s[2 * kc][1]);
                pb[kc].y = pack2<DT>(s[2 * kc][2], s[2 * kc][3]);
                pb[kc].z = pack2<DT>(s[2 * kc + 1][0], s[2 * kc + 1][1]);
                pb[kc].w = pack2<DT>(s[2 * kc + 1][2], s[2 * kc + 1][3]);
                if constexpr (F8) {
                    lsum = fmaf(lo_to_f32<DT>(pb[kc].x), imu[2 * kc][0], lsum);
                    lsum = fmaf(hi_to_f32<DT>(pb[kc].x), imu[2 * kc][1], lsum);
                    lsum = fmaf(lo_to_f32<DT>(pb[kc].y), imu[2 * kc][2], lsum);
                    lsum = fmaf(hi_to_f32<DT>(pb[kc].y), imu[2 * kc][3], lsum);
                    lsum = fmaf(lo_to_f32<DT>(pb[kc].z), imu[2 * kc + 1][0], lsum);
                    lsum = fmaf(hi_to_f32<DT>(pb[kc].z), imu[2 * kc + 1][1], lsum);
                    lsum = fmaf(lo_to_f32<DT>(pb[kc].w), imu[2 * kc + 1][2], lsum);
                    lsum = fmaf(hi_to_f32<DT>(pb[kc].w), imu[2 * kc + 1][3], lsum);
                } else {
                    lsum = dot2<DT>(pb[kc].x, kOnes2<DT>, lsum);
                    lsum = dot2<DT>(pb[kc].y, kOnes2<DT>, lsum);
                    lsum = dot2<DT>(pb[kc].z, kOnes2<DT>, lsum);
                    lsum = dot2<DT>(pb[kc].w, kOnes2<DT>, lsum);
                }
            }

            // ---- O^T += V^T P^T; V^T fragments by transposed LDS reads of the row-major V tile
            __builtin_amdgcn_s_setprio(2);
            const uint16_t* vbuf = lds_v[buf] + v_tr_off;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const ps16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (ps16x4_t __attribute__((address_space(3)))*)(vbuf + 32 * kc * VR + 16 * mt));
                    const ps16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (ps16x4_t __attribute__((address_space(3)))*)(vbuf + (32 * kc + 16) * VR + 16 * mt));
                    const uint2 l2 = __builtin_bit_cast(uint2, lo);
                    const uint2 h2 = __builtin_bit_cast(uint2, hi);
                    const uint4 va = make_uint4(l2.x, l2.y, h2.x, h2.y);
                    o[mt] = mfma16x16x32<DT>(va, pb[kc], o[mt]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
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
    if (!row_live || pos >= L) return;
    uint16_t* dst = static_cast<uint16_t*>(a.out) +
                    ((row0 + pos) * a.num_q_heads + g * G + rho % G) * D + 4 * lg;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        uint2 w;
        w.x = pack2<DT>(o[mt][0] * inv, o[mt][1] * inv);
        w.y = pack2<DT>(o[mt][2] * inv, o[mt][3] * inv);
        *reinterpret_cast<uint2*>(dst + 16 * mt) = w;
    }
}

// ---------------------------------------------------------------------------
// head_dim 128: prefill on 32x32x16 matrix-core products, software-pipelined.
//
// One workgroup (8 waves) owns 256 query rows of one (sequence, kv head); each
// wave owns 32 rows, so every K/V fragment read from LDS feeds a 32-row product
// (half the LDS bytes per flop of 16-row waves).  Per 64-key tile and wave:
//   S^T[key][row] = K Q^T : 2 key blocks x 8 steps of v_mfma_f32_32x32x16
//     (A = K rows from LDS, B = Q^T kept in registers); lane l holds 16 keys
//     8*(r/4) + 4*(l/32) + r%4 of row l%32 per key block, so a row lives in
//     lanes l and l^32 only;
//   O^T[d][row] += V^T P^T : 4 d blocks x 4 steps of 16 keys (A = V^T
//     fragments by ds_read_b64_tr_b16, B = P^T straight from the lane's own
//     probabilities: step ks uses accumulator values 8*(ks%2) .. +7 of key
//     block ks/2, which are keys 16 ks + 4 (l/32) + {0..3, 8..11}).
// K/V tiles go from HBM straight into LDS (global_load_lds_dwordx4: a wave's
// 64 lanes fill 1 KiB = 4 token rows; waves 0..3 copy K, waves 4..7 V, four
// LDS buffers of each), with the 16-byte chunks of each row permuted by an XOR
// of the row index so that neither the K fragment reads nor the transposed V
// reads meet bank conflicts.  The two waves on a SIMD work half a tile apart
// (one does S, softmax, PV of tile t; the other PV of tile t-1, then S and
// softmax of tile t), so that one wave's softmax runs on the vector ALUs while
// the other's products keep the matrix core busy; the product phases run at a
// raised wave priority, so that a ready product is not held back by the other
// wave's vector instructions.
// The softmax is optimistic: probabilities are taken against the running max m
// and only if some score exceeds m by more than 2^8 (log2 domain) is the row max
// raised, O and the sum rescaled and the tile redone -- an exact rewrite of the
// softmax ("vLLM-Ascend 原理", §四 ATB fused attention), with p <= 256.
// Row sums add the same 16-bit probabilities that enter the PV product.
// Over the FP8 cache (F8) the same waves move the same blocks, but through
// registers: the codes of tile t+1 are loaded as tile t begins and widened into
// the 16-bit layout at its end (two LDS buffers would do; the four of the
// 16-bit ring are kept), and the softmax applies the per-key factors.

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int DT>
__device__ __forceinline__ f32x16_t mfma32x32x16(const uint4& a, const uint4& b, f32x16_t c) {
    if constexpr (DT == kF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
}

// 16-byte global -> LDS copy of each lane's bytes at sbase + voff (sbase a
// wave-uniform 64-bit base in scalar registers, voff a 32-bit per-lane offset,
// so that no address arithmetic runs on the vector ALUs); the wave's LDS
// destination is lds_base + kLdsOff + 16 * lane.  Written as an instruction the
// compiler does not model, so that it adds no waits of its own for these
// copies: the kernel waits for them explicitly (vmcnt) before the barrier that
// publishes a buffer, and no buffer is read in the tile in which it is being
// filled.  The copy takes its LDS base from m0, formed in m0 itself so that no
// per-copy constants occupy scalar registers; the sequence saves and restores
// m0, so whatever the compiler keeps there is left as it was.
template <uint32_t kLdsOff>
__device__ __forceinline__ void load_lds16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_add_u32 m0, %3, %4\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(voff), "s"(sbase), "s"(lds_base), "i"(kLdsOff)
                 : "scc");
}

constexpr int kTileElems = kKT * kPD;   // one K or V tile in LDS, 16 KiB

constexpr int kW16 = 8;                 // waves per workgroup
static_assert(kW16 == kSearchWaves, "the work-order search takes one candidate per wave");
constexpr int kRows16 = 32 * kW16;      // query rows per workgroup
constexpr int kQkAhead = 6;             // K fragment reads in flight ahead of the products
constexpr int kPvAhead = 4;             // products whose V fragments are read ahead

template <int DT, int SH, bool F8>
__global__ __launch_bounds__(64 * kW16, 1) void prefill16_kernel(PrefillArgs a) {
    static_assert(!F8 || SH == 0, "FP8 pools come in 16-token blocks");
    const int G = a.group;          // q heads per kv head, 1 .. kRows16
    const int P = kRows16 / G;      // positions per workgroup; rows P G .. kRows16-1 idle
    // separate arrays so that the compiler can tell the in-flight copies from
    // the buffers being read
    __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t lds_k2[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t lds_k3[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t lds_v2[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t lds_v3[kTileElems];
    // FP8 only, per key of each buffered tile: k scale times scale_log2; the
    // mantissa factor mu of the v scale; 1/mu as two 16-bit parts (hi, lo) in
    // pair order (word 2p: the hi parts of keys 2p, 2p+1; word 2p+1: their lo parts)
    __shared__ __attribute__((aligned(16))) float lds_c1[F8 ? 4 : 1][F8 ? kKT : 4];
    __shared__ __attribute__((aligned(16))) float lds_mu[F8 ? 4 : 1][F8 ? kKT : 4];
    __shared__ __attribute__((aligned(16))) uint32_t lds_imu[F8 ? 4 : 1][F8 ? kKT : 4];
    auto kbuf = [&](auto i) __attribute__((always_inline)) -> uint16_t* {
        constexpr int I = decltype(i)::value;
        return I == 0 ? lds_k0 : I == 1 ? lds_k1 : I == 2 ? lds_k2 : lds_k3;
    };
    auto vbuf = [&](auto i) __attribute__((always_inline)) -> uint16_t* {
        constexpr int I = decltype(i)::value;
        return I == 0 ? lds_v0 : I == 1 ? lds_v1 : I == 2 ? lds_v2 : lds_v3;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);   // 0..7: rows 32*wave .. 32*wave+31
    const int lr = lane & 31;
    const int h = lane >> 5;

    const int g = blockIdx.x % a.num_kv_heads;
    int b, qtile;
    SeqLens picked;   // the search's own (clamped) lengths of sequence b
    // the search's flags live in the last K buffer, which no copy fills before
    // the first barrier of the tile loop
    if (!prefill_item(a, P, blockIdx.x / a.num_kv_heads, b, qtile, picked, reinterpret_cast<int*>(lds_k3)))
        return;               // uniform
    b = uniform(b);           // the same in every lane: let the compiler know
    qtile = uniform(qtile);
    const int64_t row0 = uniform(picked.r0);
    const int L = uniform(picked.len);   // > 0: the sequence has this item
    const int max_keys = a.max_blocks_per_seq * kBlockSize;
    const int ctx = uniform(picked.ctx);
    const int pos0 = qtile * P;
    if (qtile < 0 || pos0 >= L) return;
    const int pos_end = min(L, pos0 + P);
    const int n_keys = min(ctx + pos_end, max_keys);
    const int ntiles = (n_keys + kKT - 1) / kKT;
    // (16-token tables: the stride is max_blocks_per_seq, already in a register)
    const int32_t* table = a.block_tables + (int64_t)b * (SH == 0 ? a.max_blocks_per_seq : a.table_stride);
    const int64_t row_stride = (int64_t)a.num_kv_heads * kPD;

    // ---- Q^T fragments: row rho, elements 16 kk + 8 h .. +7
    uint4 qf[8];
    const int rho = wave * 32 + lr;
    const bool row_live = rho < P * G;   // a row of this workgroup's positions
    const int qpos = ctx + pos0 + rho / G;
    {
        const int pos = pos0 + rho / G;
        const bool ok = row_live && pos < L;
        const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                              ((row0 + (ok ? pos : 0)) * a.num_q_heads + g * G + rho % G) * kPD + 8 * h;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            qf[kk] = ok ? *reinterpret_cast<const uint4*>(src + 16 * kk) : make_uint4(0, 0, 0, 0);
    }
    const int wave_pos_lo = pos0 + (wave * 32) / G;
    const int wave_q_lo = ctx + wave_pos_lo;
    const bool has_rows = wave_pos_lo < pos_end;   // uniform

    // ---- staging.  Waves 0..3 copy the K blocks and waves 4..7 the V blocks:
    // wave w copies block q = w % 4 of each tile (tile rows 16 q .. 16 q + 15) as
    // 4 copies of 4 token rows.  Lane i writes LDS slot i % 16 of
    // row 4 j + i / 16 and so reads chunk (i % 16) ^ f(row) of that token row:
    // f = row & 15 for K, (row & 3) << 2 for V.  Rows past the last key read the
    // block's first row (blocks past it the sequence's first block): any finite
    // data will do, since their probabilities are exactly 0.
    typedef const __attribute__((address_space(4))) int32_t ctab_t;
    const ctab_t* ctab = (const ctab_t*)table;
    const uint32_t rs2 = (uint32_t)(row_stride * 2);          // bytes between token rows
    const int64_t block_bytes = (int64_t)kBlockSize * rs2;
    const uint32_t goff = (uint32_t)(g * kPD * 2);
    const int l15 = lane & 15;
    const int l4 = lane >> 4;
    // chunk of copy j: l15 ^ (4 j + l4) = (l15 ^ l4) ^ 4 j
    const bool kwave = wave < 4;          // uniform: this wave copies K (else V)
    const int q = wave & 3;               // block of the tile this wave copies
    const uint32_t koff0 = goff + (uint32_t)((l15 ^ l4) << 4);
    const uint32_t voff = goff + (uint32_t)((l15 ^ (l4 << 2)) << 4);
    const int nb32 = (int)min(a.num_blocks, (int64_t)INT32_MAX);
    int first_blk = sub_block<SH>(ctab[0], 0);
    first_blk = first_blk >= 0 && first_blk < nb32 ? first_blk : 0;

    // Block ids are read through the constant address space (scalar loads): for
    // the copies of a tile, one tile ahead, so that the load has returned by the
    // time the next barrier has passed.  Ids of blocks past the keys become the
    // sequence's first block, ids out of range block 0.
    const int key_blocks = (n_keys + kBlockSize - 1) / kBlockSize;   // >= 1, <= max_blocks_per_seq
    auto raw_block = [&](int tt) __attribute__((always_inline)) -> int {   // uniform, branch-free
        const int blk = tt * 4 + q;
        const int pb = ctab[min(blk, key_blocks - 1) >> SH];
        return blk < key_blocks ? sub_block<SH>(pb, blk) : first_blk;
    };
    auto valid_block = [&](int pb) __attribute__((always_inline)) -> int { return pb >= 0 && pb < nb32 ? pb : 0; };
    auto block_of_scalar = [&](int tt) __attribute__((always_inline)) -> int { return valid_block(raw_block(tt)); };
    // byte offset of this lane's 16 bytes of copy j within a block
    uint32_t coff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        coff[j] = (uint32_t)(4 * j + l4) * rs2 + (kwave ? (koff0 ^ (uint32_t)(j << 6)) : voff);
    // copies this wave's block of tile tt into dst (a K buffer for K waves, V for V waves)
    auto stage = [&](int tt, int pb, uint16_t* dst) __attribute__((always_inline)) {
        const int nval = n_keys - (tt * kKT + 16 * q);   // valid rows of this block (uniform)
        const char* src = static_cast<const char*>(kwave ? a.k_cache : a.v_cache) + pb * block_bytes;
        const uint32_t lb = uniform((uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)(dst + 16 * q * kPD));
        constexpr uint32_t kRow4 = 4 * kPD * 2;   // LDS bytes of 4 token rows
        if (nval >= kBlockSize) {
            load_lds16_sv<0 * kRow4>(src, coff[0], lb);
            load_lds16_sv<1 * kRow4>(src, coff[1], lb);
            load_lds16_sv<2 * kRow4>(src, coff[2], lb);
            load_lds16_sv<3 * kRow4>(src, coff[3], lb);
        } else {   // the sequence's last, partial block
            auto off = [&](int j) __attribute__((always_inline)) -> uint32_t {
                const int r = 4 * j + l4;
                return r < nval ? coff[j] : coff[j] - (uint32_t)r * rs2;
            };
            load_lds16_sv<0 * kRow4>(src, off(0), lb);
            load_lds16_sv<1 * kRow4>(src, off(1), lb);
            load_lds16_sv<2 * kRow4>(src, off(2), lb);
            load_lds16_sv<3 * kRow4>(src, off(3), lb);
        }
    };

    // ---- FP8 staging, through registers.  Wave w moves block q of each tile as
    // above: lane i takes token row r8 = i / 4 of the block, codes 32 (i % 4) ..
    // +31, and that row's scale.  The codes of tile t+1 are loaded as tile t
    // begins and at its end widened to 16 bits (K exact, V times 2^e, e the
    // exponent of the row's v scale) and written to the tile's buffers in the layout above
    // (chunk c of tile row R at slot c ^ f(R)), with the per-key factors.  Rows
    // past the keys or in a block outside the pool stage zero codes with k scale
    // 1 and v scale 1; the choice is applied when the codes are widened, so that
    // nothing waits for the loads before then.
    const int r8 = lane >> 2;
    const int p8 = lane & 3;
    const uint32_t off8 = (uint32_t)(r8 * row_stride + g * kPD + 32 * p8);   // bytes
    const uint32_t soff8 = (uint32_t)((g * kBlockSize + r8) * 4);             // bytes
    struct Staged8 {
        uint4 c0, c1;
        float sc;
        bool ok;
    };
    Staged8 st8;
    auto load8 = [&](int tt, int pb, Staged8& st) __attribute__((always_inline)) {
        const int nval = n_keys - (tt * kKT + 16 * q);   // valid rows of this block (uniform)
        const bool blk_ok = pb >= 0 && pb < nb32;        // uniform
        const int64_t pblk = blk_ok ? pb : 0;
        const char* src = static_cast<const char*>(kwave ? a.k_cache : a.v_cache) + pblk * (kBlockSize * row_stride);
        const char* ssrc = reinterpret_cast<const char*>(kwave ? a.k_scales : a.v_scales) +
                           pblk * ((int64_t)a.num_kv_heads * kBlockSize * 4);
        st.c0 = *reinterpret_cast<const uint4*>(src + off8);
        st.c1 = *reinterpret_cast<const uint4*>(src + off8 + 16);
        st.sc = *reinterpret_cast<const float*>(ssrc + soff8);
        st.ok = blk_ok && r8 < nval;
    };
    auto store8 = [&](const Staged8& st, auto par) __attribute__((always_inline)) {
        constexpr int B = decltype(par)::value;
        const uint32_t w[8] = {st.c0.x, st.c0.y, st.c0.z, st.c0.w, st.c1.x, st.c1.y, st.c1.z, st.c1.w};
        const float sc = st.ok ? st.sc : 1.f;
        uint2 e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = fp8x4_to_16<DT>(st.ok ? w[k] : 0u, kwave ? 1.f : sc);
        char* dst = reinterpret_cast<char*>(kwave ? kbuf(par) : vbuf(par));
        const int R = 16 * q + r8;
        const int f = kwave ? r8 : (r8 & 3) << 2;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<uint4*>(dst + R * kPD * 2 + (((4 * p8 + c) ^ f) << 4)) =
                make_uint4(e[2 * c].x, e[2 * c].y, e[2 * c + 1].x, e[2 * c + 1].y);
        if (p8 == 0) {
            if (kwave) {
                lds_c1[B][R] = sc * a.scale_log2;
            } else {
                const float mu = scale_mantissa(sc);
                const float imu = 1.f / mu;
                const uint16_t hi = f32_to_bits<DT>(imu);
                const uint16_t lo = f32_to_bits<DT>(imu - lo_to_f32<DT>(hi));
                lds_mu[B][R] = mu;
                uint16_t* iw = reinterpret_cast<uint16_t*>(lds_imu[B]);
                iw[4 * (R >> 1) + (R & 1)] = hi;
                iw[4 * (R >> 1) + 2 + (R & 1)] = lo;
            }
        }
    };

    // ---- LDS read addresses (bytes).  K fragment of step kk: row 32 kb + lr,
    // chunk 2 kk + h, stored at slot (2 kk + h) ^ (lane & 15).
    uint32_t kaddr[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kaddr[kk] = (uint32_t)(lr * kPD + (((2 * kk + h) ^ l15) << 3)) * 2u;
    // V^T fragments: within each 16-lane group (h, dsub) lane j reads 4 elements of
    // row 4 h + j / 4 (+ 8, + 16 ks), columns 32 db + 16 dsub + 4 (j % 4)
    const int jq = l15 >> 2;
    const int dsub = (lane >> 4) & 1;
    uint32_t vaddr[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int slot = 4 * (db ^ jq) + 2 * dsub + ((l15 >> 1) & 1);
        vaddr[db] = (uint32_t)((4 * h + jq) * kPD + slot * 8 + 4 * (l15 & 1)) * 2u;
    }

    f32x16_t o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    f32x16_t sc[2];                 // S^T of the current tile
    float m = -INFINITY;            // running max of the lane's row (log2 domain, scaled)
    float lsum0 = 0.f, lsum1 = 0.f; // this lane's share of the row sum
    const float cs = a.scale_log2;

    auto qk = [&](const uint16_t* kbuf, f32x16_t (&s)[2]) __attribute__((always_inline)) {
        const char* base = reinterpret_cast<const char*>(kbuf);
        __builtin_amdgcn_s_setprio(2);   // the matrix core is the shared resource
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint4 ka = *reinterpret_cast<const uint4*>(base + kaddr[kk] + kb * 32 * kPD * 2);
                s[kb] = mfma32x32x16<DT>(ka, qf[kk], s[kb]);
            }
        // K reads kQkAhead products ahead of their use
        __builtin_amdgcn_sched_group_barrier(0x100, kQkAhead, 2);
#pragma unroll
        for (int i = 0; i < 16 - kQkAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kQkAhead, 2);
        __builtin_amdgcn_s_setprio(0);
    };

    // Pipeline.  At tile t the products read K(t), V(t) and (late waves, see
    // below) V(t-1).  K waves copy K(t+3) into the buffer of K(t-1) (at the end
    // of tile t), V waves copy V(t+2) into that of V(t-2) (after tile t's
    // barrier): both last read before this tile's barrier.  Every wave issues 4
    // copies per tile, so a K wave waiting until at most 8 are outstanding has
    // K(t) in LDS, and a V wave waiting until at most 4 has V(t).  Tiles past
    // the last are clamped to it: those copies refill buffers nobody reads again.
    // prologue: K(0..2) or V(0..1)
    const int clampt = ntiles - 1;
    if constexpr (F8) {
        load8(0, raw_block(0), st8);
        store8(st8, I0());
    } else {   // all block ids first: their loads are then in flight together
        const int id0 = block_of_scalar(0);
        const int id1 = block_of_scalar(min(1, clampt));
        const int id2 = block_of_scalar(min(2, clampt));
        if (kwave) {
            stage(0, id0, lds_k0);
            stage(min(1, clampt), id1, lds_k1);
            stage(min(2, clampt), id2, lds_k2);
        } else {
            stage(0, id0, lds_v0);
            stage(min(1, clampt), id1, lds_v1);
        }
    }
    const int ahead = F8 ? 1 : kwave ? 3 : 2;   // tiles between the products and this wave's copies
    int pb_next = raw_block(min(ahead, clampt));
    // everything, Q included: the prologue copies were issued back to back, so
    // this costs little more than waiting for the first ones, and afterwards no
    // load the compiler knows of is outstanding inside the loop (over FP8 the
    // compiler places the waits for its own loads)
    if constexpr (!F8) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    // ---- O^T += V^T P^T over one tile
    auto pv = [&](const uint16_t* vb, const uint4 (&pb)[4]) __attribute__((always_inline)) {
        const char* vbase = reinterpret_cast<const char*>(vb);
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const ps16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (ps16x4_t __attribute__((address_space(3)))*)(vbase + vaddr[db] + (16 * ks) * kPD * 2));
                const ps16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (ps16x4_t __attribute__((address_space(3)))*)(vbase + vaddr[db] + (16 * ks + 8) * kPD * 2));
                const uint2 l2 = __builtin_bit_cast(uint2, lo);
                const uint2 h2 = __builtin_bit_cast(uint2, hi);
                o[db] = mfma32x32x16<DT>(make_uint4(l2.x, l2.y, h2.x, h2.y), pb[ks], o[db]);
            }
        // V reads (two per product) kPvAhead products ahead of their use
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvAhead, 1);
#pragma unroll
        for (int i = 0; i < 16 - kPvAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kPvAhead, 1);
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- softmax of tile t: S(t) becomes probabilities pb (16-bit) against the
    // running max; their sums are added to the row sums
    auto softmax = [&](int t, uint4 (&pb)[4]) __attribute__((always_inline)) {
        const int k0 = t * kKT;
        if (k0 + kKT - 1 > wave_q_lo) {   // diagonal tile: causal mask by select
            const int lim = qpos - k0 - 4 * h;   // key offset 32 kb + 8 (r/4) + r%4 must not exceed it
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sc[kb][r] = -INFINITY;
        }
        float lmax0 = -INFINITY, lmax1 = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            lmax0 = __builtin_elementwise_maximum(lmax0, sc[0][r]);
            lmax1 = __builtin_elementwise_maximum(lmax1, sc[1][r]);
        }
        const float lmax = __builtin_elementwise_maximum(lmax0, lmax1);
        auto probs = [&](float nmu) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kb = ks >> 1, r0 = 8 * (ks & 1);
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[i] = pack2<DT>(fast_exp2(fmaf(sc[kb][r0 + 2 * i], cs, nmu)),
                                     fast_exp2(fmaf(sc[kb][r0 + 2 * i + 1], cs, nmu)));
                pb[ks] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        };
        probs(m == -INFINITY ? 0.f : -m);
        if (__any(lmax * cs > m + 8.f)) {   // raise the row max (rows of lanes l, l^32 agree)
            const float mb = xor32_max(lmax) * cs;
            const bool raise = mb > m + 8.f;
            const float mn = raise ? mb : m;
            const float alpha = raise ? fast_exp2(m - mn) : 1.f;   // exp2(-inf) = 0
            lsum0 *= alpha;
            lsum1 *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] *= alpha;
            m = mn;
            const uint4 keep[4] = {pb[0], pb[1], pb[2], pb[3]};
            probs(m == -INFINITY ? 0.f : -m);
            if (!raise) {   // rows whose max stays: their probabilities were right
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) pb[ks] = keep[ks];
            }
        }
#pragma unroll
        for (int ks = 0; ks < 4; ks += 2) {
            lsum0 = dot2<DT>(pb[ks].x, kOnes2<DT>, lsum0);
            lsum1 = dot2<DT>(pb[ks].y, kOnes2<DT>, lsum1);
            lsum0 = dot2<DT>(pb[ks].z, kOnes2<DT>, lsum0);
            lsum1 = dot2<DT>(pb[ks].w, kOnes2<DT>, lsum1);
            lsum0 = dot2<DT>(pb[ks + 1].x, kOnes2<DT>, lsum0);
            lsum1 = dot2<DT>(pb[ks + 1].y, kOnes2<DT>, lsum1);
            lsum0 = dot2<DT>(pb[ks + 1].z, kOnes2<DT>, lsum0);
            lsum1 = dot2<DT>(pb[ks + 1].w, kOnes2<DT>, lsum1);
        }
    };

    // ---- softmax over the FP8 cache.  x = S k_scale scale_log2 - m per key (the
    // factor from LDS; the mask applies to x, so a zero scale never meets -inf);
    // P times mu of each key goes to the PV product rounded once, and the row
    // sums add each rounded weight times 1/mu (two 16-bit parts, so v_dot2 takes
    // them exactly to float32 accuracy).  m = -inf means reference 0: the first
    // live tile always raises the max.
    auto softmax8 = [&](int t, auto par, uint4 (&pb)[4]) __attribute__((always_inline)) {
        constexpr int B = decltype(par)::value;
        const float nmu = m == -INFINITY ? 0.f : -m;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {   // keys 32 kb + 8 j + 4 h + i
                const float4 c = *reinterpret_cast<const float4*>(&lds_c1[B][32 * kb + 8 * j + 4 * h]);
                sc[kb][4 * j] = fmaf(sc[kb][4 * j], c.x, nmu);
                sc[kb][4 * j + 1] = fmaf(sc[kb][4 * j + 1], c.y, nmu);
                sc[kb][4 * j + 2] = fmaf(sc[kb][4 * j + 2], c.z, nmu);
                sc[kb][4 * j + 3] = fmaf(sc[kb][4 * j + 3], c.w, nmu);
            }
        const int k0 = t * kKT;
        if (k0 + kKT - 1 > wave_q_lo) {   // diagonal tile: causal mask by select
            const int lim = qpos - k0 - 4 * h;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sc[kb][r] = -INFINITY;
        }
        float lmax0 = -INFINITY, lmax1 = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            lmax0 = __builtin_elementwise_maximum(lmax0, sc[0][r]);
            lmax1 = __builtin_elementwise_maximum(lmax1, sc[1][r]);
        }
        const float lmax = __builtin_elementwise_maximum(lmax0, lmax1);
        // word i of pb[ks] holds keys 16 ks + 8 (i / 2) + 4 h + 2 (i % 2) + {0, 1}
        auto probs = [&](float sub) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kb = ks >> 1, r0 = 8 * (ks & 1);
                const float4 mu0 = *reinterpret_cast<const float4*>(&lds_mu[B][16 * ks + 4 * h]);
                const float4 mu1 = *reinterpret_cast<const float4*>(&lds_mu[B][16 * ks + 8 + 4 * h]);
                const float mu[8] = {mu0.x, mu0.y, mu0.z, mu0.w, mu1.x, mu1.y, mu1.z, mu1.w};
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[i] = pack2<DT>(fast_exp2(sc[kb][r0 + 2 * i] - sub) * mu[2 * i],
                                     fast_exp2(sc[kb][r0 + 2 * i + 1] - sub) * mu[2 * i + 1]);
                pb[ks] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        };
        probs(0.f);
        const float lim_x = m == -INFINITY ? -INFINITY : 8.f;
        if (__any(lmax > lim_x)) {   // raise the row max (rows of lanes l, l^32 agree)
            const float mb = xor32_max(lmax);   // relative to m, or absolute while m = -inf
            const bool raise = mb > lim_x;
            const float mn = raise ? (m == -INFINITY ? mb : m + mb) : m;
            const float alpha = raise ? fast_exp2(m - mn) : 1.f;   // exp2(-inf) = 0
            lsum0 *= alpha;
            lsum1 *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] *= alpha;
            m = mn;
            probs(raise ? mb : 0.f);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {   // (hi, lo) of 1/mu for the pairs of words 0, 1 and 2, 3
            const uint4 i0 = *reinterpret_cast<const uint4*>(&lds_imu[B][16 * ks + 4 * h]);
            const uint4 i1 = *reinterpret_cast<const uint4*>(&lds_imu[B][16 * ks + 8 + 4 * h]);
            lsum0 = dot2<DT>(pb[ks].x, i0.x, lsum0);
            lsum1 = dot2<DT>(pb[ks].x, i0.y, lsum1);
            lsum0 = dot2<DT>(pb[ks].y, i0.z, lsum0);
            lsum1 = dot2<DT>(pb[ks].y, i0.w, lsum1);
            lsum0 = dot2<DT>(pb[ks].z, i1.x, lsum0);
            lsum1 = dot2<DT>(pb[ks].z, i1.y, lsum1);
            lsum0 = dot2<DT>(pb[ks].w, i1.z, lsum0);
            lsum1 = dot2<DT>(pb[ks].w, i1.w, lsum1);
        }
    };
    auto smax = [&](int t, auto par, uint4 (&pb)[4]) __attribute__((always_inline)) {
        if constexpr (F8) softmax8(t, par, pb);
        else softmax(t, pb);
    };

    // Ping-pong: the two waves on each SIMD (w and w + 4) work half a tile apart.
    // Waves 0..3 do [S(t), softmax(t)] then [PV(t)]; waves 4..7 do [PV(t-1)]
    // then [S(t), softmax(t)], keeping P(t-1) in registers across the barrier.
    // While one wave's softmax keeps the vector ALUs busy, the other wave's
    // products keep the matrix core busy.
    // A wave with rows computes every tile of the workgroup: tiles wholly past its
    // rows' keys are masked to probabilities of exactly 0 (at most one such tile),
    // which costs less than the accumulator copies that skipping them per tile
    // makes the compiler insert.  A wave without rows only copies and syncs.  Each
    // role runs a loop of its own, so that the register allocation of one does not
    // constrain the other's.
    const bool late = !kwave;               // waves 4..7
    uint4 pkeep[4];                         // late waves: P of the previous tile
    constexpr int kIdle = 0, kEarly = 1, kLate = 2;
    auto body = [&](int t, auto par, auto role) __attribute__((always_inline)) {
        constexpr int B = decltype(par)::value;          // t & 3
        constexpr int R = decltype(role)::value;
        uint16_t* kcur = kbuf(std::integral_constant<int, B>());   // K(t)
        const int pb_copy = pb_next;   // block id of this tile's copy
        if constexpr (F8) {
            // tile t was written during tile t-1; the codes of tile t+1 go out now
            __syncthreads();
            load8(min(t + 1, clampt), pb_next, st8);
        } else {
            // K waves copy K(t+3) into the buffer of K(t-1) at the end of the tile
            // (below); V waves copy V(t+2) into that of V(t-2) (read at tile t-2
            // and, by the late waves, at tile t-1) right after the barrier
            if (kwave) __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8): K(t) is in
            else __builtin_amdgcn_s_waitcnt(0x0F74);         // vmcnt(4): V(t) is in
            __syncthreads();
            if (!kwave) stage(min(t + ahead, clampt), valid_block(pb_next), vbuf(std::integral_constant<int, (B + 2) & 3>()));
        }
        // The next copy's block id is a scalar load, which shares its wait counter
        // with the LDS reads and may complete out of order: the first LDS wait
        // after it waits for it too.  It is issued after the K products, so that
        // the softmax (no LDS waits) covers its latency.
        if constexpr (R == kLate) {
            if (B != 0 || t >= 1) pv(vbuf(std::integral_constant<int, (B + 3) & 3>()), pkeep);
            qk(kcur, sc);
            pb_next = raw_block(min(t + 1 + ahead, clampt));
            smax(t, par, pkeep);
        } else if constexpr (R == kEarly) {
            uint4 pb[4];
            qk(kcur, sc);
            pb_next = raw_block(min(t + 1 + ahead, clampt));
            smax(t, par, pb);
            pv(vbuf(std::integral_constant<int, B>()), pb);
        } else {
            pb_next = raw_block(min(t + 1 + ahead, clampt));
        }
        // FP8: widen tile t+1 into its buffers (last read at tile t-3, or t-2 by
        // the late waves' V products); past the last tile this refills buffers
        // that nobody reads again
        if constexpr (F8) store8(st8, std::integral_constant<int, (B + 1) & 3>());
        // the K waves' copy goes out after their PV, where they wait for the next
        // barrier anyway, so that it does not delay this tile's S^T products
        // (1.5% faster than issuing it after the barrier); K(t-1)'s buffer is
        // not read during tile t
        if constexpr (!F8)
            if (kwave) stage(min(t + ahead, clampt), valid_block(pb_copy), kbuf(std::integral_constant<int, (B + 3) & 3>()));
    };
    auto tile_loop = [&](auto role) __attribute__((always_inline)) {
        for (int t = 0; t < ntiles; t += 4) {
            body(t, I0(), role);
            if (t + 1 < ntiles) body(t + 1, I1(), role);
            if (t + 2 < ntiles) body(t + 2, I2(), role);
            if (t + 3 < ntiles) body(t + 3, I3(), role);
        }
    };
    if (!has_rows) tile_loop(std::integral_constant<int, kIdle>());
    else if (late) tile_loop(std::integral_constant<int, kLate>());
    else tile_loop(std::integral_constant<int, kEarly>());
    // late waves: PV of their last tile (its V buffer is not refilled after the loop)
    if (late && has_rows) {
        const int tl = ntiles - 1;
        switch (tl & 3) {
            case 0: pv(lds_v0, pkeep); break;
            case 1: pv(lds_v1, pkeep); break;
            case 2: pv(lds_v2, pkeep); break;
            default: pv(lds_v3, pkeep); break;
        }
    }

    if (!has_rows) return;
    // ---- epilogue: full row sum, normalise, store the row if it exists
    const float l = xor32_sum(lsum0 + lsum1);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int pos = pos0 + rho / G;
    if (!row_live || pos >= L) return;
    uint16_t* dst = static_cast<uint16_t*>(a.out) +
                    ((row0 + pos) * a.num_q_heads + g * G + rho % G) * kPD + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            uint2 w;
            w.x = pack2<DT>(o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv);
            w.y = pack2<DT>(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
            *reinterpret_cast<uint2*>(dst + 32 * db + 8 * r4) = w;
        }
}

template <int DT, bool F8, int D>
static hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t s, dim3 grid) {
    // the block shift is a template argument (a runtime one costs the 16-token
    // case measurable time); FP8 pools only come in 16-token blocks
    if constexpr (!F8) {
        if (a.block_shift == 1) return launch(prefill_kernel<DT, F8, D, 1>, grid, dim3(512), s, a);
    }
    return launch(prefill_kernel<DT, F8, D, 0>, grid, dim3(512), s, a);
}

// the 16x16x32 kernel: head_dim 64, over either cache
template <bool F8>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
    const int positions = kRows / a.group;
    const int64_t qtiles = (a.max_q_len + positions - 1) / positions;
    const int64_t wgs = qtiles * a.num_seqs * a.num_kv_heads;
    if (wgs == 0) return hipSuccess;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    if (a.head_dim != 64) return hipErrorInvalidValue;   // head_dim 128 runs prefill16_kernel
    return a.dtype == kF16 ? launch_prefill_g<kF16, F8, 64>(a, s, grid)
                           : launch_prefill_g<kBF16, F8, 64>(a, s, grid);
}

template <int DT, bool F8>
static hipError_t launch_prefill16_g(const PrefillArgs& a, hipStream_t s, dim3 grid) {
    if constexpr (F8) {   // FP8 pools only come in 16-token blocks
        return launch(prefill16_kernel<DT, 0, true>, grid, dim3(64 * kW16), s, a);
    } else {
        return a.block_shift == 1 ? launch(prefill16_kernel<DT, 1, false>, grid, dim3(64 * kW16), s, a)
                                  : launch(prefill16_kernel<DT, 0, false>, grid, dim3(64 * kW16), s, a);
    }
}

// head_dim 128: the 32x32x16 kernel; head_dim 64: the 16x16x32 one
template <bool F8>
static hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t s) {
    if (a.head_dim != kPD) return launch_prefill_t<F8>(a, s);
    const int positions = kRows16 / a.group;
    const int64_t qtiles = (a.max_q_len + positions - 1) / positions;
    const int64_t wgs = qtiles * a.num_seqs * a.num_kv_heads;
    if (wgs == 0) return hipSuccess;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    return a.dtype == kF16 ? launch_prefill16_g<kF16, F8>(a, s, grid) : launch_prefill16_g<kBF16, F8>(a, s, grid);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) { return launch_prefill_d<false>(a, s); }
hipError_t launch_prefill_fp8(const PrefillArgs& a, hipStream_t s) { return launch_prefill_d<true>(a, s); }

}  // namespace pa
