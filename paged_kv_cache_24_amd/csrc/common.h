// Device helpers shared by the gfx950 kernels of libpa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pa {

constexpr int kBlockSize = 16;   // tokens per KV block as the kernels walk the cache
constexpr int kWave = 64;        // CDNA wavefront width

// The kernels walk the cache in 16-token blocks.  A cache of 32-token blocks
// ([NB][32][Hkv][D]) is the same memory as [2 NB][16][Hkv][D]: 16-token block
// j of a sequence is half j % 2 of its table entry j / 2.  `shift` is
// log2(block_size / 16).  A negative entry stays negative, and an entry at or
// above 2^(31 - shift) comes out negative, so the callers' range check on the
// result (against num_blocks << shift) still rejects every bad entry.
__device__ __forceinline__ int sub_block(int entry, int j, int shift) {
    return entry < 0 ? -1 : (int)(((uint32_t)entry << shift) | ((uint32_t)j & ((1u << shift) - 1u)));
}
// The same with the shift known at compile time; a 16-token table (SH = 0)
// already names 16-token blocks, so its entries pass through untouched.
template <int SH>
__device__ __forceinline__ int sub_block(int entry, int j) {
    if constexpr (SH == 0) return entry;
    else return sub_block(entry, j, SH);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- conversion

// low / high 16-bit element of a packed dword, widened to float32
template <int DT>
__device__ __forceinline__ float lo_to_f32(uint32_t w) {
    if constexpr (DT == kF16) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    } else {
        return __uint_as_float(w << 16);
    }
}
template <int DT>
__device__ __forceinline__ float hi_to_f32(uint32_t w) {
    if constexpr (DT == kF16) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    } else {
        return __uint_as_float(w & 0xffff0000u);
    }
}

// float32 -> 16-bit storage, round to nearest even
template <int DT>
__device__ __forceinline__ uint16_t f32_to_bits(float x) {
    if constexpr (DT == kF16) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    } else {
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    }
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// two float32 -> one packed dword of 16-bit values (a in the low half), RNE;
// a single v_cvt_pk_{bf16,f16}_f32
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2_t v = {a, b};
    if constexpr (DT == kF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    }
}

// dot product of two packed pairs, accumulated in float32
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == kF16) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                      c, false);
    } else {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
    }
}

// packed pair (1, 1) of the 16-bit type: dot2(p, kOnes2, s) adds both halves of p to s
template <int DT>
constexpr uint32_t kOnes2 = DT == kF16 ? 0x3C003C00u : 0x3F803F80u;

// 8-element dot product of two 16-byte vectors
template <int DT>
__device__ __forceinline__ float dot8(const uint4& a, const uint4& b) {
    float s = dot2<DT>(a.x, b.x, 0.f);
    s = dot2<DT>(a.y, b.y, s);
    s = dot2<DT>(a.z, b.z, s);
    return dot2<DT>(a.w, b.w, s);
}

// ------------------------------------------------------------ DPP reductions
// DPP control codes (GFX9 encoding)
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // reverse within each 8 lanes
constexpr int kDppMirror = 0x140;     // reverse within each 16 lanes
constexpr int kDppRowRor8 = 0x128;    // rotate each 16-lane row by 8 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N = 8 or 16); every lane gets its group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    if constexpr (N == 16) x += dpp<kDppMirror>(x);
    return x;
}

// Max over aligned groups of N lanes (N = 8 or 16); every lane gets its group's max.
template <int N>
__device__ __forceinline__ float group_max(float x) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    x = fmaxf(x, dpp<kDppQuadXor1>(x));
    x = fmaxf(x, dpp<kDppQuadXor2>(x));
    x = fmaxf(x, dpp<kDppHalfMirror>(x));
    if constexpr (N == 16) x = fmaxf(x, dpp<kDppMirror>(x));
    return x;
}

// Sum over aligned groups of 4 lanes.
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp<kDppQuadXor1>(x);
    return x + dpp<kDppQuadXor2>(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over lanes {l, l^16} and {l, l^32} on the VALU (gfx950 lane
// swaps, no LDS round trip).  permlane16_swap(x, x) returns the even 16-lane
// rows of each row pair in its first result and the odd rows in its second;
// permlane32_swap(x, x) the low and high halves of the wave.
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// --------------------------------------------------------- FP8 (OCP E4M3)
// Hardware conversions of gfx950, both exact where used here:
//  * v_cvt_scalef32_pk_{f16,bf16}_fp8 turns two E4M3 codes into two 16-bit
//    values times 2^e, e the exponent of the scale operand (its mantissa is
//    ignored).  Every E4M3 value is exact in fp16 and bf16.
//  * v_cvt_pk_f32_fp8 turns two codes into two float32.
//  * v_cvt_pk_fp8_f32 rounds two float32 to E4M3, nearest-even; inputs must
//    already be clamped to +-448 (it does not saturate).

// codes 2*HI, 2*HI+1 of w -> packed 16-bit pair, times 2^exponent(pow2_scale)
template <int DT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_16(uint32_t w, float pow2_scale) {
    if constexpr (DT == kF16) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, pow2_scale, HI));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, pow2_scale, HI));
    }
}

// 4 codes of w -> 2 packed 16-bit pairs
template <int DT>
__device__ __forceinline__ uint2 fp8x4_to_16(uint32_t w, float pow2_scale) {
    return make_uint2(fp8x2_to_16<DT, false>(w, pow2_scale), fp8x2_to_16<DT, true>(w, pow2_scale));
}

// codes 2*HI, 2*HI+1 of w -> two float32 (exact)
template <bool HI>
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// 1 <= mantissa factor < 2 with s = 2^e * factor (s positive, normal): the part
// of a scale that the conversions above leave out
__device__ __forceinline__ float scale_mantissa(float s) {
    return __uint_as_float((__float_as_uint(s) & 0x007fffffu) | 0x3f800000u);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte K/V load.  NT: marked non-temporal, for calls in which no block is
// read twice -- the streaming hint lets HBM reads run measurably faster on
// gfx950, but it also keeps shared (prefix) blocks from being served from cache.
template <bool NT>
__device__ __forceinline__ uint4 load_kv(const uint16_t* p) {
    if constexpr (NT) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ------------------------------------------------------- decode work order
// A decode wave's work item: one partition of one (sequence, kv head, q-head
// chunk) unit.  Items are numbered partition-major, so that every sequence's
// first partitions run first and the empty items of short sequences (partitions
// past their end) cluster at the end of the grid; then by sequence, kv head and
// head chunk, so that adjacent workgroups read all kv heads of a block -- one
// contiguous stretch of the pool -- at about the same time.
//
// When blocks may be shared (no PA_DECODE_STREAM_KV: a prefix held once for a
// group of consecutive sequences), the workgroup index is also permuted so
// that runs of kXcdRun consecutive workgroups execute on one XCD: the
// dispatcher deals workgroup x to XCD x % 8, and each XCD has its own L2, so
// the sequences of a run read a shared block through one L2 instead of
// several.  The XCD of a run rotates by one from each round of eight runs to
// the next, so that no XCD is tied to the same sequences in every partition.
constexpr int kXcds = 8;
constexpr int kXcdRun = 32;

// Workgroup index after the XCD-run permutation above (identity when NT).
template <bool NT>
__device__ __forceinline__ int64_t decode_workgroup() {
    int64_t x = blockIdx.x;
    if constexpr (!NT) {
        constexpr int64_t R = (int64_t)kXcds * kXcdRun;
        if (x < (int64_t)(gridDim.x / R) * R) {   // whole rounds of R workgroups; the rest unpermuted
            const int64_t t = x / kXcds;
            const int64_t round = t / kXcdRun;
            // run (round, slot) executes on XCD (slot + round) % 8
            const int64_t slot = (x % kXcds - round % kXcds + kXcds) % kXcds;
            x = round * R + slot * kXcdRun + t % kXcdRun;
        }
    }
    return x;
}

struct DecodeItem {
    int part, b, g, hc;
};

template <bool NT>
__device__ __forceinline__ bool decode_item(const DecodeArgs& a, int wave, DecodeItem& it) {
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.head_chunks;
    const int64_t item = decode_workgroup<NT>() * 4 + wave;
    if (item >= units * a.num_parts) return false;
    it.part = (int)(item / units);
    int64_t u = item - (int64_t)it.part * units;
    it.hc = (int)(u % a.head_chunks);
    u /= a.head_chunks;
    it.g = (int)(u % a.num_kv_heads);
    it.b = (int)(u / a.num_kv_heads);
    return true;
}

// Tokens of sequence b, clamped to what its table row can name.
__device__ __forceinline__ int seq_tokens(const DecodeArgs& a, int b) {
    const int max_tokens = a.max_blocks_per_seq * kBlockSize;
    const int n = a.seq_lens[b];
    return n < 0 ? 0 : (n > max_tokens ? max_tokens : n);
}

__device__ __forceinline__ int ceil_blocks(int n) { return (n + kBlockSize - 1) / kBlockSize; }

// Sum over the 64 lanes; every lane gets it.
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

// Inclusive prefix sum over the lanes in lane order.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off);
        x += lane >= off ? y : 0;
    }
    return x;
}

// ------------------------------------------- balanced split of decode work
// The blocks of all sequences form one stream, sequence after sequence, T =
// sum_b ceil(n_b / 16) blocks.  It is cut into S = num_items / upb equal
// stretches of C = ceil(T / S) blocks (at least kMinStretch), and stretch s is
// processed by upb = num_kv_heads * head_chunks adjacent waves, one per unit
// (kv head, q-head chunk): wave w = s * upb + ui.  Every wave gets the same
// work whatever the mix of lengths, where fixed partitions leave the grid's
// last round to the longest sequences; and the waves that read one block are
// neighbours, so all kv heads of a block -- one contiguous stretch of the pool
// -- leave HBM together.  T and the sequence holding a stretch's first block
// come from a prefix sum of the lengths, a wave-wide scan of seq_lens in
// device memory: nothing is read on the host, so the launch is capturable.
//
// The part of one sequence that one stretch covers is a segment.  A segment
// that is the whole sequence is finished in place; every other one leaves the
// partial state of unit ui in slot (b + s) * upb + ui, which is unique: the
// segments of one sequence fall in consecutive stretches, and a later sequence
// starts in the stretch where the previous one ends or after it.  Slots
// therefore number fewer than (num_seqs + S) * upb.
constexpr int kMinStretch = 16;
constexpr int kStretchStride = 1;

__device__ __forceinline__ int balanced_stretch(const DecodeArgs& a, int total) {
    const int stretches = a.num_items / (a.num_kv_heads * a.head_chunks);
    const int c = (total + stretches - 1) / stretches;
    return c > kMinStretch ? c : kMinStretch;
}

// The block counts of a stream's items (sequences, or the owners of the
// sequence groups) held in registers, lane l holding items l, l + 64, ...: all
// of them arrive in one round of loads, not one dependent round per 64 items
// (under a saturated memory system each round costs microseconds).  Holds up
// to kScanItems items; the launchers check that.
constexpr int kScanRegs = 12;
constexpr int kScanItems = kScanRegs * kWave;

struct BlockCounts {
    int c[kScanRegs];

    template <typename Count>
    __device__ __forceinline__ BlockCounts(int n, Count count) {
        const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
        for (int k = 0; k < kScanRegs; ++k) {
            const int i = k * kWave + lane;
            c[k] = i < n ? count(i) : 0;
        }
    }
    // blocks of the items before `before` (every lane gets it)
    __device__ __forceinline__ int prefix(int before) const {
        const int lane = threadIdx.x & (kWave - 1);
        int t = 0;
#pragma unroll
        for (int k = 0; k < kScanRegs; ++k) t += k * kWave + lane < before ? c[k] : 0;
        return uniform(wave_sum(t));
    }
    __device__ __forceinline__ int total() const { return prefix(kScanItems); }
    // the item holding stream block s (< total), and the stream position of its first block
    __device__ __forceinline__ void locate(int s, int& item, int& pos) const {
        int run = 0;
        item = 0;
        pos = 0;
#pragma unroll
        for (int k = 0; k < kScanRegs; ++k) {
            const int incl = wave_inclusive_scan(c[k]);
            const int sum = uniform(__shfl(incl, kWave - 1));
            if (run + sum > s) {
                const unsigned long long hit = __ballot(run + incl > s);
                const int f = __ffsll(hit) - 1;
                item = k * kWave + f;
                pos = run + __shfl(incl - c[k], f);
                break;
            }
            run += sum;
        }
        item = uniform(item);
        pos = uniform(pos);
    }
};

__device__ __forceinline__ BlockCounts sequence_blocks(const DecodeArgs& a) {
    return BlockCounts(a.num_seqs, [&](int i) { return ceil_blocks(seq_tokens(a, i)); });
}

// Calls segment(b, g, hc, n, j0, j1, whole, slot) for every segment of this
// wave's stretch, in stream order: blocks j0 .. j1-1 of unit (b, g, hc) of a
// sequence of n tokens; whole = the segment is the entire sequence.
template <bool NT, typename Segment>
__device__ __forceinline__ void balanced_walk(const DecodeArgs& a, int wave, Segment&& segment) {
    const int upb = a.num_kv_heads * a.head_chunks;
    const int64_t w = decode_workgroup<NT>() * 4 + wave;
    const int64_t nst = a.num_items / upb;
    int64_t st = w / upb;   // stretch, in dispatch order
    const int ui = (int)(w - st * upb);
    if (st >= nst) return;
    if constexpr (kStretchStride > 1) {   // dispatch order i -> stretch (i % Q) * F + i / Q
        const int64_t f = nst / kStretchStride;
        if (st < f * kStretchStride) st = (st % kStretchStride) * f + st / kStretchStride;
    }
    const BlockCounts counts = sequence_blocks(a);
    const int total = counts.total();
    const int stretch = balanced_stretch(a, total);
    const int64_t lo = st * stretch;
    if (lo >= total) return;
    int s = (int)lo;
    const int s1 = (int)min((int64_t)total, lo + stretch);
    // the sequence b holding block s, and the stream position pb of its first block
    int b, pb;
    counts.locate(s, b, pb);
    const int g = ui / a.head_chunks;
    const int hc = ui - g * a.head_chunks;
    while (s < s1 && b < a.num_seqs) {
        const int n = seq_tokens(a, b);
        const int nblk = ceil_blocks(n);
        if (s >= pb + nblk) {   // past this sequence (also skips empty ones)
            pb += nblk;
            ++b;
            continue;
        }
        const int j0 = s - pb;
        const int j1 = min(nblk, j0 + (s1 - s));
        segment(b, g, hc, n, j0, j1, j0 == 0 && j1 == nblk, ((int64_t)b + st) * upb + ui);
        s += j1 - j0;
    }
}

// ------------------------------------------------- sequence groups' stream
// With sequence groups (shared prefixes) the balanced split runs over owners,
// group after group: the group's shared run, then each member's blocks past
// it (owner_blocks, written by the plan kernel).
constexpr int kMaxGroupSeqs = 5;   // S = 16 / G with G >= 3

__device__ __forceinline__ int group_owners(const DecodeArgs& a) {
    const int groups = (a.num_seqs + a.seqs_per_wave - 1) / a.seqs_per_wave;
    return groups * (a.seqs_per_wave + 1);
}

__device__ __forceinline__ BlockCounts owner_counts(const DecodeArgs& a) {
    return BlockCounts(group_owners(a), [&](int i) { return a.owner_blocks[i]; });
}

// Calls segment(grp, g, sel, j0, j1, cnt, st) for every segment of this wave's
// stretch st (kv head g), in stream order: blocks j0 .. j1-1 of owner
// (group grp, member sel; sel < 0: the group's shared run) of cnt blocks.
template <bool NT, typename Segment>
__device__ __forceinline__ void grouped_walk(const DecodeArgs& a, int wave, Segment&& segment) {
    const int64_t w = decode_workgroup<NT>() * 4 + wave;
    const int64_t nst = a.num_items / a.num_kv_heads;
    const int64_t st = w / a.num_kv_heads;
    const int g = (int)(w - st * a.num_kv_heads);
    if (st >= nst) return;
    const int owners = group_owners(a);
    const BlockCounts counts = owner_counts(a);
    const int total = counts.total();
    const int stretch = balanced_stretch(a, total);
    const int64_t lo = st * stretch;
    if (lo >= total) return;
    int s = (int)lo;
    const int s1 = (int)min((int64_t)total, lo + stretch);
    // the owner o holding block s, and the stream position po of its first block
    int o, po;
    counts.locate(s, o, po);
    const int S1 = a.seqs_per_wave + 1;
    while (s < s1 && o < owners) {
        const int cnt = a.owner_blocks[o];
        if (s >= po + cnt) {   // past this owner (also skips empty ones)
            po += cnt;
            ++o;
            continue;
        }
        const int grp = o / S1;
        const int j0 = s - po;
        const int j1 = min(cnt, j0 + (s1 - s));
        segment(grp, g, o - grp * S1 - 1, j0, j1, cnt, st);
        s += j1 - j0;
    }
}

// Enqueue `kernel(a)` and return the status of that launch itself.  Every kernel
// of the library takes one argument struct by value.  hipLaunchKernel's return
// value belongs to this launch only: an error left on the thread by an earlier,
// unrelated call is neither reported here nor cleared (hipGetLastError would do
// both).
template <typename Args>
inline hipError_t launch(void (*kernel)(Args), dim3 grid, dim3 block, hipStream_t stream,
                         const Args& a) {
    void* args[] = {const_cast<Args*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream);
}

}  // namespace pa
