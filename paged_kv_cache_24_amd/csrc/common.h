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
