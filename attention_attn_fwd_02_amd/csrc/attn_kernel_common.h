// attn_kernel_common.h -- device-side helpers shared by the attention kernels
// (prefill, decode, backward, rotary embedding): vector types, wave-pair
// reductions, 16-bit element traits, the rotation of a feature pair and buffer
// resources.  Included by the .hip sources only.
#ifndef ATTN_KERNEL_COMMON_H
#define ATTN_KERNEL_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_internal.h"

namespace attn_impl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

#define NEG_INF (-__builtin_inff())

// ---------------------------------------------------------------------------
// small wave-level helpers
// ---------------------------------------------------------------------------

// v_permlane32_swap on (x, x) leaves, in every lane, the pair {x[lane], x[lane ^ 32]}
// (in an order that depends on the half); the symmetric combinations below are
// therefore identical in both lanes of a pair.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-bit element traits: MFMA and round-to-nearest-even packing of two fp32.
template <int DT> struct Elem16;
template <> struct Elem16<ATTN_IMPL_BF16> {
    typedef bf16x8 vec8;
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    // the two elements of a packed dword, exactly, as fp32
    static __device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
};
template <> struct Elem16<ATTN_IMPL_FP16> {
    typedef f16x8 vec8;
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ float lo(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
    static __device__ __forceinline__ float hi(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
};

// ---------------------------------------------------------------------------
// rotary position embedding of one feature pair
// ---------------------------------------------------------------------------

// The bits of a dword as fp32.  The argument is taken by value on purpose: hipcc
// compiles __builtin_bit_cast applied directly to an element of a vector value
// (v[i]) into a read of element 0 (an element of a vector is not addressable), so
// elements are always copied into a scalar first.
__device__ __forceinline__ float u2f(uint32_t w) { return __builtin_bit_cast(float, w); }

// fp64 -> fp32 with rounding to odd: truncate toward zero, then set the last
// fraction bit when the truncation was inexact.  A following round-to-nearest-even
// into a format with at least two fewer fraction bits (bf16, fp16) then equals one
// direct rounding of the fp64 value (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", IEEE
// Transactions on Computers 57(4), 2008).
__device__ __forceinline__ float round_odd_f32(double d) {
    float f = (float)d;                         // nearest even
    const double back = (double)f;
    if (back != d) {
        uint32_t u = __builtin_bit_cast(uint32_t, f);
        if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;   // one step toward zero
        u |= 1u;
        f = __builtin_bit_cast(float, u);
    }
    return f;
}

// Turn the pair (a, b) through the angle with cosine c and sine s:
// (a c - b s, a s + b c).  In fp64 both products of a 16-bit value and an fp32
// table entry are exact, so each result rounds once (in the difference or sum);
// the results come back rounded to odd, ready for one nearest-even rounding into
// the 16-bit storage type.
__device__ __forceinline__ void rope_rotate(float a, float b, float c, float s, float& ra, float& rb) {
    const double da = a, db = b, dc = c, ds = s;
    ra = round_odd_f32(da * dc - db * ds);
    rb = round_odd_f32(da * ds + db * dc);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // raw buffer: stride 0, num_records = bytes (loads past it return zero)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// voffset that always lies past num_records (per-head slices are < 2^31 bytes and
// the tile offset added through soffset is < 2^31): the DMA lane writes zeros
// into a padding slot without touching memory.
constexpr uint32_t OOB_VOFFSET = 0x7fff0000u;

// cache-policy operand of the buffer intrinsics: the non-temporal hint (nt), for
// data read exactly once
constexpr int CPOL_NT = 2;

}  // namespace attn_impl

#endif
