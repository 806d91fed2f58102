// attn_kernel_common.h -- device-side helpers shared by the attention kernels
// (prefill and decode): vector types, wave-pair reductions, 16-bit element
// traits and buffer resources.  Included by the .hip sources only.
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
};

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

}  // namespace attn_impl

#endif
