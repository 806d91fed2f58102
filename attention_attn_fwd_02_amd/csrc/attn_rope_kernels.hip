// attn_rope_kernels.hip -- rotary position embedding of the keys, the pass that
// runs ahead of attention when Q and K carry positions.
//
// The FIBER page ("A Thread-Register Decoupled GPU Execution Model for Efficient
// Tensor Computation") lists RoPE among the vector operations that sit between
// the GEMMs of a transformer block (background; evaluation set-up, "Workloads"),
// and the VDCores page evaluates the QKV projection fused with RoPE (evaluation,
// dynamic fusion, Fig. 12).  The rotation is the rotary embedding of the RoPE paper
// the FIBER page cites: feature pair i of the row at position p turns through the
// angle whose cosine and sine the caller tabulates at [p][i].
//
// Queries are rotated inside the attention kernel as their fragments are loaded
// (each query element is loaded by exactly one workgroup, so that costs nothing
// extra).  Every key tile, in contrast, is read by all the query tiles of its head,
// so the keys are rotated once, here, into the caller's buffer (the contents a
// KV cache holds), and the attention kernel reads that copy.  The pass is bound by
// HBM: one read of K and one write of the rotated copy, 16-byte accesses, rows
// contiguous across consecutive threads; the tables (a few MiB) stay in L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_internal.h"
#include "attn_kernel_common.h"

namespace attn_impl {

// One thread per 8 pairs (16 features) of a row; 256 threads per workgroup.
// LAYOUT 1: pairs (2i, 2i+1), the thread owns features 16t .. 16t+15 (pairs 8t ..
// 8t+7).  LAYOUT 2: pairs (i, i + D/2), the thread owns features 8t .. 8t+7 and
// their partners D/2 + 8t .. (pairs 8t .. 8t+7).
template <int DT, int D, int LAYOUT>
__global__ __launch_bounds__(256) void attn_rope_k(RopeParams p) {
    typedef Elem16<DT> E;
    constexpr int TPR = D / 16;          // threads per row
    constexpr int HALF = D / 2;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / TPR;
    const int t = (int)(gid % TPR);
    if (row >= p.rows) return;
    const int pos = (int)(row % p.S);
    const uint8_t* src = (const uint8_t*)p.x + row * (2 * D);
    uint8_t* dst = (uint8_t*)p.y + row * (2 * D);
    const float4* ctab = (const float4*)(p.rcos + (int64_t)pos * HALF + 8 * t);
    const float4* stab = (const float4*)(p.rsin + (int64_t)pos * HALF + 8 * t);
    const float4 c0 = ctab[0], c1 = ctab[1], s0 = stab[0], s1 = stab[1];
    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    // a: the first element of each pair, b: the second, both as dwords of two
    const int off_a = (LAYOUT == 1) ? 32 * t : 16 * t;
    const int off_b = (LAYOUT == 1) ? 32 * t + 16 : D + 16 * t;
    const u32x4 wa = *(const u32x4*)(src + off_a);
    const u32x4 wb = *(const u32x4*)(src + off_b);
    u32x4 ya, yb;
    if constexpr (LAYOUT == 1) {
        // dword e of the 32 bytes holds pair 8t + e as (lo, hi)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float r0, r1, r2, r3;
            rope_rotate(E::lo(wa[e]), E::hi(wa[e]), cs[e], sn[e], r0, r1);
            rope_rotate(E::lo(wb[e]), E::hi(wb[e]), cs[4 + e], sn[4 + e], r2, r3);
            ya[e] = E::pack(r0, r1);
            yb[e] = E::pack(r2, r3);
        }
    } else {
        // element j of wa pairs with element j of wb, as pair 8t + j
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a0, b0, a1, b1;
            rope_rotate(E::lo(wa[e]), E::lo(wb[e]), cs[2 * e], sn[2 * e], a0, b0);
            rope_rotate(E::hi(wa[e]), E::hi(wb[e]), cs[2 * e + 1], sn[2 * e + 1], a1, b1);
            ya[e] = E::pack(a0, a1);
            yb[e] = E::pack(b0, b1);
        }
    }
    *(u32x4*)(dst + off_a) = ya;
    *(u32x4*)(dst + off_b) = yb;
}

template <int DT, int D>
static const void* pick_rope(int layout) {
    return layout == 1 ? (const void*)&attn_rope_k<DT, D, 1>
         : layout == 2 ? (const void*)&attn_rope_k<DT, D, 2> : nullptr;
}

const void* select_rope(int dtype, int D, int layout) {
    if (dtype == ATTN_IMPL_BF16)
        return D == 64 ? pick_rope<ATTN_IMPL_BF16, 64>(layout)
             : D == 128 ? pick_rope<ATTN_IMPL_BF16, 128>(layout) : nullptr;
    if (dtype == ATTN_IMPL_FP16)
        return D == 64 ? pick_rope<ATTN_IMPL_FP16, 64>(layout)
             : D == 128 ? pick_rope<ATTN_IMPL_FP16, 128>(layout) : nullptr;
    return nullptr;
}

}  // namespace attn_impl
