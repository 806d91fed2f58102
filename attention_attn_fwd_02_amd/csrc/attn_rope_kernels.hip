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

// One thread per 8 pairs (16 features) of HB rows at one position (the same
// position of HB consecutive heads, so each table entry is loaded once for HB rows);
// 256 threads per workgroup.  LAYOUT 1: pairs (2i, 2i+1), the thread owns features
// 16t .. 16t+15 (pairs 8t .. 8t+7).  LAYOUT 2: pairs (i, i + D/2), the thread owns
// features 8t .. 8t+7 and their partners D/2 + 8t .. (pairs 8t .. 8t+7).
template <int DT, int D, int LAYOUT, int HB>
__global__ __launch_bounds__(256) void attn_rope_k(RopeParams p) {
    typedef Elem16<DT> E;
    constexpr int TPR = D / 16;          // threads per row
    constexpr int HALF = D / 2;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r = gid / TPR;         // (head group, position)
    const int t = (int)(gid % TPR);
    if (r >= p.rows / HB) return;
    const int pos = (int)(r % p.S);
    const int64_t row0 = (r / p.S) * HB * p.S + pos;
    const float4* ctab = (const float4*)(p.rcos + (int64_t)pos * HALF + 8 * t);
    const float4* stab = (const float4*)(p.rsin + (int64_t)pos * HALF + 8 * t);
    const float4 c0 = ctab[0], c1 = ctab[1], s0 = stab[0], s1 = stab[1];
    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    // a: the first element of each pair, b: the second, both as dwords of two
    const int off_a = (LAYOUT == 1) ? 32 * t : 16 * t;
    const int off_b = (LAYOUT == 1) ? 32 * t + 16 : D + 16 * t;
    u32x4 wa[HB], wb[HB];
#pragma unroll
    for (int i = 0; i < HB; ++i) {
        const uint8_t* src = (const uint8_t*)p.x + (row0 + (int64_t)i * p.S) * (2 * D);
        wa[i] = *(const u32x4*)(src + off_a);
        wb[i] = *(const u32x4*)(src + off_b);
    }
#pragma unroll
    for (int i = 0; i < HB; ++i) {
        u32x4 ya, yb;
        if constexpr (LAYOUT == 1) {
            // dword e of the 32 bytes holds pair 8t + e as (lo, hi)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float r0, r1, r2, r3;
                rope_rotate(E::lo(wa[i][e]), E::hi(wa[i][e]), cs[e], sn[e], r0, r1);
                rope_rotate(E::lo(wb[i][e]), E::hi(wb[i][e]), cs[4 + e], sn[4 + e], r2, r3);
                ya[e] = E::pack(r0, r1);
                yb[e] = E::pack(r2, r3);
            }
        } else {
            // element j of wa pairs with element j of wb, as pair 8t + j
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a0, b0, a1, b1;
                rope_rotate(E::lo(wa[i][e]), E::lo(wb[i][e]), cs[2 * e], sn[2 * e], a0, b0);
                rope_rotate(E::hi(wa[i][e]), E::hi(wb[i][e]), cs[2 * e + 1], sn[2 * e + 1], a1, b1);
                ya[e] = E::pack(a0, a1);
                yb[e] = E::pack(b0, b1);
            }
        }
        uint8_t* dst = (uint8_t*)p.y + (row0 + (int64_t)i * p.S) * (2 * D);
        *(u32x4*)(dst + off_a) = ya;
        *(u32x4*)(dst + off_b) = yb;
    }
}

template <int DT, int D, int LAYOUT>
static const void* pick_rope_hb(int hb) {
    return hb == 4 ? (const void*)&attn_rope_k<DT, D, LAYOUT, 4>
         : hb == 2 ? (const void*)&attn_rope_k<DT, D, LAYOUT, 2>
         : hb == 1 ? (const void*)&attn_rope_k<DT, D, LAYOUT, 1> : nullptr;
}
template <int DT, int D>
static const void* pick_rope(int layout, int hb) {
    return layout == 1 ? pick_rope_hb<DT, D, 1>(hb) : layout == 2 ? pick_rope_hb<DT, D, 2>(hb) : nullptr;
}

const void* select_rope(int dtype, int D, int layout, int hb) {
    if (dtype == ATTN_IMPL_BF16)
        return D == 64 ? pick_rope<ATTN_IMPL_BF16, 64>(layout, hb)
             : D == 128 ? pick_rope<ATTN_IMPL_BF16, 128>(layout, hb) : nullptr;
    if (dtype == ATTN_IMPL_FP16)
        return D == 64 ? pick_rope<ATTN_IMPL_FP16, 64>(layout, hb)
             : D == 128 ? pick_rope<ATTN_IMPL_FP16, 128>(layout, hb) : nullptr;
    return nullptr;
}

}  // namespace attn_impl
