// attn_fwd_internal.h -- what the C-ABI entry point and the kernels share:
// the kernel parameter block and the kernel-selection hook.  Not installed.
#ifndef ATTN_FWD_INTERNAL_H
#define ATTN_FWD_INTERNAL_H

#include <stdint.h>

#define ATTN_IMPL_BF16 0
#define ATTN_IMPL_FP16 1
#define ATTN_IMPL_FP32 2

namespace attn_impl {

// Everything a kernel needs, passed by value as its only argument.
struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;       // may be null
    int B, Hq, Hkv, Sq, Sk;
    float c;          // |scale| * log2(e), strictly positive
    int q_mode;       // 0: use Q as is; 1: use -Q (negative scale); 2: use 0 (zero scale)
    int nq;           // query tiles per head
    int xcd_remap;    // 1: give each XCD whole bundles of key/value-head groups
    int gbundle;      // key/value-head groups per bundle (divides B * Hkv)
};

struct KernelChoice {
    const void* fn;   // __global__ function, or null when the combination is unsupported
    int bm;           // queries per workgroup
    int threads;      // threads per workgroup
};

KernelChoice select_kernel(int dtype, int D, int causal);

}  // namespace attn_impl

#endif
