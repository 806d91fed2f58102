// attn_fwd_api.cpp -- the C-ABI entry points declared in include/attn_fwd.h:
// argument validation on the host, kernel selection and one launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_fwd.h"
#include "attn_fwd_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// n1 * n2 * ... fits comfortably in a signed 64-bit element offset
bool product_fits(int64_t a, int64_t b, int64_t c, int64_t d) {
    const int64_t lim = INT64_C(1) << 60;
    int64_t x = a;
    if (x > lim / b) return false;
    x *= b;
    if (x > lim / c) return false;
    x *= c;
    if (x > lim / d) return false;
    return true;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Sq, int Sk, int D,
                        float scale, int causal, int dtype, hipStream_t stream) {
    using namespace attn_impl;
    if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || D < 1) return ATTN_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_BF16 && dtype != ATTN_FP16 && dtype != ATTN_FP32) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return ATTN_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
    if (!product_fits(B, Hq, Sq, D) || !product_fits(B, Hkv, Sk, D)) return ATTN_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    // one (batch, head) slice of Q, K or V is addressed with 32-bit byte offsets
    const int64_t esize = (dtype == ATTN_FP32) ? 4 : 2;
    const int64_t slice_lim = (INT64_C(1) << 31) - (INT64_C(1) << 20);
    if ((int64_t)Sq * D * esize > slice_lim || (int64_t)Sk * D * esize > slice_lim)
        return ATTN_ERR_UNSUPPORTED;

    const KernelChoice kc = select_kernel(dtype, D, causal ? 1 : 0);
    if (!kc.fn) return ATTN_ERR_UNSUPPORTED;

    AttnParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Sq = Sq;
    p.Sk = Sk;
    // fold log2(e) into the scale; its sign and a zero scale are moved onto Q
    const double c = fabs((double)scale) * 1.4426950408889634;
    p.c = (scale == 0.0f) ? 1.0f : (float)c;
    p.q_mode = (scale == 0.0f) ? 2 : (scale < 0.0f ? 1 : 0);
    if (!(p.c > 0.0f) || !isfinite(p.c)) return ATTN_ERR_INVALID_ARG;
    p.nq = (Sq + kc.bm - 1) / kc.bm;

    const int64_t groups = (int64_t)B * Hkv;
    const int64_t per_group = (int64_t)(Hq / Hkv) * p.nq;
    const int64_t nwg = groups * per_group;
    if (nwg > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
    // Bundle enough key/value-head groups to fill the workgroup slots of one XCD
    // (32 CUs x 2 workgroups), heaviest query tiles of the whole bundle first; the
    // bundle count must divide the groups (and split over the 8 XCDs to remap).
    int gb = 1;
    while (gb * per_group < 64 && groups % (2 * gb) == 0) gb *= 2;
    p.gbundle = gb;
    p.xcd_remap = ((groups / gb) % 8 == 0) ? 1 : 0;

    void* args[] = {&p};
    const hipError_t err = hipLaunchKernel(kc.fn, dim3((unsigned)nwg), dim3(kc.threads), args, 0,
                                           stream);
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" const char* attn_status_str(int status) {
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}
