// attn_fwd_api.cpp -- the C-ABI entry points declared in include/attn_fwd.h:
// argument validation on the host, kernel selection and one launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_fwd.h"
#include "attn_fwd_internal.h"
#include "attn_fwd_tile_map.h"

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

// Checks shared by both entry points (everything but the kernel choice).
int check_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale, int dtype) {
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
    return ATTN_OK;
}

// log2(e) folded into the scale; its sign and a zero scale move onto Q
void fold_scale(float scale, float* c, int* q_mode) {
    const double cc = fabs((double)scale) * 1.4426950408889634;
    *c = (scale == 0.0f) ? 1.0f : (float)cc;
    *q_mode = (scale == 0.0f) ? 2 : (scale < 0.0f ? 1 : 0);
}

// Chunking of the keys for the split-KV pass.  nsplit_req <= 0 chooses: enough
// chunks that about 1024 waves (four per CU) stream K/V at once, but no chunk
// shorter than 256 keys.  Chunks are whole 32-key tiles; the count actually used
// is ceil(Sk / chunk), which never exceeds the request.
struct DecodePlan { int nsplit, chunk; };
DecodePlan decode_plan(int B, int Hkv, int Sk, int nsplit_req) {
    const int64_t groups = (int64_t)B * Hkv;
    int64_t ns = nsplit_req;
    if (ns <= 0) {
        ns = (1024 + groups - 1) / groups;
        const int64_t cap = (Sk + 255) / 256;
        if (ns > cap) ns = cap;
    }
    if (ns < 1) ns = 1;
    if (ns > Sk) ns = Sk;
    int64_t chunk = (Sk + ns - 1) / ns;
    chunk = (chunk + 31) / 32 * 32;
    DecodePlan pl;
    pl.chunk = (int)chunk;
    pl.nsplit = (int)((Sk + chunk - 1) / chunk);
    return pl;
}

size_t decode_workspace(int64_t rows, int D, int nsplit) {
    return (size_t)nsplit * (size_t)rows * ((size_t)D + 1) * sizeof(float);
}

// Multiplier and shift of the division by d (1 <= d < 2^31) for dividends below 2^31.

// Everything one prefill launch needs, decided on the host before anything is enqueued.
struct FwdLaunch {
    const void* fn;
    unsigned nwg;
    int threads;
    attn_impl::AttnParams p;
};

// Kernel choice, scale folding and launch mapping of the prefill kernel (arguments
// already validated).  rope: 0, or the rotary layout with its tables (then k is the
// rotated copy).  Enqueues nothing, so every error is returned before any launch.
int prepare_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale, int causal,
                int dtype, int rope, const float* rcos, const float* rsin, FwdLaunch* out) {
    using namespace attn_impl;
    const KernelChoice kc = select_kernel(dtype, D, causal ? 1 : 0, rope, (int64_t)B * Hq, Sq);
    if (!kc.fn) return ATTN_ERR_UNSUPPORTED;

    AttnParams& p = out->p;
    p.rcos = rcos;
    p.rsin = rsin;
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
    fold_scale(scale, &p.c, &p.q_mode);
    if (!(p.c > 0.0f) || !isfinite(p.c)) return ATTN_ERR_INVALID_ARG;
    p.nq = (Sq + kc.bm - 1) / kc.bm;

    const int64_t groups = (int64_t)B * Hkv;
    const int64_t per_group = (int64_t)(Hq / Hkv) * p.nq;
    const int64_t nwg = groups * per_group;
    if (nwg > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
    plan_tile_map(p, groups, per_group, Hq / Hkv);
    out->fn = kc.fn;
    out->nwg = (unsigned)nwg;
    out->threads = kc.threads;
    return ATTN_OK;
}

int enqueue_fwd(FwdLaunch& L, hipStream_t stream) {
    void* args[] = {&L.p};
    const hipError_t err = hipLaunchKernel(L.fn, dim3(L.nwg), dim3(L.threads), args, 0, stream);
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Sq, int Sk, int D,
                        float scale, int causal, int dtype, hipStream_t stream) {
    int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, dtype);
    if (st != ATTN_OK) return st;
    FwdLaunch L;
    st = prepare_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, dtype, 0, nullptr,
                     nullptr, &L);
    if (st != ATTN_OK) return st;
    return enqueue_fwd(L, stream);
}

extern "C" int attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                             void* k_rot, const float* rope_cos, const float* rope_sin,
                             int rope_layout, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                             float scale, int causal, int dtype, hipStream_t stream) {
    using namespace attn_impl;
    const int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, dtype);
    if (st != ATTN_OK) return st;
    if (!k_rot || !rope_cos || !rope_sin) return ATTN_ERR_INVALID_ARG;
    if (!aligned(k_rot, 16) || !aligned(rope_cos, 16) || !aligned(rope_sin, 16))
        return ATTN_ERR_INVALID_ARG;
    if (rope_layout != ATTN_ROPE_INTERLEAVED && rope_layout != ATTN_ROPE_HALVES)
        return ATTN_ERR_INVALID_ARG;
    if (Sq > Sk) return ATTN_ERR_INVALID_ARG;
    if (dtype == ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
    // the attention kernel addresses the tables with 32-bit byte offsets
    if ((int64_t)Sk * (D / 2) * 4 > (INT64_C(1) << 31) - (INT64_C(1) << 20)) return ATTN_ERR_UNSUPPORTED;

    // heads per thread of the key pass: the largest of 4, 2, 1 dividing Hkv
    const int hb = (Hkv % 4 == 0) ? 4 : (Hkv % 2 == 0) ? 2 : 1;
    const void* rk = select_rope(dtype, D, rope_layout, hb);
    if (!rk) return ATTN_ERR_UNSUPPORTED;
    // the attention launch is fully decided (scale, kernel, grid) before the key
    // pass is enqueued, so an error leaves k_rot and every output untouched
    FwdLaunch L;
    const int sp = prepare_fwd(q, k_rot, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, dtype,
                               rope_layout, rope_cos, rope_sin, &L);
    if (sp != ATTN_OK) return sp;
    RopeParams rp;
    rp.x = k;
    rp.y = k_rot;
    rp.rcos = rope_cos;
    rp.rsin = rope_sin;
    rp.rows = (int64_t)B * Hkv * Sk;
    rp.S = Sk;
    const int64_t threads = rp.rows / hb * (D / 16);
    const int64_t nblk = (threads + 255) / 256;
    if (nblk > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
    void* a1[] = {&rp};
    if (hipLaunchKernel(rk, dim3((unsigned)nblk), dim3(256), a1, 0, stream) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    return enqueue_fwd(L, stream);
}

extern "C" int attn_fwd_decode_workspace(int B, int Hq, int Hkv, int Sq, int Sk, int D, int nsplit,
                                         size_t* bytes) {
    using namespace attn_impl;
    if (!bytes) return ATTN_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || D < 1 || Hq % Hkv != 0)
        return ATTN_ERR_INVALID_ARG;
    if (!product_fits(B, Hq, Sq, D) || !product_fits(B, Hkv, Sk, D)) return ATTN_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if ((int64_t)(Hq / Hkv) * Sq > 32) return ATTN_ERR_UNSUPPORTED;
    const DecodePlan pl = decode_plan(B, Hkv, Sk, nsplit);
    *bytes = decode_workspace((int64_t)B * Hq * Sq, D, pl.nsplit);
    return ATTN_OK;
}

namespace {

// The split-KV pass and the merge.  The partial results go to `workspace` (at
// least `workspace_bytes` bytes), or with `scratch_call` to the library's static
// device scratch (the workspace arguments are then ignored, and a call whose
// partial results would not fit it is refused).
int decode_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale, int causal, int dtype,
                int nsplit, void* workspace, size_t workspace_bytes, bool scratch_call,
                hipStream_t stream) {
    using namespace attn_impl;
    const int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, dtype);
    if (st != ATTN_OK) return st;
    if (dtype == ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
    if ((int64_t)(Hq / Hkv) * Sq > 32) return ATTN_ERR_UNSUPPORTED;
    DecodeParams dp;
    fold_scale(scale, &dp.c, &dp.q_mode);
    if (!(dp.c > 0.0f) || !isfinite(dp.c)) return ATTN_ERR_INVALID_ARG;
    const DecodePlan pl = decode_plan(B, Hkv, Sk, nsplit);
    const int64_t rows = (int64_t)B * Hq * Sq;
    const size_t need = decode_workspace(rows, D, pl.nsplit);
    const int64_t nwg = (int64_t)B * Hkv * pl.nsplit;
    if (nwg > INT32_MAX || rows > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
    const void* fs = select_decode_split(dtype, D, causal ? 1 : 0);
    const void* fm = select_decode_merge(dtype, D);
    if (!fs || !fm) return ATTN_ERR_UNSUPPORTED;
    // every check above is made before the scratch lookup (the first runtime call)
    if (scratch_call) {
        if (need > DECODE_SCRATCH_BYTES) return ATTN_ERR_UNSUPPORTED;
        if (decode_scratch(&workspace, &workspace_bytes) != 0) return ATTN_ERR_LAUNCH;
    }
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return ATTN_ERR_INVALID_ARG;

    dp.q = q;
    dp.k = k;
    dp.v = v;
    dp.opart = (float*)workspace;
    dp.lpart = dp.opart + (size_t)pl.nsplit * (size_t)rows * (size_t)D;
    dp.B = B;
    dp.Hq = Hq;
    dp.Hkv = Hkv;
    dp.Sq = Sq;
    dp.Sk = Sk;
    dp.chunk = pl.chunk;
    dp.nsplit = pl.nsplit;
    void* a1[] = {&dp};
    if (hipLaunchKernel(fs, dim3((unsigned)nwg), dim3(64), a1, 0, stream) != hipSuccess)
        return ATTN_ERR_LAUNCH;

    MergeParams mp;
    mp.opart = dp.opart;
    mp.lpart = dp.lpart;
    mp.o = o;
    mp.lse = lse;
    mp.rows = rows;
    mp.nsplit = pl.nsplit;
    void* a2[] = {&mp};
    if (hipLaunchKernel(fm, dim3((unsigned)rows), dim3(D), a2, 0, stream) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int Sq, int Sk, int D,
                               float scale, int causal, int dtype, int nsplit,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, dtype, nsplit,
                       workspace, workspace_bytes, false, stream);
}

extern "C" int attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                       float scale, int causal, int dtype, int nsplit,
                                       hipStream_t stream) {
    return decode_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, dtype, nsplit,
                       nullptr, 0, true, stream);
}

namespace {

// Workgroups that share the query heads of one K/V head in the dK/dV pass: doubled
// (while it divides the Hq/Hkv query heads of a group) until the pass has at least
// 1024 workgroups, two rounds of the two that fit on each CU.  One for every shape
// whose K/V heads already fill it.
int bwd_splits(int B, int Hq, int Hkv, int Sk) {
    const int64_t base = (int64_t)B * Hkv * ((Sk + 127) / 128);
    const int R = Hq / Hkv;
    int ns = 1;
    while (base * ns < 1024 && R % (2 * ns) == 0) ns *= 2;
    return ns;
}

// Bytes of the workspace: three fp32 values per query row, then (several splits) the
// partial dK and dV of every split, starting on a 256-byte boundary.
bool bwd_layout(int B, int Hq, int Hkv, int Sq, int Sk, int D, size_t* bytes, size_t* part_off,
                int* nsplit) {
    const int ns = bwd_splits(B, Hq, Hkv, Sk);
    if (!product_fits(B, Hq, Sq, 12) || !product_fits((int64_t)B * Hkv, Sk, D, (int64_t)ns * 8)) return false;
    const size_t rows_bytes = (size_t)3 * (size_t)B * (size_t)Hq * (size_t)Sq * sizeof(float);
    const size_t off = (rows_bytes + 255) / 256 * 256;
    const size_t part = ns > 1 ? (size_t)ns * 2 * (size_t)B * Hkv * Sk * D * sizeof(float) : 0;
    *bytes = off + part;
    *part_off = off;
    *nsplit = ns;
    return true;
}

}  // namespace

extern "C" int attn_bwd_workspace(int B, int Hq, int Hkv, int Sq, int Sk, int D, size_t* bytes) {
    if (!bytes || B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || D < 1 || Hq % Hkv != 0)
        return ATTN_ERR_INVALID_ARG;
    size_t off;
    int ns;
    if (!bwd_layout(B, Hq, Hkv, Sq, Sk, D, bytes, &off, &ns)) return ATTN_ERR_INVALID_ARG;
    return ATTN_OK;
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv,
                        int B, int Hq, int Hkv, int Sq, int Sk, int D,
                        float scale, int causal, int dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    using namespace attn_impl;
    int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, dtype);
    if (st != ATTN_OK) return st;
    if (!lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return ATTN_ERR_INVALID_ARG;
    if (dtype == ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)B * Hq * Sq;
    size_t need = 0, part_off = 0;
    int nsplit = 1;
    if (!bwd_layout(B, Hq, Hkv, Sq, Sk, D, &need, &part_off, &nsplit)) return ATTN_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return ATTN_ERR_INVALID_ARG;
    const int64_t kvelems = (int64_t)B * Hkv * Sk * D;
    const int64_t n_pre = (rows + (256 / (D / 8)) - 1) / (256 / (D / 8));
    const int64_t n_kv = (int64_t)B * Hkv * ((Sk + 127) / 128) * nsplit;
    const int64_t n_q = (int64_t)B * Hq * ((Sq + 127) / 128);
    const int64_t n_red = (kvelems / 8 + 255) / 256;
    const int64_t q_start = (n_kv + 7) / 8 * 8;
    if (n_pre > INT32_MAX || q_start + n_q > INT32_MAX || n_red > INT32_MAX)
        return ATTN_ERR_UNSUPPORTED;
    const BwdKernels kf = select_bwd(dtype, D, causal ? 1 : 0);
    if (!kf.pre || !kf.main || !kf.reduce) return ATTN_ERR_UNSUPPORTED;

    BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.l2row = (float*)workspace;
    p.drow = p.l2row + rows;
    p.sinit = p.drow + rows;
    p.part = nsplit > 1 ? (float*)((uint8_t*)workspace + part_off) : nullptr;
    p.nsplit = nsplit;
    p.kvelems = kvelems;
    p.n_kv = (int)n_kv;
    p.q_start = (int)q_start;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Sq = Sq;
    p.Sk = Sk;
    p.c = (float)((double)scale * 1.4426950408889634);
    // The dK/dV pass starts its score accumulators at -LSE2/ce and multiplies by ce:
    // below 2^-100 in magnitude the scores' contribution c.s is far under one ulp of
    // LSE2, so ce = 2^-100 (which keeps -LSE2/ce finite) gives the same fp32 weights
    // exp2(-LSE2); a zero or tiny scale thus never overflows the start value.
    p.ce = fabsf(p.c) >= 0x1p-100f ? p.c : 0x1p-100f;
    if (!isfinite(p.c)) return ATTN_ERR_INVALID_ARG;   // |scale| * log2(e) past the fp32 range
    p.scale = scale;
    p.rows = rows;
    void* args[] = {&p};
    if (hipLaunchKernel(kf.pre, dim3((unsigned)n_pre), dim3(256), args, 0, stream) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    if (hipLaunchKernel(kf.main, dim3((unsigned)(q_start + n_q)), dim3(256), args, 0, stream) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    if (nsplit > 1 &&
        hipLaunchKernel(kf.reduce, dim3((unsigned)n_red), dim3(256), args, 0, stream) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    return ATTN_OK;
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
