// attn_fwd_internal.h -- what the C-ABI entry point and the kernels share:
// the kernel parameter block and the kernel-selection hook.  Not installed.
#ifndef ATTN_FWD_INTERNAL_H
#define ATTN_FWD_INTERNAL_H

#include <stddef.h>
#include <stdint.h>

#define ATTN_IMPL_BF16 0
#define ATTN_IMPL_FP16 1
#define ATTN_IMPL_FP32 2

namespace attn_impl {

// Everything a kernel needs, passed by value as its only argument.
// Division by a launch constant d >= 1 of a non-negative n < 2^31 as a multiply and a
// shift: n / d = (n * m) >> s with s = 31 + ceil(log2 d), m = ceil(2^s / d) < 2^32
// (the round-up method of Granlund and Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994: m*d - 2^s < d <= 2^ceil(log2 d), so the product
// overshoots n/d by less than 1/d and the floor is exact).
struct FastDiv { uint32_t m, s; };

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
    int gbundle;      // key/value-head groups per bundle (divides B * Hkv), a power of two
    int R;            // query heads per key/value head, Hq / Hkv
    FastDiv div_bu;   // by the workgroups per bundle, gbundle * R * nq
    FastDiv div_gr;   // by gbundle * R
    FastDiv div_r;    // by R
    FastDiv div_hkv;  // by Hkv
    const float* rcos;  // rotary embedding tables [Sk][D/2] (kernels built with it only)
    const float* rsin;
};

// Rotary embedding of K into the rotated copy the attention then reads.
struct RopeParams {
    const void* x;      // [rows][D] 16-bit
    void* y;            // [rows][D] 16-bit
    const float* rcos;  // [S][D/2]
    const float* rsin;
    int64_t rows;       // B * H * S
    int S;              // row r sits at position r % S
};
const void* select_rope(int dtype, int D, int layout, int hb);

struct KernelChoice {
    const void* fn;   // __global__ function, or null when the combination is unsupported
    int bm;           // queries per workgroup
    int threads;      // threads per workgroup
};

// rope: 0 none, 1 interleaved pairs (2i, 2i+1), 2 split halves (i, i + D/2); the
// rotary variants exist for the 16-bit types only
// heads = B * Hq; with Sq it decides the fp32 variant (keys split between the waves of
// a 32-query workgroup when 128-query workgroups would be fewer than the CUs)
KernelChoice select_kernel(int dtype, int D, int causal, int rope, int64_t heads, int Sq);
// the fp32 part of select_kernel (attn_fwd32_kernels.hip)
KernelChoice select_kernel32(int D, int causal, int64_t heads, int Sq);

// Split-KV pass for few query rows: one wave per (batch, K/V head, chunk).
struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    float* opart;     // [nsplit][B*Hq*Sq][D]: each chunk's O, normalised over the chunk
    float* lpart;     // [nsplit][B*Hq*Sq]: each chunk's natural-log LSE (-inf: no visible key)
    int B, Hq, Hkv, Sq, Sk;
    float c;          // |scale| * log2(e), strictly positive
    int q_mode;       // as in AttnParams
    int chunk;        // keys per chunk, a multiple of 32
    int nsplit;       // chunks per (batch, K/V head); workgroup w = (b*Hkv + g) * nsplit + chunk
};

// Merge of the chunks' partial results into O and LSE.
struct MergeParams {
    const float* opart;
    const float* lpart;
    void* o;          // [B*Hq*Sq][D], 16-bit element type
    float* lse;       // may be null
    int64_t rows;     // B*Hq*Sq
    int nsplit;
};

// Gradients: workspace rows of D_i = dO_i.O_i and LSE_i log2(e), then dK/dV and dQ.
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;   // the forward's natural-log LSE, [B*Hq*Sq]
    void* dq;
    void* dk;
    void* dv;
    float* l2row;       // workspace: LSE * log2(e) per query row
    float* drow;        // workspace: -(dO . O) per query row
    float* sinit;       // workspace: -LSE * log2(e) / ce per query row
    float* part;        // workspace (nsplit > 1): fp32 partial dK, dV per split,
                        // [nsplit][2][B*Hkv*Sk*D], dK unscaled
    int B, Hq, Hkv, Sq, Sk;
    int nsplit;         // workgroups sharing the query heads of one K/V head (divides Hq/Hkv)
    float c;            // scale * log2(e) (any sign)
    float ce;           // c, or 2^-100 when c is zero (the weights are then exp2(-LSE2))
    float scale;
    int64_t rows;       // B*Hq*Sq
    int64_t kvelems;    // B*Hkv*Sk*D
    int n_kv;           // dK/dV workgroups of the combined launch
    int q_start;        // first dQ workgroup (n_kv rounded up to a multiple of 8)
};
struct BwdKernels { const void* pre; const void* main; const void* reduce; };
BwdKernels select_bwd(int dtype, int D, int causal);   // null members: unsupported

const void* select_decode_split(int dtype, int D, int causal);   // null: unsupported
const void* select_decode_merge(int dtype, int D);

// Bytes of the static device scratch that the allocation-free decode entry point
// uses for the chunks' partial results (16 MiB).
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)16 << 20;
// Device address and size of the current device's scratch (looked up once per
// device and cached); 0 on success, nonzero when the runtime cannot provide it.
int decode_scratch(void** ptr, size_t* bytes);

}  // namespace attn_impl

#endif
