/*
 * attn_fwd.h -- C ABI of the fused attention forward for AMD Instinct MI355X (gfx950).
 *
 * The operation.  The page "A Thread-Register Decoupled GPU Execution Model for
 * Efficient Tensor Computation" (introduction) names multi-head attention,
 * Equ. 1, as the core of the transformer block and the FlashAttention series as
 * its fused, tiled implementation; its evaluation ("Workloads", Tbl. III) runs
 * the prefill attention of Llama-family models with L_context = 4096 and
 * d_head = 128, and the grouped-query (GQA) and multi-query (MQA) variants.  The
 * formula of Equ. 1 is not in the extracted text; it is read as scaled
 * dot-product attention per head:
 *
 *     O[b,h,i,:] = sum_j softmax_j( scale * Q[b,h,i,:] . K[b,g(h),j,:] ) * V[b,g(h),j,:]
 *     LSE[b,h,i] = ln sum_j exp( scale * Q[b,h,i,:] . K[b,g(h),j,:] )
 *
 * over the visible keys j, where g(h) = h / (Hq / Hkv) (consecutive groups of
 * query heads share one key/value head; Hkv = Hq is plain multi-head attention,
 * Hkv = 1 is multi-query attention) and, with causal != 0, key j is visible from
 * query i iff j <= i + (Sk - Sq) (the mask is aligned to the bottom-right corner,
 * so the last query sees every key).  A query that sees no key gets O = 0 and
 * LSE = -inf.
 *
 * Numerics: scores, the running softmax statistics and O accumulate in fp32;
 * for 16-bit inputs the softmax weights are rounded to the input type (round to
 * nearest even) before they multiply V, and O is rounded once to the input type.
 * fp32 inputs use fp32 products throughout.  Non-finite inputs propagate; they
 * are not checked.
 *
 * Execution: every entry point validates its arguments on the host, then only
 * enqueues kernel launches on the given stream: it allocates no memory, issues
 * no memset or copy and does not synchronise.  Calls may therefore be captured
 * into a HIP graph (stream capture) and replayed; a replay reads the buffers'
 * contents at replay time.  Every kernel reduces in a fixed order without
 * atomics, so equal inputs give bit-identical outputs from run to run.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
typedef enum {
    ATTN_BF16 = 0,   /* bfloat16 */
    ATTN_FP16 = 1,   /* IEEE binary16 */
    ATTN_FP32 = 2    /* IEEE binary32 */
} attn_dtype_t;

/* Return codes.  Every code is returned synchronously; the library never
 * aborts, prints or exits. */
typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,   /* a null or misaligned pointer, a size < 1, Hq % Hkv != 0,
                                   a non-finite scale or one whose magnitude times log2(e)
                                   leaves the fp32 range (|scale| above about 2.36e38),
                                   an unknown dtype, or sizes whose element counts
                                   overflow 64-bit offsets */
    ATTN_ERR_UNSUPPORTED = 2,   /* a head dimension D other than 64 or 128, a grid too
                                   large for one launch, or one (batch, head) slice of
                                   q, k or v of 2 GiB - 1 MiB or more */
    ATTN_ERR_LAUNCH = 3         /* the HIP runtime refused the kernel launch */
} attn_status_t;

/*
 * attn_fwd -- enqueue one fused attention forward on `stream`.
 *
 * Arguments (all pointers are device pointers, owned by the caller):
 *   q      [B][Hq][Sq][D]   input, element type `dtype`, 16-byte aligned
 *   k      [B][Hkv][Sk][D]  input, element type `dtype`, 16-byte aligned
 *   v      [B][Hkv][Sk][D]  input, element type `dtype`, 16-byte aligned
 *   o      [B][Hq][Sq][D]   output, element type `dtype`, 16-byte aligned; every
 *                           element is written
 *   lse    [B][Hq][Sq]      output, fp32, natural log, 4-byte aligned; may be NULL,
 *                           in which case no log-sum-exp is written
 *   B, Hq, Hkv, Sq, Sk      sizes, each >= 1; Hq must be a multiple of Hkv
 *   D                       head dimension: 64 or 128
 *   scale                   any finite value with |scale| * log2(e) inside the fp32
 *                           range (1/sqrt(D) is the usual choice)
 *   causal                  0: every key is visible; otherwise the bottom-right
 *                           causal mask described above
 *   dtype                   an attn_dtype_t
 *   stream                  HIP stream to enqueue on (NULL: the default stream)
 *
 * All tensors are contiguous with D fastest.  q/o and k/v may not overlap o or
 * lse.  The library allocates no memory and keeps no state between calls.  The
 * call validates its arguments on the host before touching the device, enqueues
 * one kernel and returns without synchronising: results are ready when `stream`
 * reaches that point.  On any error nothing is enqueued and no output is
 * written.  Results are deterministic: the same inputs give bitwise-identical
 * outputs on every call.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int D,
             float scale, int causal, int dtype, hipStream_t stream);

/*
 * Split-KV attention for few query rows (decoding).
 *
 * The page "A Thread-Register Decoupled GPU Execution Model for Efficient Tensor
 * Computation" evaluates decoding with FlashDecoding (evaluation set-up,
 * "Workloads"; L_context = 4096, d_head = 128) and describes it in its results
 * ("Decoding and Training Workloads Speedup") as matrix-vector work plus the
 * softmax, bound by memory, with a distinct KV cache per sequence.  The result is
 * the attention of attn_fwd above, computed in two passes: the keys of every
 * (batch, K/V head) are cut into nsplit chunks streamed concurrently, each chunk
 * giving an fp32 partial O normalised over its own keys and that chunk's
 * log-sum-exp; a second kernel merges them exactly,
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 * The query rows of one K/V head's group, (Hq / Hkv) * Sq of them, share every
 * K/V byte read, so they must number at most 32.
 *
 * attn_fwd_decode_workspace -- bytes of device workspace attn_fwd_decode needs
 * for these sizes and this nsplit; written to *bytes.  Returns ATTN_OK,
 * ATTN_ERR_INVALID_ARG (a size < 1, Hq % Hkv != 0, null `bytes`, overflowing
 * sizes) or ATTN_ERR_UNSUPPORTED (D not 64 or 128, (Hq / Hkv) * Sq > 32).
 */
int attn_fwd_decode_workspace(int B, int Hq, int Hkv, int Sq, int Sk, int D, int nsplit,
                              size_t* bytes);

/*
 * attn_fwd_decode -- enqueue the two kernels on `stream`.
 *
 * q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal: exactly as for attn_fwd
 * (same layouts, alignment, mask and empty-row convention), except that dtype
 * must be ATTN_BF16 or ATTN_FP16 (ATTN_FP32 gives ATTN_ERR_UNSUPPORTED) and
 * (Hq / Hkv) * Sq must be at most 32 (else ATTN_ERR_UNSUPPORTED).
 *   nsplit           chunks per (batch, K/V head); <= 0 lets the library choose
 *                    (about four waves per CU, chunks of at least 256 keys).
 *                    Chunks are whole 32-key tiles, so the count used is
 *                    ceil(Sk / chunk) and may be below the request.
 *   workspace        device memory owned by the caller, 16-byte aligned, at least
 *                    the size attn_fwd_decode_workspace reports for the same
 *                    arguments (else ATTN_ERR_INVALID_ARG); overwritten, and in use
 *                    until `stream` has run both kernels
 *   workspace_bytes  its size
 * The library allocates nothing.  Results are deterministic (fixed merge order);
 * they differ from attn_fwd's by rounding only.
 */
int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int Sq, int Sk, int D,
                    float scale, int causal, int dtype, int nsplit,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_fwd_decode_noalloc -- attn_fwd_decode for callers that cannot allocate
 * device memory or bring a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).
 *
 * Same arguments, kernels and results as attn_fwd_decode (bit for bit), without
 * the workspace: the chunks' partial results go to a static device array of
 * 16 MiB (ATTN_DECODE_SCRATCH_BYTES) inside the library, one per GPU, held until
 * the process ends.  Calls whose partial results would not fit (the size
 * attn_fwd_decode_workspace reports exceeds it) return ATTN_ERR_UNSUPPORTED.  The
 * first call on a device looks up that device's copy of the array (a runtime
 * query, no allocation; make it outside graph capture); ATTN_ERR_LAUNCH if the
 * runtime cannot provide it.  Nothing is allocated, no memset or copy is issued.
 * Every call on one GPU shares the array: calls that may overlap on one GPU
 * (different streams without ordering between them) race and give wrong results;
 * calls on one stream are ordered and safe.  Other errors are those of
 * attn_fwd_decode (minus the workspace checks).
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
int attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Sq, int Sk, int D,
                            float scale, int causal, int dtype, int nsplit, hipStream_t stream);

/*
 * Gradients of attn_fwd (the FlashAttention backward the FIBER page evaluates as
 * its training workload: evaluation set-up, "Workloads"; results, "Decoding and
 * Training Workloads Speedup").  For an output gradient dO and the weights
 * P_ij = exp(scale q_i.k_j - LSE_i) over visible pairs,
 *     dV = P^T dO,  dS = P o (dO V^T - rowsum(dO o O)),  dQ = scale dS K,
 *     dK = scale dS^T Q,
 * with the dK and dV of a key/value head summed over the query heads that read it.
 *
 * attn_bwd_workspace -- device workspace bytes attn_bwd needs for these sizes: three
 * fp32 values per query row and, for grouped-query shapes whose K/V heads alone
 * give the dK/dV pass fewer than 1024 workgroups, fp32 partial dK and dV for each of
 * the workgroups that share a K/V head's query heads (up to the Hq/Hkv of them);
 * ATTN_ERR_INVALID_ARG for a null `bytes`, a size < 1, Hq not a multiple of Hkv or
 * overflowing sizes.
 *
 * attn_bwd -- enqueue the kernels on `stream` (two, three with partial sums).
 *   q, k, v, B, Hq, Hkv, Sq, Sk, D, scale, causal, dtype: as given to attn_fwd
 *   o      [B][Hq][Sq][D]  attn_fwd's output for these inputs
 *   lse    [B][Hq][Sq]     attn_fwd's log-sum-exp (fp32, required here)
 *   dout   [B][Hq][Sq][D]  gradient of the loss with respect to o
 *   dq     [B][Hq][Sq][D]  output; dk, dv [B][Hkv][Sk][D] outputs; all fully written,
 *                          element type `dtype`, 16-byte aligned, not overlapping
 *                          any input
 *   workspace, workspace_bytes: caller-owned device memory of at least the size
 *                          attn_bwd_workspace reports, 16-byte aligned
 * dtype must be ATTN_BF16 or ATTN_FP16 (ATTN_FP32: ATTN_ERR_UNSUPPORTED).  Errors
 * are those of attn_fwd, plus ATTN_ERR_INVALID_ARG for a null lse, dout, dq, dk or
 * dv, a misaligned pointer, or a missing or short workspace.  Gradients accumulate
 * in fp32 and are rounded once; P and dS are rounded to `dtype` before they
 * multiply Q, K or dO.  Deterministic: no atomics, fixed summation order.  Keys
 * that no query sees get dK = dV = 0.
 */
int attn_bwd_workspace(int B, int Hq, int Hkv, int Sq, int Sk, int D, size_t* bytes);
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Sq, int Sk, int D,
             float scale, int causal, int dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Attention with the rotary position embedding applied to Q and K on the way in.
 *
 * The FIBER page lists RoPE among the vector operations between the GEMMs of a
 * transformer block (background; evaluation set-up, "Workloads") and the VDCores
 * page evaluates QKV projection fused with RoPE (evaluation, dynamic fusion,
 * Fig. 12).  The rotation is that of the RoPE paper the FIBER page cites: the D
 * features of a row form D/2 pairs, and pair i of a row at position p becomes
 *     (a, b) -> (a c - b s, a s + b c),   c = rope_cos[p][i],  s = rope_sin[p][i].
 * Key j sits at position j; query i at position i + (Sk - Sq) (the alignment of the
 * causal mask).  Each rotated element is computed in fp64 and rounded once (nearest
 * even) into `dtype`, so the result equals attn_fwd applied to Q and K first
 * rotated by a separate step that writes `dtype` tensors.
 *
 * attn_fwd_rope -- enqueue two kernels on `stream`: the keys are rotated into
 * k_rot (one HBM pass), then attn_fwd's kernel runs on k_rot with each query
 * fragment rotated in registers as it is loaded.
 *   q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal: as for attn_fwd
 *   k_rot       [B][Hkv][Sk][D] output, element type `dtype`, 16-byte aligned: the
 *               rotated keys (what a KV cache holds); must not overlap any input
 *   rope_cos, rope_sin  [Sk][D/2] fp32 device tables, 16-byte aligned (row p is
 *               position p; only rows 0 .. Sk-1 are read)
 *   rope_layout ATTN_ROPE_INTERLEAVED: pairs are features (2i, 2i+1);
 *               ATTN_ROPE_HALVES: pairs are features (i, i + D/2)
 * dtype must be ATTN_BF16 or ATTN_FP16 (ATTN_FP32: ATTN_ERR_UNSUPPORTED).  Errors
 * are those of attn_fwd, plus ATTN_ERR_INVALID_ARG for a null or misaligned k_rot
 * or table, an unknown layout, or Sq > Sk (queries would sit at negative
 * positions).  Every check, the attention launch's included, is made before the
 * key pass is enqueued: on any error nothing is enqueued and k_rot, o and lse are
 * untouched.  Deterministic; nothing is allocated.
 */
typedef enum {
    ATTN_ROPE_INTERLEAVED = 1,
    ATTN_ROPE_HALVES = 2
} attn_rope_layout_t;

int attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse, void* k_rot,
                  const float* rope_cos, const float* rope_sin, int rope_layout,
                  int B, int Hq, int Hkv, int Sq, int Sk, int D,
                  float scale, int causal, int dtype, hipStream_t stream);

/* Static, human-readable name of a return code ("unknown status" otherwise). */
const char* attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
