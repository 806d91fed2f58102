// attn_fwd_kernels.hip -- fused attention forward kernels for gfx950 (MI355X).
//
// The operation is the multi-head scaled dot-product attention of Equ. 1 on the
// page "A Thread-Register Decoupled GPU Execution Model for Efficient Tensor
// Computation" (introduction), computed the FlashAttention way that the same
// page names: one pass over key tiles with an online softmax, so the score
// matrix never leaves the chip.  The page's observation that attention is GEMM
// interleaved with SIMD/SFU softmax work, and its point that a score should feed
// the softmax straight from registers (programming-model section, Fig. 8), shape
// the register dataflow below; the decomposition over head and token blocks
// follows the VDCores page ("VDCores: Resource Decoupled Programming and
// Execution for Asynchronous GPUs", adaptive scheduling in its section 4.2).
//
// 16-bit path (bf16, fp16), per workgroup of 4 waves (one per SIMD):
//   * the workgroup owns BM = 256 consecutive queries of one (batch, head); each
//     wave owns 64 of them as two 32-query column blocks;
//   * the wave computes S^T = K_tile . Q^T with v_mfma_f32_32x32x16_{bf16,f16}:
//     K (keys x D) is the A operand read from LDS, Q^T the B operand held in
//     VGPRs for the whole kernel.  In the 32x32 accumulator layout every lane
//     holds one query column, so the row max and row sum of the online softmax
//     are in-lane reductions plus one v_permlane32_swap between the two
//     half-waves;
//   * the weights P^T are rounded to 16 bits in registers and feed the next MFMA
//     directly as its B operand: O^T (D x queries) += V^T . P^T.  The key order
//     inside each 16-key MFMA step is permuted so that P^T needs no data
//     movement; V is stored transposed (and permuted to match) in LDS;
//   * K and V tiles of 64 keys are double-buffered in LDS: the next tile's
//     global loads are issued before the current tile's MFMAs and written to the
//     other LDS buffer afterwards, one barrier per tile.
// fp32 path: the same dataflow with v_mfma_f32_32x32x2_f32 (true fp32 products),
// 32 queries per wave, 32-key tiles, single-buffered LDS.
//
// The mask, the grouped-head mapping and the empty-row convention are those of
// include/attn_fwd.h.
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
    // acc + lo + hi of a packed pair, in fp32 (one v_dot2c with (1, 1))
    static __device__ __forceinline__ float dot2_ones(uint32_t w, float acc) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
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
    static __device__ __forceinline__ float dot2_ones(uint32_t w, float acc) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
    }
};

// Workgroup -> (batch, query head, query tile).  Heavy causal tiles go first.
// When the key/value-head groups split evenly over the 8 XCDs (workgroup w is
// dispatched to XCD w % 8), every XCD gets whole groups, so all query heads and
// query tiles that read one K/V head share that XCD's L2.
struct TileCoord { int b, hq, qt; };
__device__ __forceinline__ TileCoord map_tile(const AttnParams& p, int w) {
    const int R = p.Hq / p.Hkv;      // query heads per key/value head
    const int U = R * p.nq;          // workgroups per key/value head
    int g, u;
    if (p.xcd_remap) {
        const int xcd = w & 7, slot = w >> 3;
        g = xcd + 8 * (slot / U);
        u = slot % U;
    } else {
        g = w / U;
        u = w % U;
    }
    TileCoord t;
    t.qt = p.nq - 1 - u / R;
    const int r = u % R;
    t.b = g / p.Hkv;
    t.hq = (g % p.Hkv) * R + r;
    return t;
}

// ---------------------------------------------------------------------------
// 16-bit kernel
// ---------------------------------------------------------------------------
constexpr int NW = 4;            // waves per workgroup
constexpr int QBLK = 2;          // 32-query column blocks per wave
constexpr int BM16 = NW * QBLK * 32;
constexpr int BN16 = 64;         // keys per tile

template <int D> struct Lds16 {
    static constexpr int KP = D + 8;         // K row pitch (elements): +16 B against bank conflicts
    static constexpr int VP = BN16 + 8;      // V^T row pitch (elements)
    static constexpr int K_ELEMS = BN16 * KP;
    static constexpr int V_ELEMS = D * VP;
    static constexpr int BUF = K_ELEMS + V_ELEMS;
    static constexpr int BYTES = 2 * BUF * 2;  // two buffers of 16-bit elements
};

// Slot of key `kk` (0..63 within a tile) in a V^T row.  Inside every 16-key group
// the 4-key chunks 1 and 2 trade places, so that lane half h of MFMA step t reads
// its 8 keys {16t + 4h + 0..3, 16t + 8 + 4h + 0..3} as one contiguous 16-byte run,
// matching the keys that P^T holds in accumulator registers 8(t%2) .. 8(t%2)+7.
__device__ __forceinline__ int vt_slot(int kk) {
    const int ch = (kk >> 2) & 3;
    const int sw = (ch == 1) ? 2 : (ch == 2) ? 1 : ch;
    return (kk & ~15) | (sw << 2) | (kk & 3);
}

// Weights are taken relative to a per-query reference m that is raised only when a
// new score exceeds it by more than this many powers of two (then O and both sums
// are rescaled exactly); in between, weights stay below 2^8, far from overflow.
constexpr float RESCALE_LOG2 = 8.0f;

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_16(AttnParams p) {
    typedef Elem16<DT> E;
    typedef typename E::vec8 vec8;
    typedef Lds16<D> L;
    constexpr int KSTEPS = D / 16;       // MFMA k-steps for S^T
    constexpr int DBLK = D / 32;         // 32-row blocks of O^T
    constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
    constexpr int K_ITERS = BN16 * CPR / 256;
    constexpr int V_ITEMS = (BN16 / 4) * CPR;   // (4-key group, chunk) items

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 31;     // query column (S^T, O^T) / key row (K) / d row (V^T)
    const int h = lane >> 5;     // half-wave

    const TileCoord tc = map_tile(p, blockIdx.x);
    const int kvh = tc.hq / (p.Hq / p.Hkv);
    const int off = p.Sk - p.Sq;
    const int qs = tc.qt * BM16;                 // first query of the workgroup
    const int qw = qs + wave * (QBLK * 32);      // first query of this wave

    const uint16_t* __restrict__ Qg = (const uint16_t*)p.q + ((int64_t)(tc.b * p.Hq + tc.hq) * p.Sq) * D;
    const uint16_t* __restrict__ Kg = (const uint16_t*)p.k + ((int64_t)(tc.b * p.Hkv + kvh) * p.Sk) * D;
    const uint16_t* __restrict__ Vg = (const uint16_t*)p.v + ((int64_t)(tc.b * p.Hkv + kvh) * p.Sk) * D;
    uint16_t* __restrict__ Og = (uint16_t*)p.o + ((int64_t)(tc.b * p.Hq + tc.hq) * p.Sq) * D;

    // key range of the workgroup
    const int last_q = min(qs + BM16, p.Sq) - 1;
    int kend = p.Sk;
    if (CAUSAL) kend = min(p.Sk, last_q + off + 1);
    const int ntiles = kend > 0 ? (kend + BN16 - 1) / BN16 : 0;
    // key range of this wave
    const int wlast_q = min(qw + QBLK * 32, p.Sq) - 1;
    int wkend = (qw < p.Sq) ? p.Sk : 0;
    if (CAUSAL && qw < p.Sq) wkend = min(p.Sk, wlast_q + off + 1);

    // ---- Q^T fragments (B operand), kept in registers for the whole kernel
    vec8 qf[QBLK][KSTEPS];
    {
        const uint32_t qx = (p.q_mode == 1) ? 0x80008000u : 0u;
#pragma unroll
        for (int b = 0; b < QBLK; ++b) {
            const int qrow = qw + 32 * b + n;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                u32x4 raw = {0u, 0u, 0u, 0u};
                if (qrow < p.Sq && p.q_mode != 2)
                    raw = *(const u32x4*)(Qg + (int64_t)qrow * D + 16 * s + 8 * h);
                raw ^= qx;
                qf[b][s] = __builtin_bit_cast(vec8, raw);
            }
        }
    }

    f32x16 oacc[DBLK][QBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int b = 0; b < QBLK; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[d][b][r] = 0.f;
    // per query (this lane's column): reference m (log2 domain), and the partial
    // sums of this half-wave's weights in fp32 (le, for the LSE) and of the same
    // weights as rounded to 16 bits (lr, the normaliser of O, so that O is an
    // exactly normalised mix of V rows)
    float m_run[QBLK], le_run[QBLK], lr_run[QBLK];
#pragma unroll
    for (int b = 0; b < QBLK; ++b) { m_run[b] = NEG_INF; le_run[b] = 0.f; lr_run[b] = 0.f; }

    // ---- global -> register staging of one K/V tile
    u32x4 kreg[K_ITERS];
    u32x4 vreg[4];
    const int kc = tid % CPR;            // K chunk handled by this thread
    const int kr0 = tid / CPR;           // first K row handled by this thread
    const bool v_item = tid < V_ITEMS;
    const int vc = tid % CPR;            // V chunk
    const int vg = tid / CPR;            // V 4-key group

    auto load_tile = [&](int j) {
        const int k0 = j * BN16;
#pragma unroll
        for (int i = 0; i < K_ITERS; ++i) {
            const int row = k0 + kr0 + i * (256 / CPR);
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row < p.Sk) x = *(const u32x4*)(Kg + (int64_t)row * D + 8 * kc);
            kreg[i] = x;
        }
        if (v_item) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = k0 + 4 * vg + i;
                u32x4 x = {0u, 0u, 0u, 0u};
                if (row < p.Sk) x = *(const u32x4*)(Vg + (int64_t)row * D + 8 * vc);
                vreg[i] = x;
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* kb = smem + buf * L::BUF;
        uint16_t* vb = kb + L::K_ELEMS;
#pragma unroll
        for (int i = 0; i < K_ITERS; ++i) {
            const int row = kr0 + i * (256 / CPR);
            *(u32x4*)(kb + row * L::KP + 8 * kc) = kreg[i];
        }
        if (v_item) {
            const int slot = vt_slot(4 * vg);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // d = 8*vc + 2w (low halves) and 8*vc + 2w + 1 (high halves)
                const uint32_t a0 = vreg[0][w], a1 = vreg[1][w], a2 = vreg[2][w], a3 = vreg[3][w];
                u32x2 ev, od;
                ev[0] = (a0 & 0xffffu) | (a1 << 16);
                ev[1] = (a2 & 0xffffu) | (a3 << 16);
                od[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                od[1] = (a2 >> 16) | (a3 & 0xffff0000u);
                *(u32x2*)(vb + (8 * vc + 2 * w) * L::VP + slot) = ev;
                *(u32x2*)(vb + (8 * vc + 2 * w + 1) * L::VP + slot) = od;
            }
        }
    };

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        const bool more = (j + 1) < ntiles;
        if (more) load_tile(j + 1);

        const uint16_t* kb = smem + buf * L::BUF;
        const uint16_t* vb = kb + L::K_ELEMS;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int ks0 = j * BN16 + 32 * sub;     // first key of this 32-key sub-tile
            if (ks0 >= wkend) break;                 // above this wave's diagonal

            // ---- S^T = K . Q^T for 32 keys x 64 queries
            f32x16 sacc[QBLK];
#pragma unroll
            for (int b = 0; b < QBLK; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[b][r] = 0.f;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const vec8 a = *(const vec8*)(kb + (32 * sub + n) * L::KP + 16 * s + 8 * h);
#pragma unroll
                for (int b = 0; b < QBLK; ++b) sacc[b] = E::mfma(a, qf[b][s], sacc[b]);
            }

            // ---- mask: causal diagonal sub-tiles and the ragged key tail
            const bool need_mask = (ks0 + 32 > p.Sk) || (CAUSAL && (ks0 + 31 > qw + off));
            if (need_mask) {
#pragma unroll
                for (int b = 0; b < QBLK; ++b) {
                    const int qi = qw + 32 * b + n;
                    const int lim = CAUSAL ? min(p.Sk - 1, qi + off) : (p.Sk - 1);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = ks0 + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (key > lim) sacc[b][r] = NEG_INF;
                    }
                }
            }

            // ---- online softmax in the log2 domain: t = s * c, c = |scale| * log2(e)
            float mx[QBLK];
            bool raise = false;
#pragma unroll
            for (int b = 0; b < QBLK; ++b) {
                float x = NEG_INF;
#pragma unroll
                for (int r = 0; r < 16; ++r) x = fmaxf(x, sacc[b][r]);
                mx[b] = pair_max(x) * p.c;
                raise |= mx[b] > m_run[b] + RESCALE_LOG2;
            }
            if (__any(raise)) {
                // new reference = exact running max; rescale O and both sums
#pragma unroll
                for (int b = 0; b < QBLK; ++b) {
                    const float m_new = fmaxf(m_run[b], mx[b]);
                    const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run[b] - m_new);
                    m_run[b] = m_new;
                    le_run[b] *= alpha;
                    lr_run[b] *= alpha;
#pragma unroll
                    for (int d = 0; d < DBLK; ++d)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[d][b][r] *= alpha;
                }
            }
            uint32_t pk[QBLK][8];
#pragma unroll
            for (int b = 0; b < QBLK; ++b) {
                const float m_use = (m_run[b] == NEG_INF) ? 0.f : m_run[b];
                float se = 0.f, sr = 0.f;
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = fast_exp2(fmaf(sacc[b][r], p.c, -m_use));
                    const float p1 = fast_exp2(fmaf(sacc[b][r + 1], p.c, -m_use));
                    se += p0;
                    se += p1;
                    const uint32_t w = E::pack(p0, p1);
                    pk[b][r >> 1] = w;
                    sr = E::dot2_ones(w, sr);
                }
                le_run[b] += se;
                lr_run[b] += sr;
            }

            // ---- O^T += V^T . P^T  (two 16-key MFMA steps)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int t = 2 * sub + hf;
                vec8 bfr[QBLK];
#pragma unroll
                for (int b = 0; b < QBLK; ++b) {
                    u32x4 w = {pk[b][4 * hf + 0], pk[b][4 * hf + 1], pk[b][4 * hf + 2], pk[b][4 * hf + 3]};
                    bfr[b] = __builtin_bit_cast(vec8, w);
                }
#pragma unroll
                for (int d = 0; d < DBLK; ++d) {
                    const vec8 a = *(const vec8*)(vb + (32 * d + n) * L::VP + 16 * t + 8 * h);
#pragma unroll
                    for (int b = 0; b < QBLK; ++b) oacc[d][b] = E::mfma(a, bfr[b], oacc[d][b]);
                }
            }
        }

        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / lr, rounded once; LSE = ln2 * (m + log2 le)
#pragma unroll
    for (int b = 0; b < QBLK; ++b) {
        const int qi = qw + 32 * b + n;
        const float lr = pair_sum(lr_run[b]);
        const float le = pair_sum(le_run[b]);
        const float inv = (lr > 0.f) ? 1.f / lr : 0.f;
        if (qi < p.Sq) {
            uint16_t* orow = Og + (int64_t)qi * D;
#pragma unroll
            for (int d = 0; d < DBLK; ++d)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = E::pack(oacc[d][b][4 * g + 0] * inv, oacc[d][b][4 * g + 1] * inv);
                    w[1] = E::pack(oacc[d][b][4 * g + 2] * inv, oacc[d][b][4 * g + 3] * inv);
                    *(u32x2*)(orow + 32 * d + 8 * g + 4 * h) = w;
                }
            if (p.lse && h == 0) {
                const float lse = (le > 0.f) ? (m_run[b] + __log2f(le)) * 0.69314718055994531f
                                             : NEG_INF;
                p.lse[(int64_t)(tc.b * p.Hq + tc.hq) * p.Sq + qi] = lse;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel: v_mfma_f32_32x32x2_f32, 4 waves x 32 queries, 32-key tiles.
// ---------------------------------------------------------------------------
constexpr int BM32 = 128;
constexpr int BN32 = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_32(AttnParams p) {
    constexpr int KP = D + 1;       // row pitch (floats) of the K and V tiles
    constexpr int KSTEPS = D / 2;
    constexpr int DBLK = D / 32;
    __shared__ float ks[BN32 * KP];
    __shared__ float vs[BN32 * KP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 31;
    const int h = lane >> 5;

    const TileCoord tc = map_tile(p, blockIdx.x);
    const int kvh = tc.hq / (p.Hq / p.Hkv);
    const int off = p.Sk - p.Sq;
    const int qs = tc.qt * BM32;
    const int qw = qs + wave * 32;

    const float* __restrict__ Qg = (const float*)p.q + ((int64_t)(tc.b * p.Hq + tc.hq) * p.Sq) * D;
    const float* __restrict__ Kg = (const float*)p.k + ((int64_t)(tc.b * p.Hkv + kvh) * p.Sk) * D;
    const float* __restrict__ Vg = (const float*)p.v + ((int64_t)(tc.b * p.Hkv + kvh) * p.Sk) * D;
    float* __restrict__ Og = (float*)p.o + ((int64_t)(tc.b * p.Hq + tc.hq) * p.Sq) * D;

    const int last_q = min(qs + BM32, p.Sq) - 1;
    int kend = p.Sk;
    if (CAUSAL) kend = min(p.Sk, last_q + off + 1);
    const int ntiles = kend > 0 ? (kend + BN32 - 1) / BN32 : 0;
    const int wlast_q = min(qw + 32, p.Sq) - 1;
    int wkend = (qw < p.Sq) ? p.Sk : 0;
    if (CAUSAL && qw < p.Sq) wkend = min(p.Sk, wlast_q + off + 1);

    // Q^T fragments: lane (n, h) holds Q[qw + n][2s + h]
    float qf[KSTEPS];
    {
        const int qrow = qw + n;
        const float sgn = (p.q_mode == 1) ? -1.f : 1.f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            float x = 0.f;
            if (qrow < p.Sq && p.q_mode != 2) x = Qg[(int64_t)qrow * D + 2 * s + h] * sgn;
            qf[s] = x;
        }
    }
    f32x16 oacc[DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    float m_run = NEG_INF, l_run = 0.f;

    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BN32;
        __syncthreads();     // previous tile fully consumed
        for (int e = tid; e < BN32 * D; e += 256) {
            const int row = e / D, col = e % D;
            float kx = 0.f, vx = 0.f;
            if (k0 + row < p.Sk) {
                kx = Kg[(int64_t)(k0 + row) * D + col];
                vx = Vg[(int64_t)(k0 + row) * D + col];
            }
            ks[row * KP + col] = kx;
            vs[row * KP + col] = vx;
        }
        __syncthreads();
        if (k0 >= wkend) continue;

        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[n * KP + 2 * s + h], qf[s], sacc, 0, 0, 0);

        const bool need_mask = (k0 + BN32 > p.Sk) || (CAUSAL && (k0 + BN32 - 1 > qw + off));
        if (need_mask) {
            const int qi = qw + n;
            const int lim = CAUSAL ? min(p.Sk - 1, qi + off) : (p.Sk - 1);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (key > lim) sacc[r] = NEG_INF;
            }
        }
        float mx = NEG_INF;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run, mx * p.c);
        const bool empty = (m_new == NEG_INF);
        const float m_use = empty ? 0.f : m_new;
        const float alpha = empty ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sacc[r] = fast_exp2(fmaf(sacc[r], p.c, -m_use));
            rs += sacc[r];
        }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
        // O^T += V^T . P^T: step r pairs accumulator register r (key 8(r/4) + 4h + r%4)
        // with the V row of the same key
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
            for (int d = 0; d < DBLK; ++d)
                oacc[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * KP + 32 * d + n], sacc[r],
                                                                oacc[d], 0, 0, 0);
        }
    }

    const int qi = qw + n;
    const float l_tot = pair_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qi < p.Sq) {
        float* orow = Og + (int64_t)qi * D;
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) orow[32 * d + 8 * (r >> 2) + 4 * h + (r & 3)] = oacc[d][r] * inv;
        if (p.lse && h == 0) {
            const float lse = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : NEG_INF;
            p.lse[(int64_t)(tc.b * p.Hq + tc.hq) * p.Sq + qi] = lse;
        }
    }
}

// ---------------------------------------------------------------------------
// kernel selection
// ---------------------------------------------------------------------------
template <int DT, int D>
static const void* pick16(int causal) {
    return causal ? (const void*)&attn_fwd_16<DT, D, true> : (const void*)&attn_fwd_16<DT, D, false>;
}
template <int D>
static const void* pick32(int causal) {
    return causal ? (const void*)&attn_fwd_32<D, true> : (const void*)&attn_fwd_32<D, false>;
}

KernelChoice select_kernel(int dtype, int D, int causal) {
    KernelChoice kc = {nullptr, 0, 0};
    if (dtype == ATTN_IMPL_FP32) {
        kc.bm = BM32;
        kc.threads = 256;
        kc.fn = (D == 64) ? pick32<64>(causal) : (D == 128) ? pick32<128>(causal) : nullptr;
        return kc;
    }
    kc.bm = BM16;
    kc.threads = 256;
    if (dtype == ATTN_IMPL_BF16)
        kc.fn = (D == 64) ? pick16<ATTN_IMPL_BF16, 64>(causal)
              : (D == 128) ? pick16<ATTN_IMPL_BF16, 128>(causal) : nullptr;
    else if (dtype == ATTN_IMPL_FP16)
        kc.fn = (D == 64) ? pick16<ATTN_IMPL_FP16, 64>(causal)
              : (D == 128) ? pick16<ATTN_IMPL_FP16, 128>(causal) : nullptr;
    return kc;
}

}  // namespace attn_impl
