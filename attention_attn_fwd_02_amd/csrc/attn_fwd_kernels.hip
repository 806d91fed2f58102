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
// 16-bit path (bf16, fp16): workgroups of 4 waves, two workgroups per CU (two
// waves per SIMD, so one wave's MFMAs overlap the other's softmax arithmetic):
//   * the workgroup owns BM = 128 consecutive queries of one (batch, head); each
//     wave owns 32 of them, one 32-query column block;
//   * the wave computes S^T = K_tile . Q^T with v_mfma_f32_32x32x16_{bf16,f16}:
//     K (keys x D) is the A operand read from LDS, Q^T the B operand held in
//     VGPRs for the whole kernel.  In the 32x32 accumulator layout every lane
//     holds one query column, so the row max and row sums of the online softmax
//     are in-lane reductions plus one v_permlane32_swap between the half-waves;
//   * the weights P^T are rounded to 16 bits in registers and feed the next MFMA
//     directly as its B operand: O^T (D x queries) += V^T . P^T.  The A operand
//     V^T comes from the row-major V tile through ds_read_b64_tr_b16 (the LDS
//     transposing read), two reads per MFMA, in the key order P^T already has;
//   * K and V tiles of 64 keys go from HBM to LDS by buffer_load ... lds (no
//     VGPR staging; rows past Sk read as zero) into rows padded against bank
//     conflicts, double-buffered with one barrier per tile.
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

// Workgroup -> (batch, query head, query tile).  Workgroups are taken in "bundles"
// of p.gbundle consecutive key/value-head groups; inside a bundle the order is
// query tile first (heaviest causal tiles of every head in the bundle before any
// lighter one), then group, then query head.  A bundle is sized (on the host) to
// fill the workgroup slots of an XCD, which keeps the causal tail balanced while
// the K/V heads in flight stay few enough for one XCD's L2.  When the groups split
// evenly over the 8 XCDs (workgroup w is dispatched to XCD w % 8), each XCD gets
// whole bundles, so every query tile and query head that reads one K/V head runs
// on the XCD that caches it.
struct TileCoord { int b, hq, qt; };
__device__ __forceinline__ TileCoord map_tile(const AttnParams& p, int w) {
    const int R = p.Hq / p.Hkv;      // query heads per key/value head
    const int G = p.gbundle;         // key/value-head groups per bundle
    const int BU = G * R * p.nq;     // workgroups per bundle
    int bundle, u;
    if (p.xcd_remap) {
        const int xcd = w & 7, slot = w >> 3;
        bundle = xcd + 8 * (slot / BU);
        u = slot % BU;
    } else {
        bundle = w / BU;
        u = w % BU;
    }
    TileCoord t;
    t.qt = p.nq - 1 - u / (G * R);
    const int g = bundle * G + (u / R) % G;
    const int r = u % R;
    t.b = g / p.Hkv;
    t.hq = (g % p.Hkv) * R + r;
    return t;
}

// ---------------------------------------------------------------------------
// 16-bit kernel
// ---------------------------------------------------------------------------
constexpr int NW = 4;            // waves per workgroup (one per SIMD)
constexpr int QPW = 32;          // queries per wave: one 32-column block of S^T / O^T
constexpr int BM16 = NW * QPW;   // queries per workgroup
constexpr int BN16 = 64;         // keys per tile (two 32-key blocks)

// Weights are taken relative to a per-query reference m that is raised only when a
// new score exceeds it by more than this many powers of two (then O and both sums
// are rescaled exactly); in between, weights stay below 2^8, far from overflow.
constexpr float RESCALE_LOG2 = 8.0f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// LDS tiles hold K and V row-major ([key][d]) with padded rows, chosen so that
// both MFMA operand reads are free of bank conflicts (64 banks x 4 bytes):
//   K, ds_read_b128: 16 lanes read one 16-byte slot of 16 consecutive rows; a
//     pitch of 2D + 16 bytes puts those rows 16 bytes apart modulo 256;
//   V, ds_read_b64_tr_b16: 32 lanes read 64 bytes of 4 consecutive rows; a pitch
//     of 2D + 64 bytes puts those rows 64 bytes apart modulo 256.
// Every operand read is then one lane base plus a compile-time offset.
template <int D> struct Tile16 {
    static constexpr int ROW = 2 * D;                  // bytes of one K/V row in HBM
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int KPITCH = ROW + 16;
    static constexpr int VPITCH = ROW + 64;
    static constexpr int KSLOTS = KPITCH / 16;         // 16-byte LDS slots per K row
    static constexpr int VSLOTS = VPITCH / 16;
    static constexpr int KBYTES = BN16 * KPITCH;       // multiple of 1024
    static constexpr int VBYTES = BN16 * VPITCH;
    static constexpr int BUF = KBYTES + VBYTES;        // one K tile then one V tile
    static constexpr int KDMA = KBYTES / 1024;         // 1 KB DMA instructions per K tile
    static constexpr int VDMA = VBYTES / 1024;
    static constexpr int KDMA_W = (KDMA + NW - 1) / NW;   // per wave (the last may be idle)
    static constexpr int VDMA_W = (VDMA + NW - 1) / NW;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // raw buffer: stride 0, num_records = bytes (loads past it return zero)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// voffset that always lies past num_records (per-head slices are < 2^31 bytes and
// the tile offset added through soffset is < 2^31): the DMA lane writes zeros
// into a padding slot without touching memory.
constexpr uint32_t OOB_VOFFSET = 0x7fff0000u;

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_16(AttnParams p) {
    typedef Elem16<DT> E;
    typedef typename E::vec8 vec8;
    typedef Tile16<D> T;
    constexpr int KSTEPS = D / 16;       // MFMA k-steps for S^T
    constexpr int DBLK = D / 32;         // 32-row blocks of O^T

    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform across the wave; readfirstlane tells the compiler,
    // so every per-wave decision below is a scalar branch, not an exec mask
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;     // query column (S^T, O^T) / key row (K) / d row (V^T)
    const int h = lane >> 5;     // half-wave

    const TileCoord tc = map_tile(p, blockIdx.x);
    const int kvh = tc.hq / (p.Hq / p.Hkv);
    const int off = p.Sk - p.Sq;
    const int qs = tc.qt * BM16;                 // first query of the workgroup
    const int qw = qs + wave * QPW;              // first query of this wave

    const int64_t q_head = (int64_t)(tc.b * p.Hq + tc.hq) * p.Sq;
    const int64_t kv_head = (int64_t)(tc.b * p.Hkv + kvh) * p.Sk;
    const uint8_t* Qg = (const uint8_t*)p.q + q_head * T::ROW;
    const uint8_t* Kg = (const uint8_t*)p.k + kv_head * T::ROW;
    const uint8_t* Vg = (const uint8_t*)p.v + kv_head * T::ROW;
    uint16_t* __restrict__ Og = (uint16_t*)p.o + q_head * D;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(Qg, (uint32_t)p.Sq * T::ROW);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(Kg, (uint32_t)p.Sk * T::ROW);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vg, (uint32_t)p.Sk * T::ROW);

    // key range of the workgroup and of this wave
    const int last_q = min(qs + BM16, p.Sq) - 1;
    int kend = p.Sk;
    if (CAUSAL) kend = min(p.Sk, last_q + off + 1);
    const int ntiles = kend > 0 ? (kend + BN16 - 1) / BN16 : 0;
    int wkend = (qw < p.Sq) ? p.Sk : 0;
    if (CAUSAL && qw < p.Sq) wkend = min(p.Sk, min(qw + QPW, p.Sq) - 1 + off + 1);

    // ---- Q^T fragments (B operand): lane (n, h) holds Q[qw + n][16s + 8h .. +7];
    // rows past Sq read as zero
    vec8 qf[KSTEPS];
    {
        const uint32_t qx = (p.q_mode == 1) ? 0x80008000u : 0u;
        const uint32_t qz = (p.q_mode == 2) ? 0u : 0xffffffffu;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const uint32_t vo = (uint32_t)(qw + n) * T::ROW + (16 * s + 8 * h) * 2;
            u32x4 raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, vo, 0, 0));
            raw = (raw & qz) ^ qx;
            qf[s] = __builtin_bit_cast(vec8, raw);
        }
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    // per query (this lane's column): reference m (log2 domain), and the partial
    // sums of this half-wave's weights in fp32 (le, for the LSE) and of the same
    // weights as rounded to 16 bits (lr, the normaliser of O, so that O is an
    // exactly normalised mix of V rows)
    float m_run = NEG_INF, le_run = 0.f, lr_run = 0.f;

    // ---- DMA lane offsets (loop-invariant): DMA instruction i of this wave fills
    // LDS slots 64*(wave + NW*i) + lane; a slot is (row, chunk) of the padded tile,
    // and padding slots get an out-of-range offset
    constexpr int KDMA_W = T::KDMA_W, VDMA_W = T::VDMA_W;
    // fixed bounds: an array sized by a template-dependent constant makes the host
    // compilation pass drop this kernel's launch stub
    static_assert(KDMA_W <= 8 && VDMA_W <= 8, "DMA offsets per wave");
    uint32_t kvo[8], vvo[8];
#pragma unroll
    for (int i = 0; i < KDMA_W; ++i) {
        const int slot = 64 * (wave + NW * i) + lane;
        const int row = slot / T::KSLOTS, c = slot % T::KSLOTS;
        kvo[i] = (c < T::CPR) ? (uint32_t)(row * T::ROW + 16 * c) : OOB_VOFFSET;
    }
#pragma unroll
    for (int i = 0; i < VDMA_W; ++i) {
        const int slot = 64 * (wave + NW * i) + lane;
        const int row = slot / T::VSLOTS, c = slot % T::VSLOTS;
        vvo[i] = (c < T::CPR) ? (uint32_t)(row * T::ROW + 16 * c) : OOB_VOFFSET;
    }
    auto dma_tile = [&](int j, uint8_t* __restrict__ dst) {
        const uint32_t so = (uint32_t)(j * BN16) * T::ROW;     // tile start, via soffset
#pragma unroll
        for (int i = 0; i < T::KDMA_W; ++i)
            if (wave + NW * i < T::KDMA)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void_t*)(dst + 1024 * (wave + NW * i)),
                                                         16, kvo[i], so, 0, 0);
#pragma unroll
        for (int i = 0; i < T::VDMA_W; ++i)
            if (wave + NW * i < T::VDMA)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)(dst + T::KBYTES + 1024 * (wave + NW * i)),
                                                         16, vvo[i], so, 0, 0);
    };

    // lane bases of the operand reads (bytes within one buffer)
    const int k_lane = n * T::KPITCH + 16 * h;
    const int tr_row = (lane & 15) >> 2;
    const int v_lane = T::KBYTES + (4 * h + tr_row) * T::VPITCH + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1);

    if (ntiles > 0) dma_tile(0, smem);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA has landed
    __syncthreads();

    // One key tile: start the DMA of tile j+1 into `nxt`, then compute tile j from
    // `cur`.  The two LDS buffers never overlap; saying so (__restrict__) lets the
    // compiler read `cur` while the DMA into `nxt` is still in flight instead of
    // waiting for it.  Tile j+1 is waited for (vmcnt) at the barrier after the step.
    auto tile_step = [&](int j, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt) {
        if (j + 1 < ntiles) dma_tile(j + 1, nxt);

        const int k0 = j * BN16;
        if (k0 >= wkend) return;             // tile wholly above this wave's diagonal
        const uint8_t* kt = cur + k_lane;
        const uint8_t* vt = cur + v_lane;

        // ---- S^T = K . Q^T  (two 32-key blocks)
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const vec8 a = *(const vec8*)(kt + 32 * kb * T::KPITCH + 32 * s);
                sacc[kb] = E::mfma(a, qf[s], sacc[kb]);
            }
        }

        // ---- mask: causal diagonal tiles and the ragged key tail
        const bool need_mask = (k0 + BN16 > p.Sk) || (CAUSAL && (k0 + BN16 - 1 > qw + off));
        if (need_mask) {
            const int qi = qw + n;
            const int lim = (CAUSAL ? min(p.Sk - 1, qi + off) : (p.Sk - 1)) - (k0 + 4 * h);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * kb + 8 * (r >> 2) + (r & 3);    // relative to k0 + 4h
                    if (key > lim) sacc[kb][r] = NEG_INF;
                }
        }

        // ---- online softmax in the log2 domain: t = s * c, c = |scale| * log2(e)
        float mp[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mp[r & 3] = fmaxf(mp[r & 3], sacc[kb][r]);
        float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
        mx = pair_max(mx) * p.c;
        if (__any(mx > m_run + RESCALE_LOG2)) {
            // new reference = exact running max; rescale O and both sums
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            le_run *= alpha;
            lr_run *= alpha;
#pragma unroll
            for (int d = 0; d < DBLK; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
        }
        const float m_use = (m_run == NEG_INF) ? 0.f : m_run;
        uint32_t pk[2][8];
        float se[4] = {0.f, 0.f, 0.f, 0.f}, sr[2] = {0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(sacc[kb][r], p.c, -m_use));
                const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], p.c, -m_use));
                se[r & 3] += p0;
                se[(r & 3) + 1] += p1;
                const uint32_t w = E::pack(p0, p1);
                pk[kb][r >> 1] = w;
                sr[(r >> 1) & 1] = E::dot2_ones(w, sr[(r >> 1) & 1]);
            }
        le_run += (se[0] + se[1]) + (se[2] + se[3]);
        lr_run += sr[0] + sr[1];

        // ---- O^T += V^T . P^T  (four 16-key steps).  A operand from the row-major V
        // tile by two transposing reads: lane l receives V[key0 + j][32db + (l % 32)],
        // j = 0..3, with key0 = 16t + 8rr + 4h, which are exactly the keys that P^T
        // holds in accumulator registers 8(t % 2) + 4rr + j.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int kb = t >> 1, hf = t & 1;
            u32x4 bw = {pk[kb][4 * hf + 0], pk[kb][4 * hf + 1], pk[kb][4 * hf + 2], pk[kb][4 * hf + 3]};
            const vec8 bfr = __builtin_bit_cast(vec8, bw);
#pragma unroll
            for (int d = 0; d < DBLK; ++d) {
                const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t*)(vt + (16 * t) * T::VPITCH + 64 * d));
                const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t*)(vt + (16 * t + 8) * T::VPITCH + 64 * d));
                const short8_t a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[d] = E::mfma(__builtin_bit_cast(vec8, a8), bfr, oacc[d]);
            }
        }
        // interleave: weights of the first 32 keys, then P.V of those keys under the
        // weights of the second 32, then the rest of P.V
        __builtin_amdgcn_sched_group_barrier(0x002, 60, 0);
#pragma unroll
        for (int i = 0; i < 2 * DBLK; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
#pragma unroll
        for (int i = 0; i < 2 * DBLK; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    };

    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        tile_step(j, smem + buf * T::BUF, smem + (buf ^ 1) * T::BUF);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): next tile's DMA has landed
        __syncthreads();
    }

    // ---- epilogue: O = O^T / lr, rounded once; LSE = ln2 * (m + log2 le)
    {
        const int qi = qw + n;
        const float lr = pair_sum(lr_run);
        const float le = pair_sum(le_run);
        const float inv = (lr > 0.f) ? 1.f / lr : 0.f;
        if (qi < p.Sq) {
            uint16_t* orow = Og + (int64_t)qi * D;
#pragma unroll
            for (int d = 0; d < DBLK; ++d)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = E::pack(oacc[d][4 * g + 0] * inv, oacc[d][4 * g + 1] * inv);
                    w[1] = E::pack(oacc[d][4 * g + 2] * inv, oacc[d][4 * g + 3] * inv);
                    *(u32x2*)(orow + 32 * d + 8 * g + 4 * h) = w;
                }
            if (p.lse && h == 0) {
                const float lse = (le > 0.f) ? (m_run + __log2f(le)) * 0.69314718055994531f : NEG_INF;
                p.lse[q_head + qi] = lse;
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
