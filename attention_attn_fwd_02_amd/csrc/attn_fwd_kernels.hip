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
// 16-bit path (bf16, fp16): workgroups of 8 waves, one workgroup per CU (two
// waves per SIMD, so one wave's MFMAs overlap the other's softmax arithmetic):
//   * the workgroup owns BM = 256 consecutive queries of one (batch, head); each
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
//     conflicts, double-buffered with one barrier per tile, K one tile ahead of V;
//   * each wave software-pipelines its tiles in two phases of 16 MFMAs: the
//     scores of the next tile and P.V of the current one go to the matrix core
//     while the VALU computes the weights of the other 32-key block, so the two
//     units work on independent data;
//   * the softmax reference m is raised only when needed (first visible keys, or
//     a block whose weights sum past 2^8), so the common path has no max pass.
// fp32 inputs run the kernels of attn_fwd32_kernels.hip (the same dataflow with true
// fp32 products); select_kernel below hands them over.
//
// The mask, the grouped-head mapping and the empty-row convention are those of
// include/attn_fwd.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_internal.h"
#include "attn_kernel_common.h"
#include "attn_fwd_tile_map.h"

namespace attn_impl {

// ---------------------------------------------------------------------------
// 16-bit kernel
// ---------------------------------------------------------------------------
constexpr int NW = 8;            // waves per workgroup (two per SIMD, one workgroup per CU)
constexpr int QPW = 32;          // queries per wave: one 32-column block of S^T / O^T
constexpr int BM16 = NW * QPW;   // queries per workgroup
constexpr int BN16 = 64;         // keys per tile (two 32-key blocks)

// Weights are taken relative to a per-query reference m that is raised (and O and
// the weight sum rescaled exactly) only when a 32-key block's weights sum past
// 2^RESCALE_LOG2; every accepted weight is therefore below 2^8, far from overflow.
constexpr float RESCALE_LOG2 = 8.0f;
constexpr float RESCALE_SUM = 256.0f;      // 2^RESCALE_LOG2

// Issue order inside one pipeline phase: KS score MFMAs (one K read each), then
// 2*DB P.V MFMAs (two V reads each), with two VALU instructions of the softmax
// after every MFMA (the rest of the softmax fills in behind them) and the LDS
// reads kept PHASE_LOOKAHEAD MFMAs ahead of their use.
constexpr int PHASE_VALU = 2;
constexpr int PHASE_LOOKAHEAD = 4;
// LDS reads that must have been issued before MFMA i of the phase
template <int KS, int DB> constexpr int phase_reads(int i) {
    return i >= KS + 2 * DB ? KS + 4 * DB : (i < KS ? i + 1 : KS + 2 * (i - KS + 1));
}
template <int KS, int DB, int I>
__device__ __forceinline__ void phase_schedule_from() {
    if constexpr (I < KS + 2 * DB) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, PHASE_VALU, 0);   // VALU
        constexpr int more = phase_reads<KS, DB>(I + PHASE_LOOKAHEAD) - phase_reads<KS, DB>(I + PHASE_LOOKAHEAD - 1);
        if constexpr (more > 0) __builtin_amdgcn_sched_group_barrier(0x100, more, 0);   // DS read
        phase_schedule_from<KS, DB, I + 1>();
    }
}
template <int KS, int DB>
__device__ __forceinline__ void phase_schedule() {
    __builtin_amdgcn_sched_group_barrier(0x100, phase_reads<KS, DB>(PHASE_LOOKAHEAD - 1), 0);
    phase_schedule_from<KS, DB, 0>();
}


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

template <int DT, int D, bool CAUSAL, int ROPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_16(AttnParams p) {
    typedef Elem16<DT> E;
    typedef typename E::vec8 vec8;
    typedef Tile16<D> T;
    constexpr int KSTEPS = D / 16;       // MFMA k-steps for S^T
    constexpr int DBLK = D / 32;         // 32-row blocks of O^T

    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::BUF + 1024 + NW * QPW * (T::ROW + 16)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform across the wave; readfirstlane tells the compiler,
    // so every per-wave decision below is a scalar branch, not an exec mask
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;     // query column (S^T, O^T) / key row (K) / d row (V^T)
    const int h = lane >> 5;     // half-wave

    const TileCoord tc = map_tile(p, blockIdx.x);
    const int kvh = tc.kvh;
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
    const uint32_t qx = (p.q_mode == 1) ? 0x80008000u : 0u;
    const uint32_t qz = (p.q_mode == 2) ? 0u : 0xffffffffu;
    u32x4 raw[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        const uint32_t vo = (uint32_t)(qw + n) * T::ROW + (16 * s + 8 * h) * 2;
        raw[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, vo, 0, 0));
    }
    // rotary embedding: query qi sits at position qi + Sk - Sq; the tables hold
    // positions 0 .. Sk-1 and read as zero past them (rows past Sq, zero anyway).
    // Interleaved pairs: dword e of fragment s is pair 8s + 4h + e, one 16-byte
    // table load per fragment.  Split halves: element j of fragment s pairs with
    // element j of fragment s + KSTEPS/2 as pair 16s + 8h + j, two table loads
    // (entries 2s, 2s+1) per fragment pair.
    u32x4 cv[KSTEPS], sv[KSTEPS];
    if constexpr (ROPE != 0) {
        constexpr int HALF = D / 2;
        const __amdgpu_buffer_rsrc_t cr = make_rsrc(p.rcos, (uint32_t)p.Sk * HALF * 4);
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.rsin, (uint32_t)p.Sk * HALF * 4);
        const uint32_t tab = (uint32_t)(qw + n + off) * (HALF * 4);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const uint32_t to = (ROPE == 1) ? tab + (8 * s + 4 * h) * 4
                                            : tab + (16 * (s >> 1) + 8 * h) * 4 + 16 * (s & 1);
            cv[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, to, 0, 0));
            sv[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, to, 0, 0));
        }
    }
    // the fragments as MFMA operands: rotated (rotary kernels; done once the first
    // tiles' DMA is in flight, so it overlaps their latency), then the sign or zero
    // of the scale applied
    auto finish_q = [&]() {
        if constexpr (ROPE == 1) {
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float ra, rb;
                    rope_rotate(E::lo(raw[s][e]), E::hi(raw[s][e]), u2f(cv[s][e]), u2f(sv[s][e]), ra, rb);
                    raw[s][e] = E::pack(ra, rb);
                }
        } else if constexpr (ROPE == 2) {
#pragma unroll
            for (int s = 0; s < KSTEPS / 2; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t wa = raw[s][e], wb = raw[s + KSTEPS / 2][e];
                    const int t = 2 * s + (e >> 1), c0 = 2 * (e & 1);
                    float ra0, rb0, ra1, rb1;
                    rope_rotate(E::lo(wa), E::lo(wb), u2f(cv[t][c0]), u2f(sv[t][c0]), ra0, rb0);
                    rope_rotate(E::hi(wa), E::hi(wb), u2f(cv[t][c0 + 1]), u2f(sv[t][c0 + 1]), ra1, rb1);
                    raw[s][e] = E::pack(ra0, ra1);
                    raw[s + KSTEPS / 2][e] = E::pack(rb0, rb1);
                }
        }
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(vec8, (raw[s] & qz) ^ qx);
    };
    if constexpr (ROPE == 0) finish_q();

    f32x16 oacc[DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    // per query (this lane's column): reference m (log2 domain) and the partial sum
    // of this half-wave's weights, in fp32
    float m_run = NEG_INF, le_run = 0.f;
    float neg_m = -0.f;     // -m_run, or 0 while m_run is -inf (the weights' offset)

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
        kvo[i] = (c < T::CPR && wave + NW * i < T::KDMA) ? (uint32_t)(row * T::ROW + 16 * c) : OOB_VOFFSET;
    }
#pragma unroll
    for (int i = 0; i < VDMA_W; ++i) {
        const int slot = 64 * (wave + NW * i) + lane;
        const int row = slot / T::VSLOTS, c = slot % T::VSLOTS;
        vvo[i] = (c < T::CPR && wave + NW * i < T::VDMA) ? (uint32_t)(row * T::ROW + 16 * c) : OOB_VOFFSET;
    }
    // a tile past the workgroup's last one is "loaded" from an offset past
    // num_records: the DMA then writes zeros and touches no memory, and the
    // instruction needs no branch around it
    auto tile_so = [&](int j) -> uint32_t {
        return (j < ntiles) ? (uint32_t)(j * BN16) * T::ROW : OOB_VOFFSET;
    };
    auto dma_k = [&](int j, uint8_t* __restrict__ dst) {
        const uint32_t so = tile_so(j);
#pragma unroll
        for (int i = 0; i < T::KDMA_W; ++i) {
            // a wave's surplus instruction writes zeros into the spare slot past the buffers
            uint8_t* d = (wave + NW * i < T::KDMA) ? dst + 1024 * (wave + NW * i) : smem + 2 * T::BUF;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void_t*)d, 16, kvo[i], so, 0, 0);
        }
    };
    auto dma_v = [&](int j, uint8_t* __restrict__ dst) {
        const uint32_t so = tile_so(j);
#pragma unroll
        for (int i = 0; i < T::VDMA_W; ++i) {
            uint8_t* d = (wave + NW * i < T::VDMA) ? dst + 1024 * (wave + NW * i) : smem + 2 * T::BUF;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)d, 16, vvo[i], so, 0, 0);
        }
    };

    // lane bases of the operand reads (bytes within one K or V tile)
    const int k_lane = n * T::KPITCH + 16 * h;
    const int tr_row = (lane & 15) >> 2;
    const int v_lane = (4 * h + tr_row) * T::VPITCH + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1);

    // K tiles live in kbuf(0/1), V tiles in vbuf(0/1); K runs one tile ahead of V
    auto kbuf = [&](int i) -> uint8_t* { return smem + i * T::BUF; };
    auto vbuf = [&](int i) -> uint8_t* { return smem + i * T::BUF + T::KBYTES; };

    // ---- S^T block kb (32 keys) of a tile: S^T = K . Q^T over the D/16 k-steps
    auto qk_blk = [&](const uint8_t* __restrict__ kt, int kb, f32x16& sacc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const vec8 a = *(const vec8*)(kt + k_lane + 32 * kb * T::KPITCH + 32 * s);
            sacc = E::mfma(a, qf[s], sacc);
        }
    };
    // ---- mask of block kb of tile j: causal diagonal and the ragged key tail
    auto mask_blk = [&](int j, int kb, f32x16& sacc) {
        const int k0 = j * BN16 + 32 * kb;
        const bool need_mask = (k0 + 32 > p.Sk) || (CAUSAL && (k0 + 31 > qw + off));
        if (need_mask) {
            const int qi = qw + n;
            const int lim = (CAUSAL ? min(p.Sk - 1, qi + off) : (p.Sk - 1)) - (k0 + 4 * h);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + (r & 3);    // relative to k0 + 4h
                if (key > lim) sacc[r] = NEG_INF;
            }
        }
    };
    // ---- the reference m_run is raised to the max of a 32-key block (and of itself)
    // only when needed: on a lane's first visible keys, and when the block's weights
    // sum past 2^RESCALE_LOG2 (which every weight above that bound implies); O and
    // the sum are rescaled with it.  Visible keys are a prefix of every row, so a
    // block with none is followed by blocks with none.
    auto raise_ref = [&](const f32x16& s) {
        float mp[4] = {s[0], s[1], s[2], s[3]};
#pragma unroll
        for (int r = 4; r < 16; ++r) mp[r & 3] = fmaxf(mp[r & 3], s[r]);
        float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
        mx = pair_max(mx) * p.c;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        neg_m = (m_new == NEG_INF) ? 0.f : -m_new;
        le_run *= alpha;
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
    };
    // ---- weights of one 32-key block, packed to 16 bits; returns their fp32 sum
    auto weights = [&](const f32x16& s, uint32_t (&pk)[8]) -> float {
        float se[4];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(fmaf(s[r], p.c, neg_m));
            const float p1 = fast_exp2(fmaf(s[r + 1], p.c, neg_m));
            if (r < 4) {
                se[r] = p0;
                se[r + 1] = p1;
            } else {
                se[r & 3] += p0;
                se[(r & 3) + 1] += p1;
            }
            pk[r >> 1] = E::pack(p0, p1);
        }
        return (se[0] + se[1]) + (se[2] + se[3]);
    };
    // ---- O^T += V^T . P^T for one 32-key block (two 16-key steps).  A operand from
    // the row-major V tile by two transposing reads: lane l receives
    // V[key0 + j][32db + (l % 32)], j = 0..3, key0 = 16t + 8rr + 4h, exactly the keys
    // that P^T holds in accumulator registers 8(t % 2) + 4rr + j.
    auto pv_blk = [&](const uint8_t* __restrict__ vt, const uint32_t (&pk)[8], int kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int t = 2 * kb + hf;
            u32x4 bw = {pk[4 * hf + 0], pk[4 * hf + 1], pk[4 * hf + 2], pk[4 * hf + 3]};
            const vec8 bfr = __builtin_bit_cast(vec8, bw);
#pragma unroll
            for (int d = 0; d < DBLK; ++d) {
                const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t*)(vt + v_lane + (16 * t) * T::VPITCH + 64 * d));
                const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t*)(vt + v_lane + (16 * t + 8) * T::VPITCH + 64 * d));
                const short8_t a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[d] = E::mfma(__builtin_bit_cast(vec8, a8), bfr, oacc[d]);
            }
        }
    };
    // ---- one software-pipelined step over key tile j.  On entry `s1` holds block 1
    // of S(j) and `pk0` the weights of block 0 of tile j; on exit `n1` holds block 1
    // of S(j+1) and `pk0` the weights of its block 0.
    //   phase 1: S(j+1) block 0, O += P(j) block 0 . V, weights of S(j) block 1
    //   phase 2: S(j+1) block 1, O += P(j) block 1 . V, weights of S(j+1) block 0
    // The DMA of K(j+2) into `kd` and V(j+1) into `vd` runs meanwhile; `kr_` holds
    // K(j+1) and `vr_` V(j).  The four buffers are distinct (__restrict__), so the
    // compiler reads the two while the DMA into the other two is in flight.
    auto step = [&](int j, f32x16& s1, uint32_t (&pk0)[8], f32x16& n0, f32x16& n1,
                    uint8_t* __restrict__ kd, uint8_t* __restrict__ vd,
                    const uint8_t* __restrict__ kr_, const uint8_t* __restrict__ vr_) {
        if (j * BN16 >= wkend) {                        // tile wholly above this wave's diagonal
            dma_k(j + 2, kd);
            dma_v(j + 1, vd);
            return;
        }
        const bool more = (j + 1) * BN16 < wkend;       // tile j+1 is visible to this wave
        uint32_t pk1[8];
        dma_k(j + 2, kd);
        qk_blk(kr_, 0, n0);
        pv_blk(vr_, pk0, 0);
        float ts = weights(s1, pk1);
        phase_schedule<KSTEPS, DBLK>();
        if (__any(ts > RESCALE_SUM)) {
            raise_ref(s1);
            ts = weights(s1, pk1);
        }
        le_run += ts;
        if (more) {
            mask_blk(j + 1, 0, n0);
            if (__any(m_run == NEG_INF)) raise_ref(n0);
        }
        dma_v(j + 1, vd);
        qk_blk(kr_, 1, n1);
        pv_blk(vr_, pk1, 1);
        float tn = weights(n0, pk0);
        phase_schedule<KSTEPS, DBLK>();
        if (more && __any(tn > RESCALE_SUM)) {
            raise_ref(n0);
            tn = weights(n0, pk0);
        }
        le_run += more ? tn : 0.f;
        if (more) mask_blk(j + 1, 1, n1);
    };

    f32x16 sa, sb, sn;
    uint32_t pk0[8];
    // prologue: K(0), V(0), K(1) in flight; scores of tile 0 and weights of its block 0
    dma_k(0, kbuf(0));
    dma_v(0, vbuf(0));
    dma_k(1, kbuf(1));
    if constexpr (ROPE != 0) finish_q();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA has landed
    __syncthreads();
    if (0 < wkend && ntiles > 0) {
        qk_blk(kbuf(0), 0, sn);
        qk_blk(kbuf(0), 1, sa);
        mask_blk(0, 0, sn);
        mask_blk(0, 1, sa);
        raise_ref(sn);
        le_run += weights(sn, pk0);
    }
    __syncthreads();                      // K(0) is consumed before K(2) replaces it

    int j = 0;
    for (; j + 1 < ntiles; j += 2) {
        step(j, sa, pk0, sn, sb, kbuf(0), vbuf(1), kbuf(1), vbuf(0));
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        step(j + 1, sb, pk0, sn, sa, kbuf(1), vbuf(0), kbuf(0), vbuf(1));
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }
    if (j < ntiles) step(j, sa, pk0, sn, sb, kbuf(0), vbuf(1), kbuf(1), vbuf(0));

    // ---- epilogue: O = O^T / le, rounded once; LSE = ln2 * (m + log2 le).  The
    // wave stages its 32 output rows in a private LDS tile (rows padded by 16 bytes)
    // and stores them row-contiguously, 16 bytes per lane, with the non-temporal
    // hint (the output is not read again by this launch, and the lines leave the
    // cache as they are written instead of all at the end of the launch).
    {
        const int qi = qw + n;
        const float le = pair_sum(le_run);
        const float inv = (le > 0.f) ? 1.f / le : 0.f;
        constexpr int SPITCH = T::ROW + 16;
        uint8_t* stg = smem + 2 * T::BUF + 1024 + wave * (QPW * SPITCH);
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = E::pack(oacc[d][4 * g + 0] * inv, oacc[d][4 * g + 1] * inv);
                w[1] = E::pack(oacc[d][4 * g + 2] * inv, oacc[d][4 * g + 3] * inv);
                *(u32x2*)(stg + n * SPITCH + 2 * (32 * d + 8 * g + 4 * h)) = w;
            }
        constexpr int LPR = T::ROW / 16;          // lanes per row
        constexpr int RPS = 64 / LPR;             // rows per store instruction
        if (qw + QPW <= p.Sq) {
            // every row of the wave exists: all staging reads first, then the stores
            u32x4 v[QPW / RPS];
#pragma unroll
            for (int i = 0; i < QPW / RPS; ++i)
                v[i] = *(const u32x4*)(stg + (RPS * i + lane / LPR) * SPITCH + 16 * (lane % LPR));
#pragma unroll
            for (int i = 0; i < QPW / RPS; ++i)
                __builtin_nontemporal_store(
                    v[i], (u32x4*)((uint8_t*)Og + (int64_t)(qw + RPS * i + lane / LPR) * T::ROW + 16 * (lane % LPR)));
        } else {
#pragma unroll
            for (int i = 0; i < QPW / RPS; ++i) {
                const int row = RPS * i + lane / LPR;
                const u32x4 v = *(const u32x4*)(stg + row * SPITCH + 16 * (lane % LPR));
                if (qw + row < p.Sq)
                    __builtin_nontemporal_store(v, (u32x4*)((uint8_t*)Og + (int64_t)(qw + row) * T::ROW + 16 * (lane % LPR)));
            }
        }
        if (p.lse && h == 0 && qi < p.Sq) {
            const float lse = (le > 0.f) ? (m_run + __log2f(le)) * 0.69314718055994531f : NEG_INF;
            p.lse[q_head + qi] = lse;
        }
    }
}

// ---------------------------------------------------------------------------
// kernel selection
// ---------------------------------------------------------------------------
template <int DT, int D, int ROPE>
static const void* pick16r(int causal) {
    return causal ? (const void*)&attn_fwd_16<DT, D, true, ROPE> : (const void*)&attn_fwd_16<DT, D, false, ROPE>;
}
template <int DT, int D>
static const void* pick16(int causal, int rope) {
    return rope == 0 ? pick16r<DT, D, 0>(causal) : rope == 1 ? pick16r<DT, D, 1>(causal)
         : rope == 2 ? pick16r<DT, D, 2>(causal) : nullptr;
}

KernelChoice select_kernel(int dtype, int D, int causal, int rope, int64_t heads, int Sq) {
    KernelChoice kc = {nullptr, 0, 0};
    if (dtype == ATTN_IMPL_FP32) {
        if (rope != 0) return kc;
        return select_kernel32(D, causal, heads, Sq);
    }
    kc.bm = BM16;
    kc.threads = 64 * NW;
    if (dtype == ATTN_IMPL_BF16)
        kc.fn = (D == 64) ? pick16<ATTN_IMPL_BF16, 64>(causal, rope)
              : (D == 128) ? pick16<ATTN_IMPL_BF16, 128>(causal, rope) : nullptr;
    else if (dtype == ATTN_IMPL_FP16)
        kc.fn = (D == 64) ? pick16<ATTN_IMPL_FP16, 64>(causal, rope)
              : (D == 128) ? pick16<ATTN_IMPL_FP16, 128>(causal, rope) : nullptr;
    return kc;
}

}  // namespace attn_impl
