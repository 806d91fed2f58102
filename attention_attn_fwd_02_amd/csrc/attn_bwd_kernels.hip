// attn_bwd_kernels.hip -- gradients of the fused attention forward (gfx950).
//
// The page "A Thread-Register Decoupled GPU Execution Model for Efficient Tensor
// Computation" evaluates the FlashAttention backward as its training workload
// (evaluation set-up, "Workloads"; results, "Decoding and Training Workloads
// Speedup": more GEMMs than the forward, more live tensors, operand transposes and
// score recomputation).  With P_ij = exp(scale q_i.k_j - LSE_i) recomputed from the
// forward's LSE and D_i = dO_i . O_i:
//     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q
// Kernels (in stream order):
//   attn_bwd_pre   -D_i, LSE2_i = LSE_i log2(e) and -LSE2_i / ce per query row (into
//                  the workspace; ce = scale log2(e), or 2^-100 for a zero scale);
//   attn_bwd_main  the two passes below in one launch (the dQ workgroups fill the CUs
//                  the dK/dV pass's last workgroups leave idle):
//     dK/dV pass   one workgroup per (batch, K/V head, 128 keys, split), 4 waves x 32
//                  keys, two workgroups per CU (two waves per SIMD, which is why the
//                  S and dP accumulators start at -LSE2 / ce and -D instead of holding
//                  those per-query values in registers of their own): loops over its
//                  share of the query heads of the group and their 32-query tiles,
//                  accumulating dK^T and dV^T in registers (no atomics).  With one
//                  split the gradients are stored directly; a grouped-query shape with
//                  few K/V heads instead splits the query heads of a group over
//                  several workgroups (fp32 partial sums), so the pass fills the GPU;
//     dQ pass      one workgroup per (batch, query head, 128 queries), 4 waves x 32
//                  queries: loops over 32-key tiles, accumulating dQ^T;
//   attn_bwd_reduce (split shapes only) adds the partial sums in split order and
//                  stores dK, dV.
// Every product is a v_mfma_f32_32x32x16_{bf16,f16} in the layouts of the forward
// kernel: an operand whose contraction index runs along memory rows (Q, dO, K, V
// read as "rows x d") comes from LDS by ds_read_b128 out of rows padded by 16 bytes;
// one whose contraction index runs down a column (dO^T, Q^T, K^T) comes by
// ds_read_b64_tr_b16 out of rows padded by 64 bytes; the weights P and dS go from
// the accumulator registers straight into the next MFMA as packed 16-bit operands.
// Q, dO (dK/dV pass) and K (dQ pass) are therefore staged in both layouts.
// dQ is computed by its own pass rather than by atomic adds so that every gradient
// is deterministic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "attn_fwd_internal.h"
#include "attn_kernel_common.h"

namespace attn_impl {

// One 32-row tile of a [rows][D] tensor in both LDS layouts, each rounded up to
// whole 1 KB DMA instructions.
template <int D> struct BwdTile {
    static constexpr int ROW = 2 * D;
    static constexpr int CPR = D / 8;
    static constexpr int BPITCH = ROW + 16;     // ds_read_b128 layout (16-row reads conflict-free)
    static constexpr int TPITCH = ROW + 64;     // ds_read_b64_tr_b16 layout
    static constexpr int BSLOTS = BPITCH / 16;
    static constexpr int TSLOTS = TPITCH / 16;
    static constexpr int BDMA = (32 * BPITCH + 1023) / 1024;
    static constexpr int TDMA = (32 * TPITCH + 1023) / 1024;
    static constexpr int BREG = 1024 * BDMA;
    static constexpr int TREG = 1024 * TDMA;
};

constexpr int BWD_MAXDMA = 10;

// voffsets of a wave that DMAs one whole 32-row tile part in a layout of `slots`
// 16-byte slots per row: instruction i fills slots 64i + lane
template <int D>
__device__ __forceinline__ void part_offsets(int slots, int ndma, int lane, uint32_t (&vo)[BWD_MAXDMA]) {
    typedef BwdTile<D> T;
#pragma unroll
    for (int i = 0; i < BWD_MAXDMA; ++i) {
        const int slot = 64 * i + lane;
        const int row = slot / slots, c = slot % slots;
        vo[i] = (i < ndma && c < T::CPR && row < 32) ? (uint32_t)(row * T::ROW + 16 * c) : OOB_VOFFSET;
    }
}

__device__ __forceinline__ void dma_part(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, int ndma,
                                         const uint32_t (&vo)[BWD_MAXDMA], uint32_t so) {
#pragma unroll
    for (int i = 0; i < BWD_MAXDMA; ++i)
        if (i < ndma)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 1024 * i), 16, vo[i], so, 0, 0);
}

// Stage a wave's 32 x D fp32 result (lane = output row, registers = 4-runs of
// columns, the layout of an MFMA accumulator with rows on lanes) through its LDS
// region and store rows [row0, row0 + 32) below `nrows` as 16-bit values, with the
// non-temporal hint (gradients are not read again by the launch).
template <int DT, int D>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[D / 32], float mul, uint8_t* stg,
                                           uint8_t* out, int64_t row0, int nrows, int lane) {
    typedef Elem16<DT> E;
    constexpr int ROW = 2 * D;
    constexpr int SPITCH = ROW + 16;
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w;
            w[0] = E::pack(acc[d][4 * g + 0] * mul, acc[d][4 * g + 1] * mul);
            w[1] = E::pack(acc[d][4 * g + 2] * mul, acc[d][4 * g + 3] * mul);
            *(u32x2*)(stg + n * SPITCH + 2 * (32 * d + 8 * g + 4 * h)) = w;
        }
    constexpr int LPR = ROW / 16;
    constexpr int RPS = 64 / LPR;
#pragma unroll
    for (int i = 0; i < 32 / RPS; ++i) {
        const int row = RPS * i + lane / LPR;
        const u32x4 v = *(const u32x4*)(stg + row * SPITCH + 16 * (lane % LPR));
        if (row < nrows)
            __builtin_nontemporal_store(v, (u32x4*)(out + (row0 + row) * ROW + 16 * (lane % LPR)));
    }
}

// A wave's 32 x D fp32 result in the same accumulator layout, stored as fp32 rows
// [0, nrows) of `out` (row pitch D floats): lane n writes 16-byte runs of its row.
template <int D>
__device__ __forceinline__ void store_rows_f32(const f32x16 (&acc)[D / 32], float* out, int nrows, int lane) {
    const int n = lane & 31, h = lane >> 5;
    if (n >= nrows) return;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 v = {acc[d][4 * g + 0], acc[d][4 * g + 1], acc[d][4 * g + 2], acc[d][4 * g + 3]};
            *(float4*)(out + n * D + 32 * d + 8 * g + 4 * h) = v;
        }
}

// Two transposing reads give lane l the elements X[r0 + j][32 db + l % 32], j = 0..7,
// rows in the key order the 16-bit weights are packed in (see the forward kernel).
template <typename vec8, int TPITCH>
__device__ __forceinline__ vec8 tr_frag(const uint8_t* base, int v_lane, int hf, int db) {
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4_t*)(base + v_lane + (16 * hf) * TPITCH + 64 * db));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4_t*)(base + v_lane + (16 * hf + 8) * TPITCH + 64 * db));
    const short8_t a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(vec8, a8);
}

__device__ __forceinline__ int tr_lane_base(int lane, int tpitch) {
    const int h = lane >> 5, tr_row = (lane & 15) >> 2;
    return (4 * h + tr_row) * tpitch + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1);
}

// Workgroup w -> (group, block).  When the groups split evenly over the 8 XCDs
// (the dispatcher sends workgroup w to XCD w % 8), all blocks of a group run on one
// XCD, so the group's streamed operands (Q and dO, or K and V) stay in that XCD's
// L2.  With fewer groups than XCDs (a divisor of 8, e.g. the dQ pass of a shape with
// four K/V heads), each group gets 8 / ngrp XCDs of its own, its blocks dealt over
// them in turn, so that each XCD still streams a single group's operands.  Blocks
// of a group are dispatched in order of their index.
__device__ __forceinline__ void bwd_map(int w, int nblk, int ngrp, int& grp, int& blk) {
    const int xcd = w & 7, slot = w >> 3;
    if (ngrp % 8 == 0) {
        grp = 8 * (slot / nblk) + xcd;
        blk = slot % nblk;
    } else if (8 % ngrp == 0 && nblk % (8 / ngrp) == 0) {
        const int x = 8 / ngrp;                 // XCDs per group
        grp = xcd / x;
        blk = slot * x + xcd % x;
    } else {
        grp = w / nblk;
        blk = w % nblk;
    }
}

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i (stored negated), LSE2_i = LSE_i * log2(e) and -LSE2_i / ce, one
// row per D/8 lanes (16 bytes each).  With ce = 2^-100 (zero scale) the dK/dV pass's
// S + (-LSE2 / ce) rounds to -LSE2 / ce, whose product with ce is -LSE2 exactly.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void attn_bwd_pre(BwdParams p) {
    constexpr int LPR = D / 8;
    const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
    const int c = threadIdx.x % LPR;
    const bool ok = row < p.rows;
    float acc = 0.f;
    if (ok) {
        const u32x4 a = *(const u32x4*)((const uint8_t*)p.o + row * (2 * D) + 16 * c);
        const u32x4 b = *(const u32x4*)((const uint8_t*)p.dout + row * (2 * D) + 16 * c);
        if (DT == ATTN_IMPL_BF16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), acc);
                acc = fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(b[e] & 0xffff0000u), acc);
            }
        } else {
            const f16x8 ah = __builtin_bit_cast(f16x8, a), bh = __builtin_bit_cast(f16x8, b);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)ah[e], (float)bh[e], acc);
        }
    }
    // sum over the LPR lanes of the row (aligned groups of 8 or 16 lanes)
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (ok && c == 0) {
        const float l2 = p.lse[row] * 1.4426950408889634f;
        p.drow[row] = -acc;
        p.l2row[row] = l2;
        p.sinit[row] = -l2 / p.ce;
    }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int DT, int D> struct DkdvLds {
    typedef BwdTile<D> T;
    // one buffer: Q (b128 layout), Q (tr layout), dO (b128), dO (tr), -LSE2 / ce, -D
    static constexpr int BUF = 2 * (T::BREG + T::TREG) + 2048;
};

template <int DT, int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_body(const BwdParams& p, const int wid, uint8_t* buf0, uint8_t* buf1) {
    typedef Elem16<DT> E;
    typedef typename E::vec8 vec8;
    typedef BwdTile<D> T;
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    // one buffer: Q (b128 layout), Q (tr layout), dO (b128), dO (tr), -LSE2 / ce, -D
    constexpr int OFF_QB = 0, OFF_QT = T::BREG, OFF_OB = T::BREG + T::TREG;
    constexpr int OFF_OT = 2 * T::BREG + T::TREG, OFF_L = 2 * (T::BREG + T::TREG);
    constexpr int OFF_D = OFF_L + 1024, BUF = OFF_D + 1024;
    static_assert(BUF == DkdvLds<DT, D>::BUF, "dK/dV buffer layout");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31, h = lane >> 5;
    const int nkb = (p.Sk + 127) / 128;
    int kb, sg;                                  // sg = (b * Hkv + g) * nsplit + split
    bwd_map(wid, nkb, p.B * p.Hkv * p.nsplit, sg, kb);
    const int grp = sg / p.nsplit, split = sg % p.nsplit;
    const int b = grp / p.Hkv, g = grp % p.Hkv;
    const int R = p.Hq / p.Hkv;
    const int RS = R / p.nsplit;                 // query heads of this split: split*RS ..
    const int off = p.Sk - p.Sq;
    const int k0w = kb * 128 + 32 * wave;        // first key of this wave
    const int64_t kv_row0 = (int64_t)grp * p.Sk;

    // this wave's K and V rows as MFMA B operands (rows past Sk read as zero)
    vec8 kf[KSTEPS], vf[KSTEPS];
    {
        const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint8_t*)p.k + kv_row0 * T::ROW, (uint32_t)p.Sk * T::ROW);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint8_t*)p.v + kv_row0 * T::ROW, (uint32_t)p.Sk * T::ROW);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const uint32_t vo = (uint32_t)(k0w + n) * T::ROW + (16 * s + 8 * h) * 2;
            kf[s] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(kr, vo, 0, 0));
            vf[s] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(vr, vo, 0, 0));
        }
    }

    // query tiles: the RS heads of the split, each from the first tile whose last
    // query sees this workgroup's first key
    const int nqt = (p.Sq + 31) / 32;
    int qt0 = 0;
    if (CAUSAL) qt0 = max(0, kb * 128 - off) / 32;
    const int per_head = max(0, nqt - qt0);
    const int ntiles = RS * per_head;
    // Causal: the first nd query tiles of each head can cross the diagonal of some
    // wave's keys (the workgroup's last key is kb*128 + 127); they are walked first,
    // for all heads of the split, with the masked tile code, and the rest without
    // any per-element compares.  Tile t -> (head, query tile).
    int nd = 0;
    if (CAUSAL) {
        const int x = kb * 128 + 127 - off;
        nd = x > 0 ? min(per_head, max(0, (x + 31) / 32 - qt0)) : 0;
    }
    const int nfull = per_head - nd;
    const int ndiag = RS * nd;
    auto tile_at = [&](int t, int& r, int& qt) {
        if (t < ndiag) {
            r = t / nd;
            qt = qt0 + t % nd;
        } else {
            const int u = t - ndiag;
            r = u / nfull;
            qt = qt0 + nd + u % nfull;
        }
    };

    // DMA: wave 0 stages Q (b128), 1 Q (tr), 2 dO (b128), 3 dO (tr) plus -LSE2 / ce and -D
    uint32_t vo[BWD_MAXDMA];
    const int slots = (wave & 1) ? T::TSLOTS : T::BSLOTS;
    const int ndma = (wave & 1) ? T::TDMA : T::BDMA;
    part_offsets<D>(slots, ndma, lane, vo);
    const int part_off = wave == 0 ? OFF_QB : wave == 1 ? OFF_QT : wave == 2 ? OFF_OB : OFF_OT;
    const uint32_t lvo = lane < 8 ? 16u * lane : OOB_VOFFSET;
    auto dma_tile = [&](int t, uint8_t* dst) {
        const bool live = t < ntiles;
        int rr = 0, qt = 0;
        if (live) tile_at(t, rr, qt);
        const int r = split * RS + rr;
        const int q0 = qt * 32;
        const int64_t head_row0 = ((int64_t)b * p.Hq + (int64_t)g * R + r) * p.Sq;
        const void* src = (wave < 2) ? p.q : p.dout;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((const uint8_t*)src + head_row0 * T::ROW, (uint32_t)p.Sq * T::ROW);
        dma_part(rs, dst + part_off, ndma, vo, live ? (uint32_t)q0 * T::ROW : OOB_VOFFSET);
        if (wave == 3) {
            const __amdgpu_buffer_rsrc_t lr = make_rsrc(p.sinit + head_row0, (uint32_t)p.Sq * 4);
            const __amdgpu_buffer_rsrc_t dr = make_rsrc(p.drow + head_row0, (uint32_t)p.Sq * 4);
            const uint32_t so = live ? (uint32_t)q0 * 4 : OOB_VOFFSET;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lr, (lds_void_t*)(dst + OFF_L), 16, lvo, so, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void_t*)(dst + OFF_D), 16, lvo, so, 0, 0);
        }
    };

    f32x16 dvt[DBLK], dkt[DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dvt[d][r] = 0.f; dkt[d][r] = 0.f; }

    const int b_lane = n * T::BPITCH + 16 * h;
    const int t_lane = tr_lane_base(lane, T::TPITCH);

    // one query tile; `masked`: the causal mask is applied (the tiles that may cross
    // a wave's diagonal; keys past Sk need none: their K, V rows read as zero and
    // their dK, dV rows are not stored)
    auto tile = [&](int t, const uint8_t* cur, auto masked) __attribute__((always_inline)) {
        constexpr bool MASKED = CAUSAL && decltype(masked)::value;
        int rr, qt;
        tile_at(t, rr, qt);
        const int q0 = qt * 32;
        // nothing to do when every key of the wave is past Sk or past the diagonal
        // of the tile's last query
        if (k0w >= p.Sk || (CAUSAL && k0w > q0 + 31 + off)) return;
        // S = Q K^T - LSE2 / ce (queries x keys): lane = key column, registers =
        // queries 8(r/4) + 4h + r%4 of the tile; the accumulator starts at the
        // per-query offset, so that P = exp2(ce S) needs no other per-query value
        f32x16 s;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const float4 lv = *(const float4*)(cur + OFF_L + 4 * (8 * gq + 4 * h));
            s[4 * gq + 0] = lv.x; s[4 * gq + 1] = lv.y; s[4 * gq + 2] = lv.z; s[4 * gq + 3] = lv.w;
        }
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
            s = E::mfma(*(const vec8*)(cur + OFF_QB + b_lane + 32 * st), kf[st], s);
        // dP - D = dO V^T - D, the accumulator starting at -D; issued before the
        // softmax so that the matrix core works on it while the weights are computed
        f32x16 dp;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const float4 dv4 = *(const float4*)(cur + OFF_D + 4 * (8 * gq + 4 * h));
            dp[4 * gq + 0] = dv4.x; dp[4 * gq + 1] = dv4.y; dp[4 * gq + 2] = dv4.z; dp[4 * gq + 3] = dv4.w;
        }
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
            dp = E::mfma(*(const vec8*)(cur + OFF_OB + b_lane + 32 * st), vf[st], dp);
        const int key = k0w + n;
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qi = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool vis = !MASKED || key <= qi + off;
            pr[r] = vis ? fast_exp2(s[r] * p.ce) : 0.f;
        }
        // dV^T += dO^T P
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            u32x4 bw;
#pragma unroll
            for (int e = 0; e < 4; ++e) bw[e] = E::pack(pr[8 * hf + 2 * e], pr[8 * hf + 2 * e + 1]);
            const vec8 bfr = __builtin_bit_cast(vec8, bw);
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
                dvt[db] = E::mfma(tr_frag<vec8, T::TPITCH>(cur + OFF_OT, t_lane, hf, db), bfr, dvt[db]);
        }
        // dS = P o (dP - D); dK^T += Q^T dS  (the scale is applied at the end)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            u32x4 bw;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r0 = 8 * hf + 2 * e;
                bw[e] = E::pack(pr[r0] * dp[r0], pr[r0 + 1] * dp[r0 + 1]);
            }
            const vec8 bfr = __builtin_bit_cast(vec8, bw);
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
                dkt[db] = E::mfma(tr_frag<vec8, T::TPITCH>(cur + OFF_QT, t_lane, hf, db), bfr, dkt[db]);
        }
    };

    dma_tile(0, buf0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    // masked pairs of tiles up to an even count covering the diagonal ones, then
    // unmasked pairs; an odd last tile takes the masked code (right for any tile)
    const std::true_type MASK;
    const std::false_type NOMASK;
    const int nmask = min((ndiag + 1) & ~1, ntiles & ~1);
    int t = 0;
    for (; t < nmask; t += 2) {
        dma_tile(t + 1, buf1);
        tile(t, buf0, MASK);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        dma_tile(t + 2, buf0);
        tile(t + 1, buf1, MASK);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }
    for (; t + 1 < ntiles; t += 2) {
        dma_tile(t + 1, buf1);
        tile(t, buf0, NOMASK);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        dma_tile(t + 2, buf0);
        tile(t + 1, buf1, NOMASK);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }
    if (t < ntiles) {
        tile(t, buf0, MASK);
        __syncthreads();
    }

    // dK = scale (dK^T)^T, dV = (dV^T)^T, rows k0w .. k0w + 31 below Sk
    const int nrows = min(32, p.Sk - k0w);
    if (nrows <= 0) return;
    if (p.nsplit == 1) {
        uint8_t* stg = buf1 + wave * (32 * (T::ROW + 16));
        static_assert(4 * 32 * (T::ROW + 16) <= BUF, "staging fits");
        store_rows<DT, D>(dvt, 1.f, stg, (uint8_t*)p.dv, kv_row0 + k0w, nrows, lane);
        store_rows<DT, D>(dkt, p.scale, stg, (uint8_t*)p.dk, kv_row0 + k0w, nrows, lane);
    } else {
        // this split's fp32 partial sums (dK unscaled); every row below Sk is written
        // by every split, zeros where the split's queries see none of the keys
        float* pk = p.part + (int64_t)(2 * split) * p.kvelems + (kv_row0 + k0w) * D;
        store_rows_f32<D>(dkt, pk, nrows, lane);
        store_rows_f32<D>(dvt, pk + p.kvelems, nrows, lane);
    }
}

// dK = scale * (sum of the splits' partial dK), dV = sum of the partial dV, the
// splits added in index order; eight elements of each per thread.
template <int DT>
__global__ __launch_bounds__(256) void attn_bwd_reduce(BwdParams p) {
    typedef Elem16<DT> E;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= p.kvelems) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = 0.f;
        for (int sp = 0; sp < p.nsplit; ++sp) {
            const float4* src = (const float4*)(p.part + (int64_t)(2 * sp + t) * p.kvelems + i);
            const float4 x = src[0], y = src[1];
            a[0] += x.x; a[1] += x.y; a[2] += x.z; a[3] += x.w;
            a[4] += y.x; a[5] += y.y; a[6] += y.z; a[7] += y.w;
        }
        const float mul = t == 0 ? p.scale : 1.f;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = E::pack(a[2 * e] * mul, a[2 * e + 1] * mul);
        __builtin_nontemporal_store(w, (u32x4*)((uint8_t*)(t == 0 ? p.dk : p.dv) + 2 * i));
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int DT, int D, bool CAUSAL>
__device__ __forceinline__ void dq_body(const BwdParams& p, const int wid, uint8_t* buf0, uint8_t* buf1) {
    typedef Elem16<DT> E;
    typedef typename E::vec8 vec8;
    typedef BwdTile<D> T;
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    // one buffer: K (b128 layout), K (tr layout), V (b128 layout)
    constexpr int OFF_KB = 0, OFF_KT = T::BREG, OFF_VB = T::BREG + T::TREG;
    constexpr int BUF = 2 * T::BREG + T::TREG;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31, h = lane >> 5;
    const int nqb = (p.Sq + 127) / 128;
    // the query heads of one K/V head form a group, whose blocks are (query block,
    // head) with the last query blocks (the heaviest under the causal mask) first
    const int R = p.Hq / p.Hkv;
    int grp, sb;                                 // grp = b * Hkv + g
    bwd_map(wid, R * nqb, p.B * p.Hkv, grp, sb);
    const int qb = CAUSAL ? nqb - 1 - sb / R : sb / R;
    const int b = grp / p.Hkv;
    const int hq = (grp % p.Hkv) * R + sb % R;
    const int bh = b * p.Hq + hq;
    const int off = p.Sk - p.Sq;
    const int qw = qb * 128 + 32 * wave;         // first query of this wave
    const int64_t q_row0 = (int64_t)bh * p.Sq;
    const int64_t kv_row0 = (int64_t)grp * p.Sk;

    // this wave's Q and dO rows as MFMA B operands; its query's LSE2 and -D
    vec8 qf[KSTEPS], of[KSTEPS];
    {
        const __amdgpu_buffer_rsrc_t qr = make_rsrc((const uint8_t*)p.q + q_row0 * T::ROW, (uint32_t)p.Sq * T::ROW);
        const __amdgpu_buffer_rsrc_t orr = make_rsrc((const uint8_t*)p.dout + q_row0 * T::ROW, (uint32_t)p.Sq * T::ROW);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const uint32_t vo = (uint32_t)(qw + n) * T::ROW + (16 * s + 8 * h) * 2;
            qf[s] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(qr, vo, 0, 0));
            of[s] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(orr, vo, 0, 0));
        }
    }
    const int qi = qw + n;
    float l2n = 0.f, ddn = 0.f;
    if (qi < p.Sq) {
        l2n = p.l2row[q_row0 + qi];
        ddn = p.drow[q_row0 + qi];            // -D_i
    }

    // key tiles of 32: all of them, or (causal) up to the workgroup's last query's diagonal
    int kend = p.Sk;
    if (CAUSAL) kend = min(p.Sk, min(qb * 128 + 128, p.Sq) - 1 + off + 1);
    const int ntiles = kend > 0 ? (kend + 31) / 32 : 0;
    int wkend = (qw < p.Sq) ? p.Sk : 0;          // keys this wave needs
    if (CAUSAL && qw < p.Sq) wkend = min(p.Sk, min(qw + 32, p.Sq) - 1 + off + 1);

    // DMA: wave 0 stages K (b128), wave 1 K (tr), wave 2 V (b128); wave 3 none
    uint32_t vo[BWD_MAXDMA];
    const int slots = wave == 1 ? T::TSLOTS : T::BSLOTS;
    const int ndma = wave == 3 ? 0 : wave == 1 ? T::TDMA : T::BDMA;
    part_offsets<D>(slots, ndma, lane, vo);
    const int part_off = wave == 0 ? OFF_KB : wave == 1 ? OFF_KT : OFF_VB;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc((const uint8_t*)(wave == 2 ? p.v : p.k) + kv_row0 * T::ROW,
                                                (uint32_t)p.Sk * T::ROW);
    auto dma_tile = [&](int t, uint8_t* dst) {
        dma_part(rs, dst + part_off, ndma, vo, t < ntiles ? (uint32_t)(32 * t) * T::ROW : OOB_VOFFSET);
    };

    f32x16 dqt[DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[d][r] = 0.f;
    const int b_lane = n * T::BPITCH + 16 * h;
    const int t_lane = tr_lane_base(lane, T::TPITCH);

    auto tile = [&](int t, const uint8_t* cur) {
        const int kk0 = 32 * t;
        if (kk0 >= wkend) return;
        // S^T = K Q^T (keys x queries): lane = query column, registers = keys
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
            s = E::mfma(*(const vec8*)(cur + OFF_KB + b_lane + 32 * st), qf[st], s);
        // dP^T = V dO^T
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
            dp = E::mfma(*(const vec8*)(cur + OFF_VB + b_lane + 32 * st), of[st], dp);
        // the mask only on tiles that cross the diagonal or the end of the keys
        float ds[16];
        if (kk0 + 32 > p.Sk || (CAUSAL && kk0 + 31 > qw + off)) {
            const int lim = (CAUSAL ? min(p.Sk - 1, qi + off) : p.Sk - 1) - (kk0 + 4 * h);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + (r & 3);          // relative to kk0 + 4h
                const float pr = key <= lim ? fast_exp2(fmaf(s[r], p.c, -l2n)) : 0.f;
                ds[r] = pr * (dp[r] + ddn);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(fmaf(s[r], p.c, -l2n)) * (dp[r] + ddn);
        }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            u32x4 bw;
#pragma unroll
            for (int e = 0; e < 4; ++e) bw[e] = E::pack(ds[8 * hf + 2 * e], ds[8 * hf + 2 * e + 1]);
            const vec8 bfr = __builtin_bit_cast(vec8, bw);
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
                dqt[db] = E::mfma(tr_frag<vec8, T::TPITCH>(cur + OFF_KT, t_lane, hf, db), bfr, dqt[db]);
        }
    };

    dma_tile(0, buf0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        dma_tile(t + 1, buf1);
        tile(t, buf0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        dma_tile(t + 2, buf0);
        tile(t + 1, buf1);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }
    if (t < ntiles) {
        tile(t, buf0);
        __syncthreads();
    }

    // two waves' output rows per buffer
    uint8_t* stg = (wave < 2 ? buf0 : buf1) + (wave & 1) * (32 * (T::ROW + 16));
    static_assert(2 * 32 * (T::ROW + 16) <= BUF, "staging fits");
    const int nrows = min(32, p.Sq - qw);
    if (nrows > 0) store_rows<DT, D>(dqt, p.scale, stg, (uint8_t*)p.dq, q_row0 + qw, nrows, lane);
}

// ---------------------------------------------------------------------------
// The dK/dV and dQ passes in one launch: workgroups [0, n_kv) run the dK/dV pass,
// [q_start, q_start + the dQ count) the dQ pass (q_start = n_kv rounded up to a
// multiple of 8, so that both keep their XCD mapping; the workgroups between exit).
// The dispatcher hands out workgroups in order, so dQ workgroups fill the CUs that
// the last dK/dV workgroups leave idle.  Both passes share the two LDS buffers.  At
// D = 64 the buffers take 48 KiB and the passes fit 168 registers: three workgroups
// (three waves per SIMD) per CU; at D = 128, 80 KiB and 256 registers: two.
// ---------------------------------------------------------------------------
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2)))
void attn_bwd_main(BwdParams p) {
    constexpr int BUF = DkdvLds<DT, D>::BUF;
    static_assert(2 * BwdTile<D>::BREG + BwdTile<D>::TREG <= BUF, "dQ buffers fit");
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[BUF];
    const int w = blockIdx.x;
    if (w < p.n_kv) dkdv_body<DT, D, CAUSAL>(p, w, buf0, buf1);
    else if (w >= p.q_start) dq_body<DT, D, CAUSAL>(p, w - p.q_start, buf0, buf1);
}

template <int DT, int D> static BwdKernels pick_bwd(int causal) {
    BwdKernels k;
    k.pre = (const void*)attn_bwd_pre<DT, D>;
    k.main = causal ? (const void*)attn_bwd_main<DT, D, true> : (const void*)attn_bwd_main<DT, D, false>;
    k.reduce = (const void*)attn_bwd_reduce<DT>;
    return k;
}

BwdKernels select_bwd(int dtype, int D, int causal) {
    if (dtype == ATTN_IMPL_BF16) {
        if (D == 64) return pick_bwd<ATTN_IMPL_BF16, 64>(causal);
        if (D == 128) return pick_bwd<ATTN_IMPL_BF16, 128>(causal);
    } else if (dtype == ATTN_IMPL_FP16) {
        if (D == 64) return pick_bwd<ATTN_IMPL_FP16, 64>(causal);
        if (D == 128) return pick_bwd<ATTN_IMPL_FP16, 128>(causal);
    }
    BwdKernels none = {nullptr, nullptr, nullptr};
    return none;
}

}  // namespace attn_impl
