// attn_fwd32_kernels.hip -- the fp32 attention forward kernels for gfx950 (MI355X).
//
// The operation is the one of attn_fwd_kernels.hip (the page "A Thread-Register
// Decoupled GPU Execution Model for Efficient Tensor Computation", introduction,
// Equ. 1) with true fp32 products: v_mfma_f32_32x32x2_f32, 32 queries per wave,
// 32-key tiles in LDS, the same online softmax with the reference raised per tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_internal.h"
#include "attn_kernel_common.h"
#include "attn_fwd_tile_map.h"

namespace attn_impl {

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
    const int kvh = tc.kvh;
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

    // K and V tiles go through registers: the next tile's 16-byte loads are issued
    // before the current tile is computed, so their latency overlaps the MFMAs
    constexpr int NPF = BN32 * D / 4 / 256;        // float4 per thread per tile and tensor
    // (rows past Sk, and the tile after the last, are clamped to row 0 and zeroed)
    float4 kpre[NPF], vpre[NPF];
#define ATTN32_LOAD_TILE(J)                                                               \
    _Pragma("unroll") for (int i = 0; i < NPF; ++i) {                                     \
        const int e = 4 * (tid + 256 * i);                                                \
        const int row = e / D, col = e % D;                                               \
        const bool ok = (J) < ntiles && (J) * BN32 + row < p.Sk;                          \
        const int64_t off32 = ok ? (int64_t)((J) * BN32 + row) * D + col : (int64_t)col;  \
        const float4 kx = *(const float4*)(Kg + off32);                                   \
        const float4 vx = *(const float4*)(Vg + off32);                                   \
        kpre[i] = ok ? kx : make_float4(0.f, 0.f, 0.f, 0.f);                              \
        vpre[i] = ok ? vx : make_float4(0.f, 0.f, 0.f, 0.f);                              \
    }
    ATTN32_LOAD_TILE(0)
    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BN32;
        __syncthreads();     // previous tile fully consumed
#pragma unroll
        for (int i = 0; i < NPF; ++i) {
            const int e = 4 * (tid + 256 * i);
            const int row = e / D, col = e % D;
            float* kd = ks + row * KP + col;
            float* vd = vs + row * KP + col;
            kd[0] = kpre[i].x; kd[1] = kpre[i].y; kd[2] = kpre[i].z; kd[3] = kpre[i].w;
            vd[0] = vpre[i].x; vd[1] = vpre[i].y; vd[2] = vpre[i].z; vd[3] = vpre[i].w;
        }
        __syncthreads();
        ATTN32_LOAD_TILE(j + 1)
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

#undef ATTN32_LOAD_TILE

// ---------------------------------------------------------------------------
// fp32 kernel for launches with few query tiles (fewer 128-query workgroups than
// CUs): a workgroup owns 32 queries and its 4 waves split the key tiles between
// them (wave w takes tiles w, w + 4, ...), each with its own online softmax over
// its keys, in its own LDS region (no workgroup barrier in the loop); the four
// partial results are then merged exactly, as the split-KV decode merges chunks:
// with M the largest reference, O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w.
// ---------------------------------------------------------------------------
constexpr int BM32S = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_32s(AttnParams p) {
    constexpr int KP = D + 1;       // row pitch (floats) of the K and V tiles
    constexpr int KSTEPS = D / 2;
    constexpr int DBLK = D / 32;
    constexpr int WREG = 2 * BN32 * KP;                 // floats per wave: its K and V tile
    constexpr int OP = D + 1;                           // row pitch of the merge area
    static_assert(4 * 32 * OP + 8 * 32 <= 4 * WREG, "merge area inside the tile regions");
    __shared__ float lds[4 * WREG];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int h = lane >> 5;

    const TileCoord tc = map_tile(p, blockIdx.x);
    const int kvh = tc.kvh;
    const int off = p.Sk - p.Sq;
    const int qw = tc.qt * BM32S;                       // the workgroup's (and every wave's) queries

    const float* __restrict__ Qg = (const float*)p.q + ((int64_t)(tc.b * p.Hq + tc.hq) * p.Sq) * D;
    const float* __restrict__ Kg = (const float*)p.k + ((int64_t)(tc.b * p.Hkv + kvh) * p.Sk) * D;
    const float* __restrict__ Vg = (const float*)p.v + ((int64_t)(tc.b * p.Hkv + kvh) * p.Sk) * D;
    float* __restrict__ Og = (float*)p.o + ((int64_t)(tc.b * p.Hq + tc.hq) * p.Sq) * D;

    const int last_q = min(qw + BM32S, p.Sq) - 1;
    int kend = p.Sk;
    if (CAUSAL) kend = min(p.Sk, last_q + off + 1);
    const int ntiles = kend > 0 ? (kend + BN32 - 1) / BN32 : 0;

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

    float* ks = lds + wave * WREG;
    float* vs = ks + BN32 * KP;
    constexpr int NPW = BN32 * D / 4 / 64;              // float4 per lane per tile and tensor
    for (int j = wave; j < ntiles; j += 4) {
        const int k0 = j * BN32;
        // the wave's own tile: rows past Sk read as zero
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int e = 4 * (lane + 64 * i);
            const int row = e / D, col = e % D;
            const bool ok = k0 + row < p.Sk;
            const int64_t o32 = ok ? (int64_t)(k0 + row) * D + col : (int64_t)col;
            const float4 kx = *(const float4*)(Kg + o32);
            const float4 vx = *(const float4*)(Vg + o32);
            const float4 kz = ok ? kx : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 vz = ok ? vx : make_float4(0.f, 0.f, 0.f, 0.f);
            float* kd = ks + row * KP + col;
            float* vd = vs + row * KP + col;
            kd[0] = kz.x; kd[1] = kz.y; kd[2] = kz.z; kd[3] = kz.w;
            vd[0] = vz.x; vd[1] = vz.y; vd[2] = vz.z; vd[3] = vz.w;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);             // lgkmcnt(0): the wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();

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
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
            for (int d = 0; d < DBLK; ++d)
                oacc[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * KP + 32 * d + n], sacc[r],
                                                                oacc[d], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();                // every lane has read the tile
    }

    // merge: each wave leaves its unnormalised O (32 queries x D), its reference and its
    // weight sum per query in the (now free) tile regions
    __syncthreads();
    float* mo = lds + wave * 32 * OP;                   // [query][d]
    float* ml = lds + 4 * 32 * OP;                      // [wave][query]: m, then l
    const float l_tot = pair_sum(l_run);
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) mo[n * OP + 32 * d + 8 * (r >> 2) + 4 * h + (r & 3)] = oacc[d][r];
    if (h == 0) {
        ml[wave * 32 + n] = m_run;
        ml[128 + wave * 32 + n] = l_tot;
    }
    __syncthreads();
    // thread t: query t / 8, features (t % 8) + 8 i
    {
        const int q = tid >> 3, c = tid & 7;
        float m[4], l[4];
        float M = NEG_INF;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            m[w] = ml[w * 32 + q];
            l[w] = ml[128 + w * 32 + q];
            M = fmaxf(M, m[w]);
        }
        float sc[4], L = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            sc[w] = (m[w] == NEG_INF) ? 0.f : fast_exp2(m[w] - M);
            L += sc[w] * l[w];
        }
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
        const int qi = qw + q;
        if (qi < p.Sq) {
            float* orow = Og + (int64_t)qi * D;
#pragma unroll
            for (int i = 0; i < D / 8; ++i) {
                const int d = c + 8 * i;
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) acc += sc[w] * lds[w * 32 * OP + q * OP + d];
                orow[d] = acc * inv;
            }
            if (p.lse && c == 0) {
                const float lse = (L > 0.f) ? (M + __log2f(L)) * 0.69314718055994531f : NEG_INF;
                p.lse[(int64_t)(tc.b * p.Hq + tc.hq) * p.Sq + qi] = lse;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// kernel selection (fp32)
// ---------------------------------------------------------------------------
template <int D>
static const void* pick32(int causal, int split) {
    if (split) return causal ? (const void*)&attn_fwd_32s<D, true> : (const void*)&attn_fwd_32s<D, false>;
    return causal ? (const void*)&attn_fwd_32<D, true> : (const void*)&attn_fwd_32<D, false>;
}

KernelChoice select_kernel32(int D, int causal, int64_t heads, int Sq) {
    // fewer 128-query tiles than CUs: 32-query workgroups whose waves split the keys
    const int split = (heads * ((Sq + BM32 - 1) / BM32) < 256) ? 1 : 0;
    KernelChoice kc;
    kc.bm = split ? BM32S : BM32;
    kc.threads = 256;
    kc.fn = (D == 64) ? pick32<64>(causal, split) : (D == 128) ? pick32<128>(causal, split) : nullptr;
    return kc;
}

}  // namespace attn_impl
