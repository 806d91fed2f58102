// attn_decode_kernels.hip -- split-KV attention for few query rows (decoding), gfx950.
//
// The page "A Thread-Register Decoupled GPU Execution Model for Efficient Tensor
// Computation" evaluates decoding with FlashDecoding (evaluation set-up,
// "Workloads", with L_context = 4096 and d_head = 128) and notes in its results
// ("Decoding and Training Workloads Speedup") that this workload is dominated by
// matrix-vector products and the softmax and is bound by memory, with distinct
// KV caches per sequence in the multi-batch setting.  The operation is the same
// attention as the prefill kernel's; what changes is where the parallelism comes
// from: a query row sees thousands of keys, so the keys of every (batch, K/V head)
// are cut into chunks that independent waves stream concurrently, each producing
// a partial result normalised over its own chunk plus its log-sum-exp; a second
// kernel merges the partials exactly:
//
//     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) * O_s
//
// Split kernel: one 64-lane wave per (batch, K/V head, chunk).  The query rows of
// the K/V head's group (Hq/Hkv heads x Sq rows, at most 32) are the 32 columns of
// one MFMA block, so every K/V byte streamed from HBM serves all of them.  Chunks
// are walked in 32-key tiles that go HBM -> LDS by buffer_load ... lds into a
// wave-private double buffer (rows padded as in the prefill kernel, so both MFMA
// operand reads are conflict-free); scores S^T = K.Q^T and O^T += V^T.P^T use
// v_mfma_f32_32x32x16_{bf16,f16} with the prefill kernel's register layouts, and
// the softmax uses its lazily raised reference.  The path is bound by HBM bytes:
// the MFMAs and the softmax of a tile take a fraction of the time its 16 KB take
// to arrive, so the wave keeps two tiles in flight and four waves share a CU.  Each
// K/V byte is read exactly once, so the tile DMA carries the non-temporal hint (the
// lines stream through the caches instead of displacing reusable data; 13-16% more
// bandwidth than default-policy loads).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "attn_fwd_internal.h"
#include "attn_kernel_common.h"

// Scratch of the allocation-free decode entry point: the chunks' partial results
// (O and LSE per chunk and query row) of one call.  Every GPU the library runs on
// holds its own copy until the process ends; calls on one GPU share it.
static __device__ __align__(256) uint8_t scratch[attn_impl::DECODE_SCRATCH_BYTES];

namespace attn_impl {

constexpr int DKT = 32;                  // keys per decode tile
constexpr float DEC_RESCALE_SUM = 256.0f;

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (vmcnt in bits 3:0 and 15:14) and leaves the other counters alone
template <int N> constexpr int vmcnt_at_most() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}
constexpr int LGKM_ZERO = 0xC07F;        // lgkmcnt(0), vmcnt and expcnt unconstrained

template <int D> struct DecTile {
    static constexpr int ROW = 2 * D;                  // bytes of one K/V row
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int KPITCH = ROW + 16;            // see the prefill kernel's tiles
    static constexpr int VPITCH = ROW + 64;
    static constexpr int KSLOTS = KPITCH / 16;
    static constexpr int VSLOTS = VPITCH / 16;
    static constexpr int KDMA = (DKT * KPITCH + 1023) / 1024;   // 1 KB DMA instructions
    static constexpr int VDMA = (DKT * VPITCH + 1023) / 1024;
    static constexpr int KREG = 1024 * KDMA;
    static constexpr int BUF = KREG + 1024 * VDMA;              // one K tile, then one V tile
};

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(64) void attn_decode_split(DecodeParams p) {
    typedef Elem16<DT> E;
    typedef typename E::vec8 vec8;
    typedef DecTile<D> T;
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    static_assert(T::KDMA <= 16 && T::VDMA <= 16, "DMA offsets per wave");

    // two separate arrays, not one: reads of one buffer provably never alias the
    // DMA still landing in the other, so the compiler waits only where told to
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[T::BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[T::BUF];

    const int lane = threadIdx.x;
    const int n = lane & 31;            // query row of the group (S^T / O^T column)
    const int h = lane >> 5;
    const int split = blockIdx.x % p.nsplit;
    const int grp = blockIdx.x / p.nsplit;   // b * Hkv + g
    const int b = grp / p.Hkv;
    const int g = grp % p.Hkv;
    const int R = p.Hq / p.Hkv;
    const int nrows = R * p.Sq;         // <= 32, checked on the host
    const int off = p.Sk - p.Sq;

    // the group's query rows are contiguous: heads g*R .. g*R+R-1, Sq rows each
    const int64_t row0 = ((int64_t)b * p.Hq + (int64_t)g * R) * p.Sq;
    const uint8_t* Qg = (const uint8_t*)p.q + row0 * T::ROW;
    const int64_t kv_head = (int64_t)grp * p.Sk;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(Qg, (uint32_t)(nrows * T::ROW));
    const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint8_t*)p.k + kv_head * T::ROW, (uint32_t)p.Sk * T::ROW);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint8_t*)p.v + kv_head * T::ROW, (uint32_t)p.Sk * T::ROW);

    const int k0 = split * p.chunk;
    const int k1 = min(p.Sk, k0 + p.chunk);
    const int ntiles = k1 > k0 ? (k1 - k0 + DKT - 1) / DKT : 0;

    // Q^T fragments (B operand); rows past the group's read as zero
    vec8 qf[KSTEPS];
    {
        const uint32_t qx = (p.q_mode == 1) ? 0x80008000u : 0u;
        const uint32_t qz = (p.q_mode == 2) ? 0u : 0xffffffffu;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const uint32_t vo = (uint32_t)n * T::ROW + (16 * s + 8 * h) * 2;
            u32x4 raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, vo, 0, 0));
            raw = (raw & qz) ^ qx;
            qf[s] = __builtin_bit_cast(vec8, raw);
        }
    }

    // DMA lane offsets: instruction i fills LDS slots 64i + lane of the padded tile
    uint32_t kvo[16], vvo[16];
#pragma unroll
    for (int i = 0; i < T::KDMA; ++i) {
        const int slot = 64 * i + lane;
        const int row = slot / T::KSLOTS, c = slot % T::KSLOTS;
        kvo[i] = (c < T::CPR && row < DKT) ? (uint32_t)(row * T::ROW + 16 * c) : OOB_VOFFSET;
    }
#pragma unroll
    for (int i = 0; i < T::VDMA; ++i) {
        const int slot = 64 * i + lane;
        const int row = slot / T::VSLOTS, c = slot % T::VSLOTS;
        vvo[i] = (c < T::CPR && row < DKT) ? (uint32_t)(row * T::ROW + 16 * c) : OOB_VOFFSET;
    }
    // tile t of the chunk into `dst`; a tile past the chunk reads from an offset
    // past num_records (zeros, no memory traffic), so every call issues the same
    // number of instructions
    auto dma = [&](int t, uint8_t* dst) {
        const uint32_t so = (t < ntiles) ? (uint32_t)(k0 + DKT * t) * T::ROW : OOB_VOFFSET;
#pragma unroll
        for (int i = 0; i < T::KDMA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void_t*)(dst + 1024 * i), 16, kvo[i], so, 0, CPOL_NT);
#pragma unroll
        for (int i = 0; i < T::VDMA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)(dst + T::KREG + 1024 * i), 16, vvo[i], so, 0, CPOL_NT);
    };

    const int k_lane = n * T::KPITCH + 16 * h;
    const int tr_row = (lane & 15) >> 2;
    const int v_lane = T::KREG + (4 * h + tr_row) * T::VPITCH
                     + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1);

    f32x16 oacc[DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    float m_run = NEG_INF, le_run = 0.f;
    const int qi = n % p.Sq;            // query index of this lane's row within its head

    auto raise_ref = [&](const f32x16& s) {
        float mp[4] = {s[0], s[1], s[2], s[3]};
#pragma unroll
        for (int r = 4; r < 16; ++r) mp[r & 3] = fmaxf(mp[r & 3], s[r]);
        float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
        mx = pair_max(mx) * p.c;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        le_run *= alpha;
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
    };
    auto weights = [&](const f32x16& s, uint32_t (&pk)[8]) -> float {
        const float m_use = (m_run == NEG_INF) ? 0.f : m_run;
        float se[4];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(fmaf(s[r], p.c, -m_use));
            const float p1 = fast_exp2(fmaf(s[r + 1], p.c, -m_use));
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

    // one tile: scores, softmax and P.V from the buffer `cur`
    auto tile = [&](int t, const uint8_t* cur) {
        // tile t has landed once no more than one tile's DMA is outstanding
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most<T::KDMA + T::VDMA>());

        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const vec8 a = *(const vec8*)(cur + k_lane + 32 * s);
            sacc = E::mfma(a, qf[s], sacc);
        }
        // keys past the chunk or Sk, and (causal) past the row's diagonal
        const int kt = k0 + DKT * t;
        const bool need_mask = (kt + DKT > k1) || (CAUSAL && kt + DKT - 1 > off);
        if (need_mask) {
            const int lim = (CAUSAL ? min(k1 - 1, qi + off) : (k1 - 1)) - (kt + 4 * h);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + (r & 3);
                if (key > lim) sacc[r] = NEG_INF;
            }
        }
        if (__any(m_run == NEG_INF)) raise_ref(sacc);
        uint32_t pk[8];
        float ts = weights(sacc, pk);
        if (__any(ts > DEC_RESCALE_SUM)) {
            raise_ref(sacc);
            ts = weights(sacc, pk);
        }
        le_run += ts;
        // O^T += V^T . P^T over the tile's two 16-key steps
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            u32x4 bw = {pk[4 * hf + 0], pk[4 * hf + 1], pk[4 * hf + 2], pk[4 * hf + 3]};
            const vec8 bfr = __builtin_bit_cast(vec8, bw);
#pragma unroll
            for (int d = 0; d < DBLK; ++d) {
                const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t*)(cur + v_lane + (16 * hf) * T::VPITCH + 64 * d));
                const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t*)(cur + v_lane + (16 * hf + 8) * T::VPITCH + 64 * d));
                const short8_t a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[d] = E::mfma(__builtin_bit_cast(vec8, a8), bfr, oacc[d]);
            }
        }
        // every read of `cur` has returned before the DMA of tile t+2 overwrites it
        __builtin_amdgcn_s_waitcnt(LGKM_ZERO);
    };

    dma(0, buf0);
    dma(1, buf1);
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        tile(t, buf0);
        dma(t + 2, buf0);
        tile(t + 1, buf1);
        dma(t + 3, buf1);
    }
    if (t < ntiles) tile(t, buf0);
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most<0>());   // no DMA outlives the wave

    // partial result of this chunk: O normalised over the chunk, fp32; its LSE.
    // (Lanes n and n + 32 hold the same row, so the pair reduction inside the
    // branch always finds both halves active.)
    if (n < nrows) {
        const float le = pair_sum(le_run);
        const float inv = (le > 0.f) ? 1.f / le : 0.f;
        const int64_t rows = (int64_t)p.B * p.Hq * p.Sq;
        const int64_t row = row0 + n;
        float* orow = p.opart + ((int64_t)split * rows + row) * D;
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 w = {oacc[d][4 * g4 + 0] * inv, oacc[d][4 * g4 + 1] * inv,
                                  oacc[d][4 * g4 + 2] * inv, oacc[d][4 * g4 + 3] * inv};
                *(float4*)(orow + 32 * d + 8 * g4 + 4 * h) = w;
            }
        if (h == 0)
            p.lpart[(int64_t)split * rows + row] = (le > 0.f) ? (m_run + __log2f(le)) * 0.69314718055994531f : NEG_INF;
    }
}

// Merge: one workgroup of D threads per query row; thread d combines element d of
// every partial in a fixed order (deterministic).
template <int DT, int D>
__global__ __launch_bounds__(128) void attn_decode_merge(MergeParams p) {
    const int64_t row = blockIdx.x;
    const int d = threadIdx.x;
    const int64_t rows = p.rows;
    const int ns = p.nsplit;
    // the first MS partials are loaded together, before the maximum is known (one
    // memory round trip); missing ones read as an empty chunk (LSE -inf, O 0), which
    // changes neither the maximum nor the sums
    constexpr int MS = 8;
    float lv[MS], ov[MS];
#pragma unroll
    for (int s = 0; s < MS; ++s) {
        const bool live = s < ns;
        lv[s] = live ? p.lpart[(int64_t)s * rows + row] : NEG_INF;
        ov[s] = live ? p.opart[((int64_t)s * rows + row) * D + d] : 0.f;
    }
    float mx = NEG_INF;
#pragma unroll
    for (int s = 0; s < MS; ++s) mx = fmaxf(mx, lv[s]);
    for (int s = MS; s < ns; ++s) mx = fmaxf(mx, p.lpart[(int64_t)s * rows + row]);
    float sum = 0.f, acc = 0.f;
    if (mx != NEG_INF) {
#pragma unroll
        for (int s = 0; s < MS; ++s) {
            const float w = (lv[s] == NEG_INF) ? 0.f : expf(lv[s] - mx);
            sum += w;
            acc += w * ov[s];
        }
        for (int s = MS; s < ns; ++s) {
            const float l = p.lpart[(int64_t)s * rows + row];
            const float w = (l == NEG_INF) ? 0.f : expf(l - mx);
            sum += w;
            acc += w * p.opart[((int64_t)s * rows + row) * D + d];
        }
    }
    const float o = (sum > 0.f) ? acc / sum : 0.f;
    uint16_t* out = (uint16_t*)p.o + row * D + d;
    if (DT == ATTN_IMPL_BF16) {
        const __bf16 v = (__bf16)o;
        *out = __builtin_bit_cast(uint16_t, v);
    } else {
        const _Float16 v = (_Float16)o;
        *out = __builtin_bit_cast(uint16_t, v);
    }
    if (p.lse && d == 0) p.lse[row] = (sum > 0.f) ? mx + logf(sum) : NEG_INF;
}

// Device address of this GPU's `scratch`, looked up once per device (with that
// device current) and kept: host code never passes the array's name itself,
// which on the host is only a stand-in for the symbol.
namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::atomic<void*> scratch_ptr[SCRATCH_MAX_DEVICES];
std::mutex scratch_mutex;
}  // namespace

int decode_scratch(void** ptr, size_t* bytes) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return 1;
    void* a = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!a) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        a = scratch_ptr[dev].load(std::memory_order_acquire);
        if (!a) {
            void* q = nullptr;
            if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return 1;
            scratch_ptr[dev].store(q, std::memory_order_release);
            a = q;
        }
    }
    *ptr = a;
    *bytes = DECODE_SCRATCH_BYTES;
    return 0;
}

template <int DT, int D>
static const void* pick_split(int causal) {
    return causal ? (const void*)attn_decode_split<DT, D, true> : (const void*)attn_decode_split<DT, D, false>;
}

const void* select_decode_split(int dtype, int D, int causal) {
    if (dtype == ATTN_IMPL_BF16) return D == 64 ? pick_split<ATTN_IMPL_BF16, 64>(causal)
                                     : D == 128 ? pick_split<ATTN_IMPL_BF16, 128>(causal) : nullptr;
    if (dtype == ATTN_IMPL_FP16) return D == 64 ? pick_split<ATTN_IMPL_FP16, 64>(causal)
                                     : D == 128 ? pick_split<ATTN_IMPL_FP16, 128>(causal) : nullptr;
    return nullptr;
}

const void* select_decode_merge(int dtype, int D) {
    if (dtype == ATTN_IMPL_BF16) return D == 64 ? (const void*)attn_decode_merge<ATTN_IMPL_BF16, 64>
                                     : D == 128 ? (const void*)attn_decode_merge<ATTN_IMPL_BF16, 128> : nullptr;
    if (dtype == ATTN_IMPL_FP16) return D == 64 ? (const void*)attn_decode_merge<ATTN_IMPL_FP16, 64>
                                     : D == 128 ? (const void*)attn_decode_merge<ATTN_IMPL_FP16, 128> : nullptr;
    return nullptr;
}

}  // namespace attn_impl
