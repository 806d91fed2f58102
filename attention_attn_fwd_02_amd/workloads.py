"""Seeded synthetic attention inputs: the one module both sides draw from.

This module holds no attention arithmetic: it only names workloads and draws
their Q, K, V tensors from a seeded CPU generator.  The HIP path and the fp64
oracle both take the bytes produced here.

The shapes follow the prefill workloads of the page "A Thread-Register
Decoupled GPU Execution Model for Efficient Tensor Computation" (evaluation
set-up, "Workloads": Llama-family prefill attention with L_context = 4096 and
d_head = 128, plus the grouped-query variant).  No dataset or trained weights
are involved; the value distributions are stated per workload.

Recipe (identical for every workload):
  g = torch.Generator().manual_seed(seed)
  Q, K, V drawn in that order, each as one [B, H, S, D] fp32 tensor (BHSD order),
  normal draws are torch.randn(...) * sigma, uniform draws are torch.rand(...) * 2 - 1,
  then cast to the storage dtype with round-to-nearest-even (torch .to()).
"""
from dataclasses import dataclass, field
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "bf16" | "fp16" | "fp32"
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    seed: int
    q_dist: tuple = ("normal", 1.0)   # ("normal", sigma) or ("uniform", half_width)
    k_dist: tuple = ("normal", 1.0)
    v_dist: tuple = ("normal", 1.0)
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs inside the mask, over all heads."""
        return visible_pairs(self.B, self.Hq, self.Sq, self.Sk, self.causal)

    def flops(self) -> int:
        """Algorithmic FLOPs: 2*D for the score dot product plus 2*D for the
        weighted sum of V, per visible (query, key) pair."""
        return 4 * self.D * self.visible_pairs()

    def min_hbm_bytes(self) -> int:
        """Q, K, V read once, O and LSE written once."""
        es = torch.tensor([], dtype=torch_dtype(self.dtype)).element_size()
        q = self.B * self.Hq * self.Sq * self.D
        kv = 2 * self.B * self.Hkv * self.Sk * self.D
        return es * (2 * q + kv) + 4 * self.B * self.Hq * self.Sq


def visible_pairs(B, Hq, Sq, Sk, causal) -> int:
    if not causal:
        return B * Hq * Sq * Sk
    # query i sees keys 0 .. i + (Sk - Sq), clipped to [0, Sk]
    off = Sk - Sq
    tot = 0
    # closed form over the three regimes of i
    lo = max(0, -off)              # first row with at least one visible key
    full = max(lo, min(Sq, Sk - off))  # rows i >= Sk - off see all Sk keys
    # rows lo .. full-1 see i + off + 1 keys
    n = full - lo
    if n > 0:
        a = lo + off + 1
        tot += n * a + n * (n - 1) // 2
    tot += (Sq - full) * Sk
    return B * Hq * tot


def torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[name]


WORKLOADS = {
    w.name: w for w in [
        Workload("mha_fp32_b1_h2_s128_d64", "fp32", 1, 2, 2, 128, 128, 64, False, 1001,
                 note="small fp32 case, non-causal"),
        Workload("mha_bf16_b4_h16_s1024_d64", "bf16", 4, 16, 16, 1024, 1024, 64, False, 1002,
                 note="non-causal, d_head 64"),
        Workload("mha_causal_bf16_b2_h32_s4096_d128", "bf16", 2, 32, 32, 4096, 4096, 128, True,
                 1003, note="Llama-style prefill, L_context 4096, d_head 128 (headline)"),
        Workload("gqa4_causal_bf16_b1_hq32_hkv8_s8192_d128", "bf16", 1, 32, 8, 8192, 8192, 128,
                 True, 1004, v_dist=("uniform", 1.0),
                 note="grouped-query, 4 query heads per key/value head"),
        Workload("mha_causal_bf16_b1_h16_s16384_d128_peaky", "bf16", 1, 16, 16, 16384, 16384,
                 128, True, 1005, q_dist=("normal", 2.0), k_dist=("normal", 2.0),
                 note="long context; Q, K with sigma 2 make the softmax peaky"),
    ]
}

# The workload the headline metric is quoted on (bf16, causal, S = 4096, D = 128).
HEADLINE = "mha_causal_bf16_b2_h32_s4096_d128"
# The order the five workloads are listed in (smallest first).
ORDER = list(WORKLOADS)

# The rest of the pages' attention-variant set at their prefill shape (L_context 4096,
# d_head 128; FIBER page, evaluation set-up): multi-query attention, grouped-query
# attention with eight query heads per key/value head, and fp16 inputs.
VARIANTS = {
    w.name: w for w in [
        Workload("mqa_causal_bf16_b2_hq32_hkv1_s4096_d128", "bf16", 2, 32, 1, 4096, 4096, 128,
                 True, 1006, note="multi-query: all 32 query heads share one key/value head"),
        Workload("gqa8_causal_bf16_b2_hq32_hkv4_s4096_d128", "bf16", 2, 32, 4, 4096, 4096, 128,
                 True, 1007, note="grouped-query, 8 query heads per key/value head"),
        Workload("mha_causal_fp16_b2_h32_s4096_d128", "fp16", 2, 32, 32, 4096, 4096, 128, True,
                 1008, note="the headline shape with fp16 inputs"),
    ]
}


# Decoding (FIBER page, evaluation set-up: FlashDecoding with L_context = 4096 and
# d_head = 128, several sequences with distinct KV caches): one new query row per
# sequence and head against a 4096-key cache.  The batch sizes are a reading (the
# page gives none), chosen so that each workload's K/V (1 GiB for MHA, 512 MiB for
# GQA) exceeds the 256 MiB last-level cache and is measured against HBM.
DECODE = {
    w.name: w for w in [
        Workload("decode_mha_bf16_b16_h32_sk4096_d128", "bf16", 16, 32, 32, 1, 4096, 128, True,
                 1009, note="decode, multi-head: 16 sequences, 32 heads, 4096 cached keys"),
        Workload("decode_gqa8_bf16_b64_hq32_hkv4_sk4096_d128", "bf16", 64, 32, 4, 1, 4096, 128,
                 True, 1010, note="decode, grouped-query with 8 query heads per K/V head"),
    ]
}


# Training (FIBER page, evaluation set-up: FlashAttention backward with
# L_context = 4096 and d_head = 128): the gradients of the headline forward.  The
# output gradient dO is drawn after Q, K, V from the same generator, N(0, 1).
BACKWARD = {
    w.name: w for w in [
        Workload("bwd_causal_bf16_b2_h32_s4096_d128", "bf16", 2, 32, 32, 4096, 4096, 128, True,
                 1011, note="backward of the headline forward"),
        Workload("bwd_gqa8_causal_bf16_b1_hq32_hkv4_s4096_d128", "bf16", 1, 32, 4, 4096, 4096, 128,
                 True, 1013, note="backward, grouped-query with 8 query heads per K/V head"),
    ]
}


# Rotary position embedding ahead of attention (FIBER page, background and evaluation
# set-up: RoPE is one of the vector operations modelled between the GEMMs; VDCores
# page, evaluation: QKV projection fused with RoPE): the headline shape with Q and K
# rotated as they are loaded.  The cos/sin tables are inputs, built by
# `rope_tables` (the rotary embedding's frequencies with base 10000).
ROPE = {
    w.name: w for w in [
        Workload("rope_causal_bf16_b2_h32_s4096_d128", "bf16", 2, 32, 32, 4096, 4096, 128, True,
                 1012, note="headline shape, rotary embedding on Q and K (interleaved pairs)"),
    ]
}
ROPE_LAYOUT = {"rope_causal_bf16_b2_h32_s4096_d128": 1}


def rope_tables(P: int, D: int, base: float = 10000.0):
    """cos/sin tables [P, D/2] (fp32) of the rotary embedding's angles:
    position p, pair i turns by p * base^(-2i/D).  Angles and their cosines and
    sines are taken in fp64 and rounded once to fp32."""
    pos = torch.arange(P, dtype=torch.float64)[:, None]
    inv = base ** (-torch.arange(D // 2, dtype=torch.float64) * 2.0 / D)
    ang = pos * inv[None, :]
    return torch.cos(ang).to(torch.float32).contiguous(), torch.sin(ang).to(torch.float32).contiguous()


def make_dout(w: Workload, q):
    """dO for a backward workload: N(0, 1) in the storage dtype, drawn after Q, K, V."""
    g = torch.Generator().manual_seed(w.seed + 7919)
    return torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)


def bwd_flops(w: Workload) -> int:
    """Algorithmic backward FLOPs: five products of 2*D FLOPs per visible pair
    (S recomputed, dV, dP, dQ, dK)."""
    return 10 * w.D * w.visible_pairs()


def lookup(name: str) -> Workload:
    """A named workload, attention variant, decode, backward or RoPE workload."""
    for table in (WORKLOADS, VARIANTS, DECODE, BACKWARD, ROPE):
        if name in table:
            return table[name]
    raise KeyError("unknown workload %r (known: %s)" % (
        name, ", ".join(list(WORKLOADS) + list(VARIANTS) + list(DECODE) + list(BACKWARD)
                        + list(ROPE))))


def _draw(g, shape, dist):
    kind, p = dist
    if kind == "normal":
        return torch.randn(shape, generator=g, dtype=torch.float32) * p
    if kind == "uniform":
        return (torch.rand(shape, generator=g, dtype=torch.float32) * 2 - 1) * p
    raise ValueError(kind)


def make_inputs(w: Workload, seed=None):
    """Draw (q, k, v) on the CPU in w's storage dtype; contiguous BHSD."""
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    dt = torch_dtype(w.dtype)
    q = _draw(g, (w.B, w.Hq, w.Sq, w.D), w.q_dist).to(dt)
    k = _draw(g, (w.B, w.Hkv, w.Sk, w.D), w.k_dist).to(dt)
    v = _draw(g, (w.B, w.Hkv, w.Sk, w.D), w.v_dist).to(dt)
    return q, k, v


def custom(dtype, B, Hq, Hkv, Sq, Sk, D, causal, seed, q_dist=("normal", 1.0),
           k_dist=("normal", 1.0), v_dist=("normal", 1.0), name=None) -> Workload:
    """A workload of arbitrary shape with the same recipe (for parity cases)."""
    name = name or "custom_%s_b%d_hq%d_hkv%d_sq%d_sk%d_d%d_%s" % (
        dtype, B, Hq, Hkv, Sq, Sk, D, "causal" if causal else "full")
    return Workload(name, dtype, B, Hq, Hkv, Sq, Sk, D, causal, seed, q_dist, k_dist, v_dist)
