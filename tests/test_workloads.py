"""The seeded input generator and the FLOP convention (CPU only)."""
import math

import pytest
import torch

from attention_attn_fwd_02_amd import workloads as W


def test_visible_pairs_matches_enumeration():
    for Sq, Sk in [(1, 1), (5, 5), (4, 9), (9, 4), (7, 1), (1, 7), (64, 64), (17, 130)]:
        for causal in (False, True):
            brute = sum(1 for i in range(Sq) for j in range(Sk)
                        if (not causal) or j <= i + Sk - Sq)
            assert W.visible_pairs(1, 1, Sq, Sk, causal) == brute, (Sq, Sk, causal)
    assert W.visible_pairs(2, 3, 10, 10, True) == 6 * 55


def test_headline_flops():
    w = W.WORKLOADS[W.HEADLINE]
    assert (w.dtype, w.B, w.Hq, w.Sq, w.D, w.causal) == ("bf16", 2, 32, 4096, 128, True)
    assert w.flops() == 4 * 128 * 64 * (4096 * 4097 // 2)


def test_inputs_are_seeded_and_shaped():
    w = W.custom("bf16", 2, 4, 2, 33, 47, 64, True, seed=5)
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    q, k, v = a
    assert q.shape == (2, 4, 33, 64) and k.shape == (2, 2, 47, 64) and v.shape == k.shape
    assert q.dtype == torch.bfloat16 and q.is_contiguous()
    c = W.make_inputs(w, seed=6)
    assert not torch.equal(a[0], c[0])


def test_distributions():
    w = W.custom("fp32", 1, 2, 2, 4096, 4096, 64, False, seed=9, q_dist=("normal", 2.0),
                 v_dist=("uniform", 1.0))
    q, k, v = W.make_inputs(w)
    assert abs(q.std().item() - 2.0) < 0.02 and abs(k.std().item() - 1.0) < 0.01
    assert v.min().item() >= -1.0 and v.max().item() <= 1.0
    assert abs(v.std().item() - (1 / 3) ** 0.5) < 0.01


def test_all_workloads_listed():
    assert len(W.WORKLOADS) == 5
    assert W.WORKLOADS["mha_fp32_b1_h2_s128_d64"].dtype == "fp32"
    g = W.WORKLOADS["gqa4_causal_bf16_b1_hq32_hkv8_s8192_d128"]
    assert g.Hq // g.Hkv == 4


def test_attention_variants():
    """MQA, GQA with eight query heads per K/V head, and fp16, all at L = 4096, d = 128."""
    m = W.VARIANTS["mqa_causal_bf16_b2_hq32_hkv1_s4096_d128"]
    g = W.VARIANTS["gqa8_causal_bf16_b2_hq32_hkv4_s4096_d128"]
    f = W.VARIANTS["mha_causal_fp16_b2_h32_s4096_d128"]
    assert m.Hkv == 1 and g.Hq // g.Hkv == 8 and f.dtype == "fp16"
    for w in (m, g, f):
        assert (w.Sq, w.Sk, w.D, w.causal) == (4096, 4096, 128, True)
        # query-side work is the headline's: same FLOPs, fewer K/V bytes
        assert w.flops() == W.WORKLOADS[W.HEADLINE].flops()
        assert W.lookup(w.name) is w
    assert m.min_hbm_bytes() < g.min_hbm_bytes() < f.min_hbm_bytes()
    q, k, v = W.make_inputs(W.custom("fp16", 1, 2, 1, 8, 8, 64, True, seed=3))
    assert q.dtype == torch.float16 and k.shape == (1, 1, 8, 64)
    with pytest.raises(KeyError):
        W.lookup("no_such_workload")


def test_rope_tables():
    """Position 0 is the identity, pair 0 turns by one radian per position, the
    last pair by base^(-(D-2)/D) radians, and every entry is a rounded unit vector."""
    c, s = W.rope_tables(4096, 128)
    assert c.shape == (4096, 64) and c.dtype == torch.float32
    assert torch.all(c[0] == 1) and torch.all(s[0] == 0)
    assert abs(float(c[3, 0]) - math.cos(3.0)) < 1e-7 and abs(float(s[3, 0]) - math.sin(3.0)) < 1e-7
    theta = 10000.0 ** (-126.0 / 128.0)
    assert abs(float(s[4000, 63]) - math.sin(4000 * theta)) < 1e-7
    n = c.double() ** 2 + s.double() ** 2
    assert float((n - 1).abs().max()) < 2e-7
    w = W.lookup("rope_causal_bf16_b2_h32_s4096_d128")
    assert (w.B, w.Hq, w.Sq, w.D, w.causal) == (2, 32, 4096, 128, True)
    assert W.ROPE_LAYOUT[w.name] in (1, 2)
