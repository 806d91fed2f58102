"""Attention with the rotary embedding (attn_fwd_rope) against the oracle (GPU).

The oracle rotates Q (query i at position i + Sk - Sq) and K (key j at position
j) in fp64, rounds each rotated element once into the storage type and runs its
attention on the result.  Checked here: the rotated keys the library writes are
bit-identical to the oracle's; O and the LSE agree with the oracle within the
attention tolerances on every element of small and ragged shapes (both pair
layouts, bf16 and fp16, D = 64 and 128, MHA, GQA, MQA, causal and not, Sq < Sk);
the queries, rotated inside the attention kernel, are checked bit for bit by
running the plain attention kernel on the oracle's rotated Q and K; the RoPE
workload at full size on every element."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from attention_attn_fwd_02_amd import ATTN_ROPE_HALVES, ATTN_ROPE_INTERLEAVED, fwd, fwd_rope
from attention_attn_fwd_02_amd import workloads as W
from gpu_helpers import compare, say

pytestmark = pytest.mark.gpu


def run_rope(w, layout, base=10000.0, scale=None):
    dev = torch.device("cuda:0")
    q, k, v = W.make_inputs(w)
    ct, st = W.rope_tables(w.Sk, w.D, base)
    sc = w.scale if scale is None else scale
    qd, kd, vd, cd, sd = (t.to(dev) for t in (q, k, v, ct, st))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    k_rot = torch.full_like(kd, float("nan"))
    fwd_rope(qd, kd, vd, cd, sd, layout=layout, causal=w.causal, scale=sc, out=o, lse=lse,
             k_rot=k_rot)
    torch.cuda.synchronize()
    return (q, k, v, ct, st, sc), (o.cpu(), lse.cpu(), k_rot.cpu())


# (dtype, B, Hq, Hkv, Sq, Sk, D, causal, layout)
SHAPES = [
    ("bf16", 1, 2, 2, 300, 300, 128, True, ATTN_ROPE_INTERLEAVED),
    ("bf16", 1, 2, 2, 300, 300, 128, True, ATTN_ROPE_HALVES),
    ("fp16", 1, 4, 2, 100, 333, 64, True, ATTN_ROPE_HALVES),
    ("fp16", 1, 4, 2, 100, 333, 64, False, ATTN_ROPE_INTERLEAVED),
    ("bf16", 2, 4, 1, 257, 257, 128, False, ATTN_ROPE_HALVES),
    ("bf16", 1, 8, 1, 1, 513, 128, True, ATTN_ROPE_INTERLEAVED),
    ("bf16", 1, 2, 2, 1000, 1000, 64, True, ATTN_ROPE_INTERLEAVED),
    ("fp16", 1, 2, 1, 700, 700, 128, True, ATTN_ROPE_HALVES),
    ("bf16", 1, 6, 2, 300, 300, 128, True, ATTN_ROPE_HALVES),
    ("bf16", 2, 8, 4, 200, 300, 128, True, ATTN_ROPE_INTERLEAVED),   # key pass: 4 heads per thread
    ("fp16", 1, 6, 3, 150, 150, 64, False, ATTN_ROPE_HALVES),        # key pass: 1 head per thread
]


@pytest.mark.parametrize("shape", SHAPES, ids=["%s_b%d_hq%d_hkv%d_sq%d_sk%d_d%d_%s_l%d" % (
    s[0], *s[1:7], "causal" if s[7] else "full", s[8]) for s in SHAPES])
def test_rope_full_output(shape):
    dt, B, Hq, Hkv, Sq, Sk, D, causal, layout = shape
    seed = zlib.crc32(repr(shape).encode()) % 100000
    w = W.custom(dt, B, Hq, Hkv, Sq, Sk, D, causal, seed=seed)
    say("case", w.name, "layout", layout)
    (q, k, v, ct, st, sc), (o, lse, k_rot) = run_rope(w, layout)
    o_ref, lse_ref, k_ref = oracle.attn_fwd_rope(q, k, v, ct.numpy(), st.numpy(), layout,
                                                 causal=causal, scale=sc)
    assert torch.equal(k_rot.view(torch.int16), k_ref.view(torch.int16)), "rotated K differs"
    e = compare(o, lse, o_ref, lse_ref, dt, w.name)
    say("  k_rot bit-exact; max|dO| %.3g  max|dLSE| %.3g" % e)
    # the queries: the plain kernel on the oracle's rotated Q and K reproduces the
    # rotary kernel's output bit for bit
    _, q_ref = oracle.rope(q, ct.numpy(), st.numpy(), layout, pos_offset=Sk - Sq)
    dev = torch.device("cuda:0")
    o2, lse2 = fwd(q_ref.to(dev), k_ref.to(dev), v.to(dev), causal=causal, scale=sc)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu().view(torch.int16), o.view(torch.int16)), "rotated Q differs"
    assert torch.equal(lse2.cpu(), lse)


def test_rope_large_angles_and_scales():
    """A small base turns every pair fast (angles up to hundreds of radians), with
    a negative and a large scale."""
    w = W.custom("bf16", 1, 2, 1, 200, 260, 128, True, seed=77)
    for layout in (ATTN_ROPE_INTERLEAVED, ATTN_ROPE_HALVES):
        for scale in (-0.2, 0.5):
            say("case", w.name, "layout", layout, "base 3, scale", scale)
            (q, k, v, ct, st, sc), (o, lse, k_rot) = run_rope(w, layout, base=3.0, scale=scale)
            o_ref, lse_ref, k_ref = oracle.attn_fwd_rope(q, k, v, ct.numpy(), st.numpy(), layout,
                                                         causal=True, scale=sc)
            assert torch.equal(k_rot.view(torch.int16), k_ref.view(torch.int16))
            compare(o, lse, o_ref, lse_ref, "bf16", w.name)


def test_rope_deterministic_and_identity_tables():
    """Angle-zero tables reduce the rotary path to attn_fwd exactly; two calls give
    identical bits."""
    dev = torch.device("cuda:0")
    w = W.custom("bf16", 1, 4, 2, 333, 333, 128, True, seed=5)
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    ones = torch.ones(333, 64, device=dev)
    zeros = torch.zeros(333, 64, device=dev)
    o1, l1, kr = fwd_rope(q, k, v, ones, zeros, causal=True)
    o0, l0 = fwd(q, k, v, causal=True)
    ct, st = (t.to(dev) for t in W.rope_tables(333, 128))
    a = fwd_rope(q, k, v, ct, st, causal=True)
    b = fwd_rope(q, k, v, ct, st, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(kr.view(torch.int16), k.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16)) and torch.equal(l1, l0)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype != torch.float32 else x,
                           y.view(torch.int16) if y.dtype != torch.float32 else y)


def test_rope_workload_full_size_whole_output():
    """The RoPE workload at full size (B=2, H=32, S=4096, D=128, causal, bf16), in
    the launch configuration the benchmark times: every rotated key against the
    oracle, bit for bit; every element of O and the LSE within the forward bounds."""
    name = "rope_causal_bf16_b2_h32_s4096_d128"
    w = W.lookup(name)
    layout = W.ROPE_LAYOUT[name]
    say("case", name, "(full size, every element)")
    (q, k, v, ct, st, sc), (o, lse, k_rot) = run_rope(w, layout)
    _, k_ref = oracle.rope(k, ct.numpy(), st.numpy(), layout, pos_offset=0)
    assert torch.equal(k_rot.view(torch.int16), k_ref.view(torch.int16)), "rotated K differs"
    _, q_ref = oracle.rope(q, ct.numpy(), st.numpy(), layout, pos_offset=w.Sk - w.Sq)
    o_ref, lse_ref = oracle.attn_fwd(q_ref, k_ref, v, causal=True, scale=sc)
    e = compare(o, lse, o_ref, lse_ref, "bf16", name)
    say("  %s: every element, max|dO| %.4g  max|dLSE| %.4g" % ((name,) + e))
