"""Split-KV decode path (attn_fwd_decode) against the fp64 oracle (GPU).

Every output element is compared on shapes with one or a few query rows per head:
MHA, GQA, MQA, ragged chunk tails, Sq > 1 with the causal mask, Sq > Sk (rows with
no visible key), explicit and automatic chunk counts, and the decode workload at
full size (every element).  The split and merge must give a deterministic result that
agrees with the prefill path to the stated tolerance."""
import zlib

import pytest
import torch

import oracle
from attention_attn_fwd_02_amd import fwd, fwd_decode
from attention_attn_fwd_02_amd import workloads as W
from gpu_helpers import TOL_O, compare, say

pytestmark = pytest.mark.gpu

# (dtype, B, Hq, Hkv, Sq, Sk, D, causal, nsplit)
SHAPES = [
    ("bf16", 2, 8, 2, 1, 4096, 128, True, 0),
    ("bf16", 1, 32, 1, 1, 1000, 128, True, 3),       # MQA, ragged last chunk
    ("fp16", 2, 4, 4, 1, 777, 64, False, 5),
    ("bf16", 1, 8, 2, 4, 300, 128, True, 0),         # four query rows per head, causal
    ("bf16", 1, 2, 1, 8, 5, 64, True, 0),            # Sq > Sk: rows without keys
    ("bf16", 3, 16, 2, 2, 2049, 128, False, 100),    # many chunks, a 1-key tail
    ("bf16", 1, 4, 4, 1, 33, 128, False, 1),         # one chunk
    ("fp16", 1, 8, 1, 3, 513, 128, True, 0),
    ("bf16", 2, 2, 2, 1, 1, 64, True, 0),            # a single key
]


def run_decode(q, k, v, causal, nsplit, scale=None):
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    fwd_decode(qd, kd, vd, causal=causal, scale=scale, nsplit=nsplit, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("shape", SHAPES, ids=["%s_b%d_hq%d_hkv%d_sq%d_sk%d_d%d_%s_ns%d" % (
    s[0], *s[1:7], "causal" if s[7] else "full", s[8]) for s in SHAPES])
def test_decode_full_output(shape):
    dt, B, Hq, Hkv, Sq, Sk, D, causal, ns = shape
    w = W.custom(dt, B, Hq, Hkv, Sq, Sk, D, causal, seed=zlib.crc32(repr(shape).encode()) % 100000)
    say("case", w.name, "nsplit", ns)
    q, k, v = W.make_inputs(w)
    o, lse = run_decode(q, k, v, causal, ns, scale=w.scale)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=causal, scale=w.scale)
    e = compare(o, lse, o_ref, lse_ref, dt, w.name)
    say("  max|dO| %.3g  max|dLSE| %.3g" % e)


def test_decode_scales_and_peaky():
    w = W.custom("bf16", 1, 8, 2, 1, 1500, 128, False, seed=321, q_dist=("normal", 4.0),
                 k_dist=("normal", 4.0))
    q, k, v = W.make_inputs(w)
    for scale in (-0.2, 0.0, 0.088, 1.5):
        o, lse = run_decode(q, k, v, False, 0, scale=scale)
        o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=False, scale=scale)
        e = compare(o, lse, o_ref, lse_ref, "bf16", "peaky scale %g" % scale)
        say("  scale %g: max|dO| %.3g  max|dLSE| %.3g" % (scale, *e))


def test_decode_deterministic_and_matches_prefill():
    w = W.custom("bf16", 2, 16, 4, 1, 3000, 128, True, seed=11)
    q, k, v = W.make_inputs(w)
    o1, l1 = run_decode(q, k, v, True, 0, scale=w.scale)
    o2, l2 = run_decode(q, k, v, True, 0, scale=w.scale)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    dev = torch.device("cuda:0")
    op, lp = fwd(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    assert (o1.float() - op.cpu().float()).abs().max().item() <= TOL_O["bf16"]
    assert (l1 - lp.cpu()).abs().max().item() <= 1e-3


@pytest.mark.parametrize("name", list(W.DECODE))
def test_decode_workload_whole_output(name):
    """The decode workloads at full size: every element of O and the LSE against
    the oracle (one query row per sequence and head, so the oracle takes under a
    second)."""
    w = W.lookup(name)
    say("case", name, "(full size, every element)")
    q, k, v = W.make_inputs(w)
    o, lse = run_decode(q, k, v, w.causal, 0, scale=w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=w.causal, scale=w.scale)
    e = compare(o, lse, o_ref, lse_ref, w.dtype, name)
    say("  %s: every element, max|dO| %.4g  max|dLSE| %.4g" % (name, *e))
