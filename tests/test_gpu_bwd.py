"""Gradients (attn_bwd) against the fp64 oracle's chain-rule gradients (GPU).

The GPU backward consumes the GPU forward's O and LSE, as a training step would;
the oracle recomputes everything from the inputs in fp64.  Every element of dQ,
dK and dV is compared on small and ragged shapes (MHA, GQA, MQA, causal and not,
Sq != Sk with key-less rows, bf16 and fp16, D = 64 and 128).  The grouped-query
shapes here have few K/V heads, so the library splits the query heads of each
K/V head over 2 to 8 workgroups and adds their fp32 partial dK, dV in a separate
pass; the MHA shapes take the direct path."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from attention_attn_fwd_02_amd import bwd, fwd
from attention_attn_fwd_02_amd import workloads as W
from gpu_helpers import bwd_tolerance, say

pytestmark = pytest.mark.gpu


def run_bwd(w, seed_g, scale=None):
    dev = torch.device("cuda:0")
    q, k, v = W.make_inputs(w)
    g = torch.Generator().manual_seed(seed_g)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)
    sc = w.scale if scale is None else scale
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fwd(qd, kd, vd, causal=w.causal, scale=sc)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=sc, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(q, k, v, do, causal=w.causal, scale=sc)
    errs = []
    for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        gf = got.cpu().to(torch.float64).numpy()
        assert not np.isnan(gf).any(), "%s: NaN in %s (unwritten or invalid)" % (w.name, name)
        err = float(np.abs(gf - want).max())
        tol = bwd_tolerance(want, w.dtype)
        say("  %s: max|err| %.3g  max|ref| %.3g  tol %.3g" % (name, err, np.abs(want).max(), tol))
        assert err <= tol, "%s %s: max |err| %.3g > %.3g" % (w.name, name, err, tol)
        errs.append(err)
    return errs


# (dtype, B, Hq, Hkv, Sq, Sk, D, causal)
SHAPES = [
    ("bf16", 1, 2, 2, 64, 64, 128, True),
    ("bf16", 1, 2, 2, 300, 300, 128, True),      # ragged query and key tiles
    ("bf16", 2, 4, 1, 200, 333, 128, True),      # MQA, fewer queries than keys
    ("bf16", 1, 4, 2, 333, 200, 64, True),       # more queries than keys: key-less rows
    ("bf16", 1, 8, 2, 512, 512, 128, False),     # GQA
    ("fp16", 1, 2, 2, 257, 257, 128, True),
    ("fp16", 1, 4, 4, 130, 70, 64, False),
    ("bf16", 1, 2, 1, 1, 1, 64, True),
    ("bf16", 1, 2, 2, 1000, 1000, 128, True),    # several key blocks and query tiles
    ("bf16", 1, 16, 2, 768, 768, 128, True),     # 8 query heads per K/V head over 8 workgroups
    ("fp16", 1, 8, 1, 300, 260, 64, False),      # MQA, 8 partial sums per key row
    ("bf16", 1, 6, 2, 300, 300, 128, True),      # three query heads per K/V head: no split
    ("bf16", 3, 8, 4, 200, 170, 64, True),       # 12 groups, 2 splits each
]


@pytest.mark.parametrize("shape", SHAPES, ids=["%s_b%d_hq%d_hkv%d_sq%d_sk%d_d%d_%s" % (
    s[0], *s[1:7], "causal" if s[7] else "full") for s in SHAPES])
def test_bwd_full_output(shape):
    dt, B, Hq, Hkv, Sq, Sk, D, causal = shape
    seed = zlib.crc32(repr(shape).encode()) % 100000
    w = W.custom(dt, B, Hq, Hkv, Sq, Sk, D, causal, seed=seed)
    say("case", w.name)
    run_bwd(w, seed + 1)


@pytest.mark.parametrize("scale", [-0.125, -0.1, 0.0, 0.125, 0.3, 1e-39, -2e-38])
def test_bwd_other_scales(scale):
    """Signs, zero, and scales so small (a subnormal one included) that the scores
    contribute nothing: the weights are then 1/|J_i| of each row."""
    w = W.custom("bf16", 1, 2, 1, 150, 220, 128, True, seed=8)
    say("case", w.name, "scale", scale)
    run_bwd(w, 9, scale=scale)


def test_bwd_deterministic():
    dev = torch.device("cuda:0")
    w = W.custom("bf16", 1, 4, 2, 400, 400, 128, True, seed=12)
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(3)).to(q.dtype).to(dev)
    o, lse = fwd(q, k, v, causal=True)
    a = bwd(q, k, v, o, lse, do, causal=True)
    b = bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_full_size_sampled_heads():
    """The backward workload at full size (B=2, H=32, S=4096, D=128, causal bf16),
    run in the launch configuration the benchmark times; whole heads are checked
    against the oracle run on that head alone (heads do not interact)."""
    w = W.lookup("bwd_causal_bf16_b2_h32_s4096_d128")
    dev = torch.device("cuda:0")
    q, k, v = W.make_inputs(w)
    do = W.make_dout(w, q)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fwd(qd, kd, vd, causal=True, scale=w.scale)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    bwd(qd, kd, vd, o, lse, dod, causal=True, scale=w.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert not torch.isnan(t).any(), "NaN in a gradient (unwritten or invalid)"
    # sixteen whole heads of both batches (a quarter of the problem): the first and
    # last heads and fourteen drawn with a fixed seed
    rng = np.random.default_rng(w.seed)
    drawn = [divmod(int(x), w.Hq) for x in rng.choice(np.arange(1, w.B * w.Hq - 1), 14, replace=False)]
    heads = tuple([(0, 0), (w.B - 1, w.Hq - 1)] + drawn)
    say("case", w.name, "heads", heads)
    # the chosen heads stacked as a batch of one-head problems (one oracle thread each)
    sl = lambda t: torch.cat([t[b:b + 1, h:h + 1] for b, h in heads]).contiguous()
    ref = oracle.attn_bwd(sl(q), sl(k), sl(v), sl(do), causal=True, scale=w.scale)
    for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        gf = sl(got.cpu()).to(torch.float64).numpy()
        worst = 0.0
        for i, bh in enumerate(heads):
            err = float(np.abs(gf[i] - want[i]).max())
            tol = bwd_tolerance(want[i], w.dtype)
            worst = max(worst, err / tol)
            assert err <= tol, "head %s %s: max |err| %.3g > %.3g" % (bh, name, err, tol)
        say("  %s over %d heads: worst max|err| / tol %.3f" % (name, len(heads), worst))


def test_bwd_gqa_workload_full_size():
    """The grouped-query backward workload at full size (B=1, Hq=32, Hkv=4, S=4096,
    D=128, causal bf16; 8 query heads per K/V head, split over 4 workgroups), in the
    launch configuration the benchmark times, against the identity that holds at any
    size: with every K/V head repeated for its query heads the problem becomes MHA,
    whose dQ is the same and whose dK, dV summed over each group's heads are the
    grouped dK, dV (the MHA run takes the direct path, no partial sums); and one
    whole K/V-head group (its eight query heads' dQ, the shared dK, dV) against
    the oracle."""
    w = W.lookup("bwd_gqa8_causal_bf16_b1_hq32_hkv4_s4096_d128")
    R = w.Hq // w.Hkv
    dev = torch.device("cuda:0")
    q, k, v = W.make_inputs(w)
    do = W.make_dout(w, q)
    say("case", w.name)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fwd(qd, kd, vd, causal=True, scale=w.scale)
    dq, dk, dv = bwd(qd, kd, vd, o, lse, dod, causal=True, scale=w.scale)
    ke = kd.repeat_interleave(R, dim=1).contiguous()
    ve = vd.repeat_interleave(R, dim=1).contiguous()
    o2, lse2 = fwd(qd, ke, ve, causal=True, scale=w.scale)
    dq2, dk2, dv2 = bwd(qd, ke, ve, o2, lse2, dod, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    assert torch.equal(dq.view(torch.int16), dq2.view(torch.int16)), "dQ differs from MHA's"
    for name, got, exp in (("dk", dk, dk2), ("dv", dv, dv2)):
        want = exp.float().reshape(w.B, w.Hkv, R, w.Sk, w.D).sum(dim=2).double().cpu().numpy()
        gf = got.cpu().to(torch.float64).numpy()
        assert not np.isnan(gf).any(), "NaN in " + name
        err = float(np.abs(gf - want).max())
        tol = bwd_tolerance(want, w.dtype)
        say("  %s: max|grouped - summed MHA| %.3g  max|ref| %.3g  tol %.3g"
            % (name, err, np.abs(want).max(), tol))
        assert err <= tol, "%s: max |err| %.3g > %.3g" % (name, err, tol)
    # one whole K/V-head group against the oracle: its R query heads run as R
    # one-head problems on the shared K/V head (one oracle thread each); the group's
    # dK, dV are the sums of theirs over the query heads (the gradient of a shared
    # input), taken here in fp64
    g = 1
    hs = range(g * R, (g + 1) * R)
    say("  K/V group %d (query heads %d..%d) against the oracle" % (g, hs[0], hs[-1]))
    rep = lambda t: torch.cat([t[:, g:g + 1]] * R, dim=0).contiguous()
    qs = torch.cat([q[:, h:h + 1] for h in hs], dim=0).contiguous()
    dos = torch.cat([do[:, h:h + 1] for h in hs], dim=0).contiguous()
    rq, rk, rv = oracle.attn_bwd(qs, rep(k), rep(v), dos, causal=True, scale=w.scale)
    checks = (("dq", torch.cat([dq.cpu()[:, h:h + 1] for h in hs], dim=0), rq),
              ("dk", dk.cpu()[:, g:g + 1], rk.sum(axis=0, keepdims=True)),
              ("dv", dv.cpu()[:, g:g + 1], rv.sum(axis=0, keepdims=True)))
    for name, got, want in checks:
        gf = got.to(torch.float64).numpy()
        err = float(np.abs(gf - want).max())
        tol = bwd_tolerance(want, w.dtype)
        say("  %s (group %d) vs oracle: max|err| %.3g  max|ref| %.3g  tol %.3g"
            % (name, g, err, np.abs(want).max(), tol))
        assert err <= tol, "group %d %s: max |err| %.3g > %.3g" % (g, name, err, tol)
