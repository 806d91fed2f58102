"""Seeded random problems against the fp64 oracle (GPU).

The hand-picked shape lists of the other tests keep their variables apart; these
problems draw them together from one fixed seed (the same list on every run):
any query count against any key count, one to six query heads per K/V head, both
masks, bf16, fp16 and fp32, D = 64 and 128, the scale of either sign, and Q and K
spread by 0.5, 1 or 2.  Every problem checks the forward on every output element;
16-bit problems whose query rows per K/V head fit one MFMA block also run split-KV
decoding, and the 16-bit ones run the backward against the oracle's gradients."""
import numpy as np
import pytest
import torch

import oracle
from attention_attn_fwd_02_amd import bwd, fwd, fwd_decode
from attention_attn_fwd_02_amd import workloads as W
from gpu_helpers import bwd_tolerance, compare, run_gpu, say

pytestmark = pytest.mark.gpu

MAX_PAIRS = 3_000_000          # B * Hq * Sq * Sk, so the oracle takes about a second


def draw_problems(n, seed):
    """n problems (dtype, B, Hq, Hkv, Sq, Sk, D, causal, sigma, scale, seed)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dtype = str(rng.choice(["bf16", "bf16", "fp16", "fp32"]))
        D = int(rng.choice([64, 128]))
        R = int(rng.integers(1, 7))
        Hkv = int(rng.integers(1, 4))
        B = int(rng.integers(1, 3))
        u = rng.random()
        Sq = int(rng.integers(1, 9)) if u < 0.25 else int(rng.integers(1, 40)) if u < 0.4 else int(rng.integers(1, 700))
        Sk = Sq if rng.random() < 0.3 else int(rng.integers(1, 900))
        causal = bool(rng.integers(0, 2))
        sigma = float(rng.choice([0.5, 1.0, 2.0]))
        scale = float(1.0 / np.sqrt(D)) if rng.random() < 0.5 else float(rng.uniform(-0.4, 0.4))
        if B * R * Hkv * Sq * Sk > MAX_PAIRS:
            continue
        out.append((dtype, B, R * Hkv, Hkv, Sq, Sk, D, causal, sigma, scale, 5000 + len(out)))
    return out


PROBLEMS = draw_problems(36, 20261202)


def _id(p):
    return "%s_b%d_hq%d_hkv%d_sq%d_sk%d_d%d_%s_s%.2g_sc%.3g" % (
        p[0], *p[1:7], "causal" if p[7] else "full", p[8], p[9])


@pytest.mark.parametrize("prob", PROBLEMS, ids=[_id(p) for p in PROBLEMS])
def test_random_problem(prob):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal, sigma, scale, seed = prob
    w = W.custom(dtype, B, Hq, Hkv, Sq, Sk, D, causal, seed,
                 q_dist=("normal", sigma), k_dist=("normal", sigma))
    say("case", _id(prob))
    q, k, v = W.make_inputs(w)
    o, lse = run_gpu(q, k, v, causal, scale=scale)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=causal, scale=scale)
    e = compare(o, lse, o_ref, lse_ref, dtype, w.name)
    say("  forward: max|dO| %.3g  max|dLSE| %.3g" % e)
    if dtype == "fp32":
        return
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    if (Hq // Hkv) * Sq <= 32:
        od = torch.full_like(qd, float("nan"))
        ld = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=dev)
        fwd_decode(qd, kd, vd, causal=causal, scale=scale, out=od, lse=ld)
        torch.cuda.synchronize()
        e = compare(od.cpu(), ld.cpu(), o_ref, lse_ref, dtype, w.name + " decode")
        say("  decode: max|dO| %.3g  max|dLSE| %.3g" % e)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)
    og, lg = fwd(qd, kd, vd, causal=causal, scale=scale)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    bwd(qd, kd, vd, og, lg, do.to(dev), causal=causal, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(q, k, v, do, causal=causal, scale=scale)
    for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        gf = got.cpu().to(torch.float64).numpy()
        assert not np.isnan(gf).any(), "%s: NaN in %s" % (w.name, name)
        err = float(np.abs(gf - want).max())
        tol = bwd_tolerance(want, dtype)
        say("  %s: max|err| %.3g  tol %.3g" % (name, err, tol))
        assert err <= tol, "%s %s: max |err| %.3g > %.3g" % (w.name, name, err, tol)
