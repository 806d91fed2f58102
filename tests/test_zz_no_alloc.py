"""The allocation-free decode entry point (attn_fwd_decode_noalloc) against the
workspace entry point (attn_fwd_decode) and the oracle (GPU).

The two entry points run the same kernels with the same chunking, so their
outputs must agree bit for bit; both must match the oracle within the forward
tolerances.  Two calls in a row, the second smaller, check that the shared static
scratch carries nothing over from one call to the next."""
import numpy as np
import pytest
import torch

import oracle
from attention_attn_fwd_02_amd import AttnError, ATTN_ERR_UNSUPPORTED, fwd_decode, fwd_decode_noalloc
from attention_attn_fwd_02_amd import workloads as W
from gpu_helpers import compare, say

pytestmark = pytest.mark.gpu


def _run_both(w, nsplit):
    dev = torch.device("cuda:0")
    q, k, v = W.make_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o1 = torch.full_like(qd, float("nan"))
    l1 = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    o2 = torch.full_like(qd, float("nan"))
    l2 = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    fwd_decode_noalloc(qd, kd, vd, causal=w.causal, scale=w.scale, nsplit=nsplit, out=o1, lse=l1)
    fwd_decode(qd, kd, vd, causal=w.causal, scale=w.scale, nsplit=nsplit, out=o2, lse=l2)
    torch.cuda.synchronize()
    return (q, k, v), (o1.cpu(), l1.cpu()), (o2.cpu(), l2.cpu())


def test_noalloc_matches_workspace_entry_point_twice():
    # first a large call (about 4.2 MB of partial results), then a smaller one with
    # a different shape, chunking and dtype on the same scratch
    cases = [(W.custom("bf16", 64, 32, 4, 1, 4096, 128, True, seed=31), 0),
             (W.custom("fp16", 3, 8, 2, 4, 777, 64, True, seed=32), 5)]
    for w, ns in cases:
        say("case", w.name, "nsplit", ns)
        (q, k, v), (o1, l1), (o2, l2) = _run_both(w, ns)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "O differs between entry points"
        assert torch.equal(l1, l2), "LSE differs between entry points"
        o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=w.causal, scale=w.scale)
        e = compare(o1, l1, o_ref, lse_ref, w.dtype, w.name)
        say("  bitwise equal to attn_fwd_decode; max|dO| %.3g  max|dLSE| %.3g" % e)


def test_noalloc_refuses_what_does_not_fit():
    # 128 chunks x 256 query rows x (128 + 1) floats = 16.9 MB > 16 MiB: refused on
    # the host before anything is enqueued
    dev = torch.device("cuda:0")
    w = W.custom("bf16", 8, 32, 8, 1, 4096, 128, True, seed=33)
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    with pytest.raises(AttnError) as ei:
        fwd_decode_noalloc(q, k, v, causal=True, nsplit=128)
    assert ei.value.status == ATTN_ERR_UNSUPPORTED
    # the same problem with fewer chunks fits
    o, lse = fwd_decode_noalloc(q, k, v, causal=True, nsplit=16)
    o2, lse2 = fwd_decode(q, k, v, causal=True, nsplit=16)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
