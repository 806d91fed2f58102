"""Hygiene of the HIP path (GPU): outputs written exactly where they belong,
bitwise-deterministic results, any stream, no stray writes."""
import pytest
import torch

from attention_attn_fwd_02_amd import AttnError, fwd
from attention_attn_fwd_02_amd import workloads as W
from gpu_helpers import run_gpu, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _inputs(dt, B, Hq, Hkv, Sq, Sk, D, causal, seed):
    w = W.custom(dt, B, Hq, Hkv, Sq, Sk, D, causal, seed)
    return [t.to(DEV) for t in W.make_inputs(w)]


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("fp16", 64), ("fp32", 128)])
def test_deterministic(dt, D):
    say("case determinism", dt, D)
    q, k, v = _inputs(dt, 2, 8, 2, 1500, 1500, D, True, 3)
    o1, l1 = fwd(q, k, v, causal=True)
    o2, l2 = fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8))
    assert torch.equal(l1.view(torch.uint8), l2.view(torch.uint8))


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_no_writes_outside_outputs(dt):
    """O and LSE live inside larger buffers filled with a canary; only the
    output window may change."""
    say("case canaries", dt)
    B, Hq, Hkv, Sq, Sk, D = 1, 3, 1, 333, 200, 64
    q, k, v = _inputs(dt, B, Hq, Hkv, Sq, Sk, D, True, 4)
    n_o = B * Hq * Sq * D
    n_l = B * Hq * Sq
    pad = 4096
    big_o = torch.full((n_o + 2 * pad,), 7.0, dtype=q.dtype, device=DEV)
    big_l = torch.full((n_l + 2 * pad,), 7.0, dtype=torch.float32, device=DEV)
    o = big_o[pad:pad + n_o].view(B, Hq, Sq, D)
    lse = big_l[pad:pad + n_l].view(B, Hq, Sq)
    fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(big_o[:pad] == 7.0) and torch.all(big_o[pad + n_o:] == 7.0)
    assert torch.all(big_l[:pad] == 7.0) and torch.all(big_l[pad + n_l:] == 7.0)
    # the window itself was written (Sq > Sk leaves empty rows: O = 0, LSE = -inf)
    assert not torch.any(o == 7.0)
    assert torch.all(lse[:, :, :Sq - Sk] == float("-inf"))
    assert torch.all(o[:, :, :Sq - Sk] == 0)


def test_side_stream_matches_default_stream():
    say("case side stream")
    q, k, v = _inputs("bf16", 1, 4, 4, 700, 700, 128, True, 6)
    o1, l1 = fwd(q, k, v, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = fwd(q, k, v, causal=True, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_binding_rejects_bad_shapes_before_launch():
    q, k, v = _inputs("bf16", 1, 4, 2, 64, 64, 128, False, 7)
    with pytest.raises(ValueError):
        fwd(q, k[:, :1].contiguous(), v, causal=False)
    q96 = torch.zeros(1, 4, 64, 96, dtype=torch.bfloat16, device=DEV)
    k96 = torch.zeros(1, 2, 64, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(AttnError):
        fwd(q96, k96, k96)
    q3 = torch.zeros(1, 3, 64, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(AttnError):
        fwd(q3, k, v)   # Hq % Hkv != 0
