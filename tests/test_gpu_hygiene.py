"""Hygiene of the HIP path (GPU): outputs written exactly where they belong,
bitwise-deterministic results, any stream, no stray writes."""
import pytest
import torch

from attention_attn_fwd_02_amd import (AttnError, attn_bwd_workspace, attn_fwd_decode_workspace,
                                       bwd, fwd, fwd_decode, fwd_rope)
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


def test_binding_rejects_bad_output_buffers_before_launch():
    """Caller-supplied outputs and workspaces of the wrong shape, dtype, layout or
    device raise before anything is launched (a short buffer would otherwise be
    written past its end)."""
    q, k, v = _inputs("bf16", 1, 4, 2, 64, 64, 128, True, 8)
    B, Hq, Sq = 1, 4, 64
    lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=DEV)
    bad_out = [torch.empty(1, 4, 63, 128, dtype=torch.bfloat16, device=DEV),       # short
               torch.empty(1, 4, 64, 128, dtype=torch.float16, device=DEV),       # dtype
               torch.empty(1, 4, 128, 64, dtype=torch.bfloat16, device=DEV).transpose(2, 3),
               torch.empty(1, 4, 64, 128, dtype=torch.bfloat16)]                  # host
    for o in bad_out:
        with pytest.raises(ValueError):
            fwd(q, k, v, causal=True, out=o)
        with pytest.raises(ValueError):
            fwd_rope(q, k, v, *(t.to(DEV) for t in W.rope_tables(64, 128)), causal=True, out=o)
    for l in (torch.empty(B, Hq, Sq - 1, dtype=torch.float32, device=DEV),
              torch.empty(B, Hq, Sq, dtype=torch.bfloat16, device=DEV)):
        with pytest.raises(ValueError):
            fwd(q, k, v, causal=True, lse=l)
    o, lse = fwd(q, k, v, causal=True)
    dout = torch.zeros_like(q)
    for kw in ({"dq": torch.empty_like(k)}, {"dk": torch.empty_like(q)},
               {"dv": torch.empty(1, 2, 64, 128, dtype=torch.float32, device=DEV)},
               {"workspace": torch.empty(64, dtype=torch.uint8)}):
        with pytest.raises(ValueError):
            bwd(q, k, v, o, lse, dout, causal=True, **kw)
    with pytest.raises(ValueError):
        fwd_rope(q, k, v, *(t.to(DEV) for t in W.rope_tables(64, 128)), causal=True,
                 k_rot=torch.empty_like(q))
    qd = q[:, :, :1].contiguous()
    with pytest.raises(ValueError):
        fwd_decode(qd, k, v, out=torch.empty_like(q))
    torch.cuda.synchronize()


PAD = 4096


def _window(n, dtype):
    """A length-n view into a NaN-filled buffer with PAD canary elements on both sides."""
    big = torch.full((n + 2 * PAD,), float("nan"), dtype=dtype, device=DEV)
    return big, big[PAD:PAD + n]


def _canaries_intact(big, n):
    return bool(torch.all(torch.isnan(big[:PAD]))) and bool(torch.all(torch.isnan(big[PAD + n:])))


def test_bwd_no_writes_outside_outputs_and_workspace():
    """dQ, dK, dV and the workspace (here with fp32 partial sums: 4 query heads per
    K/V head split over 4 workgroups) inside canary-filled buffers; only the windows
    may change, and the gradient windows are fully written."""
    say("case bwd canaries")
    B, Hq, Hkv, Sq, Sk, D = 1, 8, 2, 333, 200, 64
    q, k, v = _inputs("bf16", B, Hq, Hkv, Sq, Sk, D, True, 8)
    o, lse = fwd(q, k, v, causal=True)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(9)).to(q.dtype).to(DEV)
    st, need = attn_bwd_workspace(B, Hq, Hkv, Sq, Sk, D)
    assert st == 0 and need > 3 * B * Hq * Sq * 4      # the split path is taken
    bq, dq = _window(q.numel(), q.dtype)
    bk, dk = _window(k.numel(), k.dtype)
    bv, dv = _window(v.numel(), v.dtype)
    bw = torch.full((need + 2 * PAD,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = bw[PAD:PAD + need]
    bwd(q, k, v, o, lse, do, causal=True, dq=dq.view(q.shape), dk=dk.view(k.shape),
        dv=dv.view(v.shape), workspace=ws)
    torch.cuda.synchronize()
    for big, win in ((bq, dq), (bk, dk), (bv, dv)):
        assert _canaries_intact(big, win.numel())
        assert not torch.any(torch.isnan(win))
    assert torch.all(bw[:PAD] == 0xA5) and torch.all(bw[PAD + need:] == 0xA5)


def test_decode_no_writes_outside_outputs_and_workspace():
    say("case decode canaries")
    B, Hq, Hkv, Sq, Sk, D = 3, 8, 2, 1, 1000, 128
    q, k, v = _inputs("bf16", B, Hq, Hkv, Sq, Sk, D, True, 10)
    st, need = attn_fwd_decode_workspace(B, Hq, Hkv, Sq, Sk, D, 0)
    assert st == 0
    bo, o = _window(q.numel(), q.dtype)
    bl, lse = _window(B * Hq * Sq, torch.float32)
    bw = torch.full((need + 2 * PAD,), 0xA5, dtype=torch.uint8, device=DEV)
    fwd_decode(q, k, v, causal=True, out=o.view(q.shape), lse=lse.view(B, Hq, Sq),
               workspace=bw[PAD:PAD + need])
    torch.cuda.synchronize()
    assert _canaries_intact(bo, o.numel()) and _canaries_intact(bl, lse.numel())
    assert not torch.any(torch.isnan(o)) and not torch.any(torch.isnan(lse))
    assert torch.all(bw[:PAD] == 0xA5) and torch.all(bw[PAD + need:] == 0xA5)


def test_rope_no_writes_outside_outputs():
    say("case rope canaries")
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 2, 300, 300, 128
    q, k, v = _inputs("bf16", B, Hq, Hkv, Sq, Sk, D, True, 11)
    ct, stab = (t.to(DEV) for t in W.rope_tables(Sk, D))
    bo, o = _window(q.numel(), q.dtype)
    bl, lse = _window(B * Hq * Sq, torch.float32)
    bk, kr = _window(k.numel(), k.dtype)
    fwd_rope(q, k, v, ct, stab, causal=True, out=o.view(q.shape), lse=lse.view(B, Hq, Sq),
             k_rot=kr.view(k.shape))
    torch.cuda.synchronize()
    for big, win in ((bo, o), (bl, lse), (bk, kr)):
        assert _canaries_intact(big, win.numel())
        assert not torch.any(torch.isnan(win))
