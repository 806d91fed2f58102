"""Parity of the HIP path with the fp64 oracle, element by element (GPU).

Small and ragged shapes, the five named workloads and the attention variants
at full size compare every output element (O and LSE); the million-key case and
the largest head slice the library accepts (8,384,512 keys of 256 bytes) compare
sampled rows the oracle computes one by one."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from attention_attn_fwd_02_amd import workloads as W
from gpu_helpers import TOL_LSE, TOL_O, check_full, compare, run_gpu, sample_rows, say

pytestmark = pytest.mark.gpu

# (dtype, B, Hq, Hkv, Sq, Sk, D, causal)
SHAPES = [
    ("bf16", 1, 2, 2, 1, 1, 64, False),
    ("bf16", 1, 2, 2, 1, 1, 128, True),
    ("bf16", 1, 1, 1, 17, 17, 128, True),
    ("bf16", 1, 2, 2, 127, 127, 64, False),
    ("bf16", 2, 3, 3, 300, 300, 128, True),      # two query tiles, ragged tail
    ("bf16", 1, 4, 1, 300, 513, 128, True),      # MQA, fewer queries than keys
    ("bf16", 1, 4, 2, 513, 300, 64, True),       # more queries than keys: empty rows
    ("bf16", 1, 8, 2, 1000, 1000, 128, True),    # GQA, several tiles
    ("bf16", 1, 6, 2, 300, 300, 128, True),      # three query heads per K/V head
    ("fp16", 3, 12, 4, 200, 200, 64, False),     # three per K/V head, 12 groups (not a multiple of 8)
    ("bf16", 2, 2, 2, 256, 64, 128, False),
    ("bf16", 1, 2, 2, 64, 700, 64, False),
    ("bf16", 1, 2, 2, 1, 700, 128, True),        # one query against many keys
    ("bf16", 1, 2, 2, 700, 1, 128, True),        # many queries, one key
    ("bf16", 1, 2, 2, 257, 257, 64, True),
    ("fp16", 1, 2, 2, 300, 300, 128, True),
    ("fp16", 1, 4, 2, 190, 260, 64, False),
    ("fp16", 1, 8, 1, 513, 513, 128, True),
    ("fp32", 1, 2, 2, 1, 1, 64, False),
    ("fp32", 1, 2, 2, 300, 300, 128, True),
    ("fp32", 1, 4, 2, 131, 77, 64, True),
    ("fp32", 2, 4, 1, 70, 190, 128, False),
    ("fp32", 1, 2, 1, 200, 333, 64, True),       # keys split between waves, more keys than queries
    ("fp32", 1, 2, 2, 300, 100, 128, True),      # keys split between waves, empty rows
    ("fp32", 2, 32, 8, 512, 512, 64, True),      # 256 tiles of 128 queries: one wave per query block
]


@pytest.mark.parametrize("shape", SHAPES, ids=["%s_b%d_hq%d_hkv%d_sq%d_sk%d_d%d_%s" % (
    s[0], *s[1:7], "causal" if s[7] else "full") for s in SHAPES])
def test_shapes_full_output(shape):
    dt, B, Hq, Hkv, Sq, Sk, D, causal = shape
    w = W.custom(dt, B, Hq, Hkv, Sq, Sk, D, causal, seed=zlib.crc32(repr(shape).encode()) % 100000)
    check_full(w)


def test_small_fp32_workload():
    check_full(W.WORKLOADS["mha_fp32_b1_h2_s128_d64"])


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.5, 2.0, 1e-39])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_other_scales(scale, dt):
    w = W.custom(dt, 1, 2, 1, 200, 333, 128, True, seed=77)
    check_full(w, scale=scale)


def test_no_lse_requested():
    w = W.custom("bf16", 1, 2, 2, 300, 300, 64, True, seed=5)
    check_full(w, want_lse=False)


def test_peaky_small():
    """Q, K with sigma 2 at D = 128: near one-hot rows (as the long-context workload)."""
    w = W.custom("bf16", 1, 2, 2, 1024, 1024, 128, True, seed=1005,
                 q_dist=("normal", 2.0), k_dist=("normal", 2.0))
    check_full(w)


def test_extreme_peaky_small():
    """sigma 4: weights collapse onto one key; O must reproduce that V row."""
    w = W.custom("bf16", 1, 2, 2, 512, 512, 128, False, seed=99,
                 q_dist=("normal", 4.0), k_dist=("normal", 4.0))
    check_full(w)


FULL = [n for n in W.ORDER if n != "mha_fp32_b1_h2_s128_d64"] + list(W.VARIANTS)


@pytest.mark.parametrize("name", FULL)
def test_full_size_whole_output(name):
    """The named workloads and the attention variants (MQA, GQA-8, fp16) at full
    size, in the launch configuration the benchmark times: every element of O and
    of the LSE against the oracle (which runs on all host cores: about 2 s for the
    D = 64 workload, 15 s at S = 4096, 30 s for GQA at S = 8192 and 60 s at
    S = 16384).  Also: rows of O lie inside the range of V (convex mixes)."""
    w = W.lookup(name)
    say("case", name, "(full size, every element)")
    q, k, v = W.make_inputs(w)
    o, lse = run_gpu(q, k, v, w.causal, scale=w.scale)
    assert torch.isfinite(o).all(), "non-finite O"
    assert torch.isfinite(lse).all(), "non-finite LSE"
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=w.causal, scale=w.scale)
    e = compare(o, lse, o_ref, lse_ref, w.dtype, name)
    say("  %s: every element, max|dO| %.4g  max|dLSE| %.4g" % (name, *e))
    vmin = v.to(torch.float32).amin().item()
    vmax = v.to(torch.float32).amax().item()
    of = o.to(torch.float32)
    assert of.amin().item() >= vmin - TOL_O[w.dtype] and of.amax().item() <= vmax + TOL_O[w.dtype]


def test_long_context_large_offsets():
    """About a million keys per K/V head (K and V 256 MiB each, byte offsets near
    2^28 inside a head, 15,626 key tiles per workgroup and a ragged last one): the
    prefill kernel on sampled rows, and split-KV decoding of the last query row,
    against the oracle."""
    from attention_attn_fwd_02_amd import fwd, fwd_decode
    w = W.custom("bf16", 1, 2, 1, 256, 1_000_003, 128, True, seed=4242)
    say("case", w.name)
    q, k, v = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o, lse = fwd(qd, kd, vd, causal=True)
    o1, l1 = fwd_decode(qd[:, :, -1:].contiguous(), kd, vd, causal=True)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 63, 64, 127, 128, 255, 256, 300, 511}
                           | set(np.random.default_rng(5).integers(0, 512, 22).tolist())))
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=True, rows=rows)
    og = o.reshape(-1, w.D)[torch.from_numpy(rows)].cpu()
    lg = lse.reshape(-1)[torch.from_numpy(rows)].cpu()
    e = compare(og, lg, o_ref, lse_ref, "bf16", w.name)
    say("  prefill, %d rows: max|dO| %.3g  max|dLSE| %.3g" % ((len(rows),) + e))
    last = np.array([255, 511])            # the last query of each head
    o_ref1, lse_ref1 = oracle.attn_fwd(q, k, v, causal=True, rows=last)
    e1 = compare(o1.reshape(-1, w.D).cpu(), l1.reshape(-1).cpu(), o_ref1, lse_ref1, "bf16", w.name)
    say("  decode, last rows: max|dO| %.3g  max|dLSE| %.3g" % e1)


@pytest.mark.parametrize("dtype,D,Sk", [
    ("bf16", 128, ((1 << 31) - (1 << 20)) // 256),    # 8,384,512 keys: K and V 2 GiB - 1 MiB each
    ("fp32", 64, ((1 << 31) - (1 << 20)) // 256),     # the fp32 kernels at the same byte limit
])
def test_largest_head_slice(dtype, D, Sk):
    """The largest K/V head slice the library accepts (2^31 - 2^20 bytes, byte
    offsets up to just below 2^31 inside a head, the out-of-range DMA offsets
    summed with tile offsets near 2^31 without wrapping): causal prefill with the
    queries at the end of the keys, on sampled rows, and split-KV decoding of the
    last row (bf16), against the oracle."""
    from attention_attn_fwd_02_amd import fwd, fwd_decode
    from attention_attn_fwd_02_amd.attn import ATTN_ERR_UNSUPPORTED, AttnError
    w = W.custom(dtype, 1, 1, 1, 130, Sk, D, True, seed=777 + D)
    say("case", w.name)
    q, k, v = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o, lse = fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 65, 127, 128, 129] + [3, 40, 77, 100, 111, 120, 125, 126])
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=True, rows=rows)
    og = o.reshape(-1, w.D)[torch.from_numpy(rows)].cpu()
    lg = lse.reshape(-1)[torch.from_numpy(rows)].cpu()
    e = compare(og, lg, o_ref, lse_ref, dtype, w.name)
    say("  prefill, %d rows: max|dO| %.3g  max|dLSE| %.3g" % ((len(rows),) + e))
    if dtype != "fp32":
        o1, l1 = fwd_decode(qd[:, :, -1:].contiguous(), kd, vd, causal=True)
        torch.cuda.synchronize()
        last = int(np.flatnonzero(rows == w.Sq - 1)[0])      # the oracle's row of query Sq - 1
        e1 = compare(o1.reshape(-1, w.D).cpu(), l1.reshape(-1).cpu(), o_ref[last:last + 1],
                     lse_ref[last:last + 1], dtype, w.name)
        say("  decode, last row: max|dO| %.3g  max|dLSE| %.3g" % e1)
    # one more key and the head slice no longer fits: refused before any launch
    k1 = torch.empty((1, 1, Sk + 1, D), dtype=kd.dtype, device=dev)
    with pytest.raises(AttnError) as ei:
        fwd(qd, k1, k1, causal=True)
    assert ei.value.status == ATTN_ERR_UNSUPPORTED
