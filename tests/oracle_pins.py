"""Pins for the fp64 oracle: facts fixed by the mathematics, not by the oracle.

Every function takes an `OracleLib` and raises AssertionError when the oracle
disagrees with the fact it checks.  `test_oracle_pins.py` runs them against the
real oracle; `test_oracle_mutants.py` runs them against deliberately broken
copies of the oracle (built on the CPU) and requires each copy to fail at least
one pin.  Together they show the pins can see a dropped term, a wrong sign or
index, or a transposed operand.

What the oracle follows: the multi-head scaled dot-product attention of Equ. 1
on the page "A Thread-Register Decoupled GPU Execution Model for Efficient
Tensor Computation" (introduction); the readings for grouped heads and for the
causal mask are stated in `oracle/attn_oracle.c`.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


# ----------------------------------------------------------------------------
# 1. Brute force at 50 significant digits on tiny inputs.
#    Visibility is written from positions: the Sq queries are the last Sq of the
#    Sk positions, and a query sees every key at or before its own position.
#    The softmax is taken without any max-subtraction (Decimal has the range),
#    so the oracle's stabilised two-pass form is checked against the raw one.
# ----------------------------------------------------------------------------
def _brute_decimal(q, k, v, scale, causal):
    getcontext().prec = 50
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    per_kv = Hq // Hkv
    o = np.zeros((B, Hq, Sq, D))
    lse = np.zeros((B, Hq, Sq))
    dscale = Decimal(scale)
    for b in range(B):
        for h in range(Hq):
            kh = h // per_kv
            for i in range(Sq):
                qpos = (Sk - Sq) + i
                vis = [j for j in range(Sk) if (not causal) or j <= qpos]
                if not vis:
                    lse[b, h, i] = -math.inf
                    continue
                e = []
                for j in vis:
                    dot = sum(Decimal(q[b, h, i, d]) * Decimal(k[b, kh, j, d]) for d in range(D))
                    e.append((dscale * dot).exp())
                z = sum(e)
                for d in range(D):
                    num = sum(ej * Decimal(v[b, kh, j, d]) for ej, j in zip(e, vis))
                    o[b, h, i, d] = float(num / z)
                lse[b, h, i] = float(z.ln())
    return o, lse


BRUTE_SHAPES = [
    # (B, Hq, Hkv, Sq, Sk, D, causal)
    (1, 1, 1, 5, 5, 3, False),
    (1, 1, 1, 5, 5, 3, True),
    (2, 4, 2, 4, 7, 3, True),    # fewer queries than keys, grouped heads
    (1, 2, 1, 7, 4, 2, True),    # more queries than keys: leading rows see nothing
    (2, 3, 3, 3, 6, 4, False),
    (1, 4, 1, 6, 6, 5, True),    # one key/value head for all query heads
]


def pin_bruteforce_decimal(orc):
    for n, (B, Hq, Hkv, Sq, Sk, D, causal) in enumerate(BRUTE_SHAPES):
        rng = _rng(100 + n)
        q = _rand(rng, (B, Hq, Sq, D), 1.5)
        k = _rand(rng, (B, Hkv, Sk, D), 1.5)
        v = _rand(rng, (B, Hkv, Sk, D))
        scale = 1.0 / math.sqrt(D) * (1.0 + 0.1 * n)
        o, lse = orc.attn_fwd(q, k, v, causal=causal, scale=scale)
        ob, lb = _brute_decimal(q, k, v, scale, causal)
        assert np.allclose(o, ob, rtol=0, atol=1e-12), ("brute O", n, np.abs(o - ob).max())
        fin = np.isfinite(lb)
        assert np.array_equal(np.isfinite(lse), fin), ("brute LSE finiteness", n)
        assert np.all(lse[~fin] == -math.inf), ("empty rows LSE", n)
        assert np.allclose(lse[fin], lb[fin], rtol=0, atol=1e-12), ("brute LSE", n)


# ----------------------------------------------------------------------------
# 2. Hand-derived worked examples (tests/golden/hand_examples.json).
# ----------------------------------------------------------------------------
def pin_hand_examples(orc):
    with open(GOLDEN) as f:
        data = json.load(f)
    for ex in data["examples"]:
        B, Hq, Hkv, Sq, Sk, D = (ex[x] for x in ("B", "Hq", "Hkv", "Sq", "Sk", "D"))
        q = np.array(ex["q"], dtype=np.float64).reshape(B, Hq, Sq, D)
        k = np.array(ex["k"], dtype=np.float64).reshape(B, Hkv, Sk, D)
        v = np.array(ex["v"], dtype=np.float64).reshape(B, Hkv, Sk, D)
        o_ref = np.array(ex["o"], dtype=np.float64).reshape(B, Hq, Sq, D)
        lse_ref = np.array([float(x) for x in ex["lse"]], dtype=np.float64).reshape(B, Hq, Sq)
        o, lse = orc.attn_fwd(q, k, v, causal=ex["causal"], scale=ex["scale"])
        assert np.allclose(o, o_ref, rtol=0, atol=1e-12), (ex["name"], o, o_ref)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse), fin), (ex["name"], lse, lse_ref)
        assert np.all(lse[~fin] == -math.inf), (ex["name"], lse)
        assert np.allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12), (ex["name"], lse, lse_ref)


# ----------------------------------------------------------------------------
# 3. Closed forms on random inputs.
# ----------------------------------------------------------------------------
def pin_constant_values(orc):
    """Softmax weights sum to one: V rows all equal c gives O = c exactly-ish."""
    rng = _rng(7)
    for causal in (False, True):
        B, Hq, Hkv, S, D = 2, 4, 2, 37, 16
        q = _rand(rng, (B, Hq, S, D), 2.0)
        k = _rand(rng, (B, Hkv, S, D), 2.0)
        c = _rand(rng, (B, Hkv, 1, D))
        v = np.broadcast_to(c, (B, Hkv, S, D)).copy()
        o, _ = orc.attn_fwd(q, k, v, causal=causal)
        expect = np.repeat(c, Hq // Hkv, axis=1)[:, :, 0, :][:, :, None, :]
        assert np.allclose(o, np.broadcast_to(expect, o.shape), rtol=0, atol=1e-13)
        ones = np.ones_like(v)
        o1, _ = orc.attn_fwd(q, k, ones, causal=causal)
        assert np.allclose(o1, 1.0, rtol=0, atol=1e-14)


def pin_uniform_attention(orc):
    """Q = 0: every score is 0, so O_i is the plain mean of V over the visible
    keys and LSE_i = ln(number of visible keys)."""
    rng = _rng(8)
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 1, 9, 13, 6
    q = np.zeros((B, Hq, Sq, D))
    k = _rand(rng, (B, Hkv, Sk, D), 3.0)
    v = _rand(rng, (B, Hkv, Sk, D))
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, causal=causal)
        for i in range(Sq):
            n = (i + Sk - Sq + 1) if causal else Sk
            mean = v[0, 0, :n, :].mean(axis=0)
            for h in range(Hq):
                assert np.allclose(o[0, h, i], mean, rtol=0, atol=1e-13), (causal, i)
                assert abs(lse[0, h, i] - math.log(n)) < 1e-13, (causal, i)


def pin_causal_boundary_rows(orc):
    """Causal with Sq = Sk: row 0 sees only key 0 (O_0 = V_0, LSE_0 = scale q0.k0);
    the last row sees every key, so it equals the non-causal result."""
    rng = _rng(9)
    B, H, S, D = 2, 3, 23, 8
    q = _rand(rng, (B, H, S, D), 2.0)
    k = _rand(rng, (B, H, S, D), 2.0)
    v = _rand(rng, (B, H, S, D))
    scale = 0.3
    oc, lc = orc.attn_fwd(q, k, v, causal=True, scale=scale)
    on, ln_ = orc.attn_fwd(q, k, v, causal=False, scale=scale)
    assert np.allclose(oc[:, :, 0], v[:, :, 0], rtol=0, atol=1e-14)
    assert np.allclose(lc[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                       rtol=0, atol=1e-13)
    assert np.allclose(oc[:, :, -1], on[:, :, -1], rtol=0, atol=1e-13)
    assert np.allclose(lc[:, :, -1], ln_[:, :, -1], rtol=0, atol=1e-13)
    # row 1 sees exactly keys 0 and 1: a two-term softmax written out
    s0 = scale * np.einsum("bhd,bhd->bh", q[:, :, 1], k[:, :, 0])
    s1 = scale * np.einsum("bhd,bhd->bh", q[:, :, 1], k[:, :, 1])
    w1 = 1.0 / (1.0 + np.exp(s0 - s1))
    o1 = (1 - w1)[..., None] * v[:, :, 0] + w1[..., None] * v[:, :, 1]
    assert np.allclose(oc[:, :, 1], o1, rtol=0, atol=1e-13)


def pin_empty_rows(orc):
    """Causal with Sq > Sk: the first Sq - Sk rows see no key: O = 0, LSE = -inf;
    the next row sees key 0 only."""
    rng = _rng(10)
    B, H, Sq, Sk, D = 1, 2, 11, 4, 5
    q = _rand(rng, (B, H, Sq, D))
    k = _rand(rng, (B, H, Sk, D))
    v = _rand(rng, (B, H, Sk, D))
    o, lse = orc.attn_fwd(q, k, v, causal=True)
    e = Sq - Sk
    assert np.all(o[:, :, :e] == 0.0)
    assert np.all(lse[:, :, :e] == -math.inf)
    assert np.all(np.isfinite(lse[:, :, e:]))
    assert np.allclose(o[:, :, e], v[:, :, 0], rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# 4. Invariants.
# ----------------------------------------------------------------------------
def pin_shift_invariance(orc):
    """K' = K + 1 u^T adds scale*(q.u) to every score of a row: O is unchanged
    and LSE shifts by scale*(q.u)."""
    rng = _rng(11)
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 2, 10, 14, 7
    q = _rand(rng, (B, Hq, Sq, D))
    k = _rand(rng, (B, Hkv, Sk, D))
    v = _rand(rng, (B, Hkv, Sk, D))
    u = _rand(rng, (D,))
    scale = 0.4
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, causal=causal, scale=scale)
        o2, lse2 = orc.attn_fwd(q, k + u, v, causal=causal, scale=scale)
        assert np.allclose(o2, o, rtol=0, atol=1e-12)
        assert np.allclose(lse2, lse + scale * (q @ u), rtol=0, atol=1e-12)


def pin_permutation(orc):
    """Non-causal: permuting the key/value rows together leaves O and LSE
    unchanged; permuting the query rows permutes O and LSE."""
    rng = _rng(12)
    B, Hq, Hkv, Sq, Sk, D = 2, 2, 1, 8, 12, 6
    q = _rand(rng, (B, Hq, Sq, D))
    k = _rand(rng, (B, Hkv, Sk, D))
    v = _rand(rng, (B, Hkv, Sk, D))
    o, lse = orc.attn_fwd(q, k, v)
    pk = rng.permutation(Sk)
    o2, lse2 = orc.attn_fwd(q, k[:, :, pk], v[:, :, pk])
    assert np.allclose(o2, o, rtol=0, atol=1e-13)
    assert np.allclose(lse2, lse, rtol=0, atol=1e-13)
    pq = rng.permutation(Sq)
    o3, lse3 = orc.attn_fwd(q[:, :, pq], k, v)
    assert np.allclose(o3, o[:, :, pq], rtol=0, atol=1e-13)
    assert np.allclose(lse3, lse[:, :, pq], rtol=0, atol=1e-13)


def pin_scale_folding(orc):
    """attn(Q, scale = s) equals attn(s Q, scale = 1); s a power of two keeps
    s Q exact."""
    rng = _rng(13)
    B, H, S, D = 1, 2, 17, 8
    q = _rand(rng, (B, H, S, D))
    k = _rand(rng, (B, H, S, D))
    v = _rand(rng, (B, H, S, D))
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, causal=causal, scale=0.25)
        o2, lse2 = orc.attn_fwd(q * 0.25, k, v, causal=causal, scale=1.0)
        assert np.allclose(o, o2, rtol=0, atol=1e-14)
        assert np.allclose(lse, lse2, rtol=0, atol=1e-14)
        o3, _ = orc.attn_fwd(q, k, v, causal=causal, scale=0.5)
        assert not np.allclose(o, o3, rtol=0, atol=1e-6)


def pin_grouped_heads(orc):
    """Grouped heads equal plain multi-head attention on K/V heads repeated
    Hq/Hkv times consecutively (the consecutive-group reading)."""
    rng = _rng(14)
    B, Hq, Hkv, S, D = 2, 6, 2, 11, 4
    q = _rand(rng, (B, Hq, S, D))
    k = _rand(rng, (B, Hkv, S, D))
    v = _rand(rng, (B, Hkv, S, D))
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, causal=causal)
        kr = np.repeat(k, Hq // Hkv, axis=1)
        vr = np.repeat(v, Hq // Hkv, axis=1)
        o2, lse2 = orc.attn_fwd(q, kr, vr, causal=causal)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
        # and the repetition really matters: head 0 differs from head Hq-1's source
        o3, _ = orc.attn_fwd(q, k[:, ::-1].copy(), v[:, ::-1].copy(), causal=causal)
        assert not np.allclose(o3, o, atol=1e-6)


def pin_peaky_limit(orc):
    """K_j = alpha * Q_i with alpha large makes key j dominate row i: O_i -> V_j
    (one-hot softmax) and LSE_i -> alpha*scale*|q_i|^2."""
    rng = _rng(15)
    B, H, S, D = 1, 1, 6, 4
    q = _rand(rng, (B, H, S, D))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = _rand(rng, (B, H, S, D)) * 0.01
    perm = [3, 0, 5, 1, 4, 2]
    alpha = 2000.0
    for i, j in enumerate(perm):
        k[0, 0, j] = alpha * q[0, 0, i]
    v = _rand(rng, (B, H, S, D))
    o, lse = orc.attn_fwd(q, k, v, scale=1.0)
    for i, j in enumerate(perm):
        assert np.allclose(o[0, 0, i], v[0, 0, j], rtol=0, atol=1e-12), (i, j)
        assert abs(lse[0, 0, i] - alpha) < 1e-9, (i, lse[0, 0, i])


# ----------------------------------------------------------------------------
# 5. Storage types: the oracle's exact widening of bf16 / fp16 / fp32 inputs
#    agrees with torch's own conversions, including fp16 subnormals, the largest
#    finite values and signed zeros.
# ----------------------------------------------------------------------------
def pin_storage_widening(orc):
    g = torch.Generator().manual_seed(16)
    x = torch.randn(4096, generator=g) * 30
    specials = torch.tensor([0.0, -0.0, 1.0, -1.0, 65504.0, -65504.0, 6.1e-5, 5.96e-8,
                             -5.96e-8, 3.0e-6, 1e-7, 3.3895e38, 1.2e-38, 9.2e-41])
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        y = torch.cat([x, specials]).to(dt)
        w = orc.widen(y)
        ref = y.to(torch.float64).numpy()
        assert np.array_equal(np.signbit(w), np.signbit(ref)), dt
        assert np.array_equal(w, ref), dt
    # and through the attention path: bf16 inputs give the fp64 result of their
    # widened values
    q = (torch.randn(1, 2, 9, 8, generator=g)).to(torch.bfloat16)
    k = (torch.randn(1, 1, 12, 8, generator=g)).to(torch.bfloat16)
    v = (torch.randn(1, 1, 12, 8, generator=g)).to(torch.bfloat16)
    o, lse = orc.attn_fwd(q, k, v, causal=True)
    o2, lse2 = orc.attn_fwd(q.double(), k.double(), v.double(), causal=True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    qh, kh, vh = (t.to(torch.float16) for t in (q, k, v))
    o3, _ = orc.attn_fwd(qh, kh, vh, causal=True)
    o4, _ = orc.attn_fwd(qh.double(), kh.double(), vh.double(), causal=True)
    assert np.array_equal(o3, o4)


# ----------------------------------------------------------------------------
# 6. An independent library routine: torch's CPU scaled_dot_product_attention
#    (math path) in fp64, with the bottom-right causal mask given explicitly.
# ----------------------------------------------------------------------------
SDPA_SHAPES = [
    # (B, Hq, Hkv, Sq, Sk, D, causal)
    (1, 2, 2, 128, 128, 64, False),
    (2, 4, 1, 96, 160, 32, True),
    (1, 8, 2, 200, 200, 128, True),
    (1, 3, 3, 150, 70, 16, True),
]


def pin_torch_sdpa(orc):
    import torch.nn.functional as F
    g = torch.Generator().manual_seed(17)
    for (B, Hq, Hkv, Sq, Sk, D, causal) in SDPA_SHAPES:
        q = torch.randn(B, Hq, Sq, D, generator=g, dtype=torch.float64) * 1.5
        k = torch.randn(B, Hkv, Sk, D, generator=g, dtype=torch.float64) * 1.5
        v = torch.randn(B, Hkv, Sk, D, generator=g, dtype=torch.float64)
        scale = 1.0 / math.sqrt(D)
        mask = None
        if causal:
            mask = torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=Sk - Sq)
        ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale,
                                             enable_gqa=(Hq != Hkv))
        scores = (q @ torch.repeat_interleave(k, Hq // Hkv, dim=1).transpose(-1, -2)) * scale
        if mask is not None:
            scores = scores.masked_fill(~mask, -math.inf)
        lse_ref = torch.logsumexp(scores, dim=-1)
        o, lse = orc.attn_fwd(q, k, v, causal=causal, scale=scale)
        live = torch.isfinite(lse_ref).numpy()
        assert np.allclose(o[live], ref.numpy()[live], rtol=0, atol=1e-12), (B, Hq, Sq, Sk)
        assert np.allclose(lse[live], lse_ref.numpy()[live], rtol=0, atol=1e-12)
        assert np.all(o[~live] == 0.0) and np.all(lse[~live] == -math.inf)


# ----------------------------------------------------------------------------
# 7. Row selection: computing a list of rows one by one gives the same values
#    as the full pass (the full-size GPU tests rely on it).
# ----------------------------------------------------------------------------
def pin_row_subset(orc):
    rng = _rng(18)
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 33, 41, 8
    q = _rand(rng, (B, Hq, Sq, D))
    k = _rand(rng, (B, Hkv, Sk, D))
    v = _rand(rng, (B, Hkv, Sk, D))
    o, lse = orc.attn_fwd(q, k, v, causal=True)
    rows = rng.integers(0, B * Hq * Sq, size=50)
    o_r, lse_r = orc.attn_fwd(q, k, v, causal=True, rows=rows)
    assert np.array_equal(o_r, o.reshape(-1, D)[rows])
    assert np.array_equal(lse_r, lse.reshape(-1)[rows])


# ----------------------------------------------------------------------------
# 8. Gradients (the backward the FIBER page evaluates as its training workload).
#    Central differences of the forward oracle -- itself pinned above -- fix every
#    gradient on tiny fp64 inputs (causal and not, grouped heads, Sq != Sk with
#    key-less rows, negative scales); a second library's automatic
#    differentiation and three exact special cases pin them at larger shapes.
# ----------------------------------------------------------------------------
BWD_FD_SHAPES = [
    (1, 1, 1, 4, 4, 3, False, 0.7),
    (1, 2, 1, 5, 6, 4, True, 0.9),      # grouped heads, fewer queries than keys
    (2, 2, 2, 6, 3, 2, True, -0.5),     # more queries than keys: rows without keys
    (1, 4, 2, 3, 5, 3, False, 1.3),
]


def pin_bwd_finite_differences(orc):
    rng = _rng(404)
    h = 1e-6
    for (B, Hq, Hkv, Sq, Sk, D, causal, scale) in BWD_FD_SHAPES:
        q = _rand(rng, (B, Hq, Sq, D))
        k = _rand(rng, (B, Hkv, Sk, D))
        v = _rand(rng, (B, Hkv, Sk, D))
        g = _rand(rng, (B, Hq, Sq, D))
        dq, dk, dv = orc.attn_bwd(q, k, v, g, causal=causal, scale=scale)

        def loss(qq, kk, vv):
            o, _ = orc.attn_fwd(qq, kk, vv, causal=causal, scale=scale)
            return float((o * g).sum())

        for which, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[which]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[which]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            err = np.abs(num - grad).max()
            assert err < 1e-6 * max(1.0, np.abs(num).max()), (which, B, Hq, Hkv, Sq, Sk, err)


def pin_bwd_special_cases(orc):
    """Exact facts: (a) Q = 0 gives uniform weights, so dk = 0 and dv_j is the sum of
    dO_i / |J_i| over the queries that see key j; (b) identical V rows make every
    dP_ij of a row equal, so dS = 0 and dq = dk = 0; (c) the weights of a row sum
    to one, so sum_j dv_j = sum of dO over rows that see any key."""
    rng = _rng(405)
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 1, 5, 7, 3
    k = _rand(rng, (B, Hkv, Sk, D))
    v = _rand(rng, (B, Hkv, Sk, D))
    g = _rand(rng, (B, Hq, Sq, D))
    q0 = np.zeros((B, Hq, Sq, D))
    for causal in (False, True):
        dq, dk, dv = orc.attn_bwd(q0, k, v, g, causal=causal, scale=0.8)
        assert np.all(dk == 0.0)
        want = np.zeros((B, Hkv, Sk, D))
        for h in range(Hq):
            for i in range(Sq):
                last = min(Sk - 1, i + Sk - Sq) if causal else Sk - 1
                for j in range(last + 1):
                    want[0, 0, j] += g[0, h, i] / (last + 1)
        assert np.allclose(dv, want, rtol=0, atol=1e-13)
        q = _rand(rng, (B, Hq, Sq, D))
        vc = np.broadcast_to(_rand(rng, (1, 1, 1, D)), v.shape).copy()
        dq, dk, dv = orc.attn_bwd(q, k, vc, g, causal=causal, scale=0.8)
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
        dq, dk, dv = orc.attn_bwd(q, k, v, g, causal=causal, scale=0.8)
        assert np.allclose(dv.sum(axis=2)[0, 0], g[0].sum(axis=(0, 1)), rtol=0, atol=1e-12)


def pin_bwd_torch_autograd(orc):
    """fp64 automatic differentiation of an explicit softmax attention in torch."""
    g0 = torch.Generator().manual_seed(406)
    for (B, Hq, Hkv, Sq, Sk, D, causal) in [(1, 2, 2, 40, 40, 16, True), (2, 4, 1, 24, 50, 8, True),
                                           (1, 3, 3, 30, 20, 16, False)]:
        q = (torch.randn(B, Hq, Sq, D, generator=g0, dtype=torch.float64) * 1.5).requires_grad_()
        k = (torch.randn(B, Hkv, Sk, D, generator=g0, dtype=torch.float64) * 1.5).requires_grad_()
        v = torch.randn(B, Hkv, Sk, D, generator=g0, dtype=torch.float64).requires_grad_()
        go = torch.randn(B, Hq, Sq, D, generator=g0, dtype=torch.float64)
        scale = 1.0 / math.sqrt(D)
        kk = torch.repeat_interleave(k, Hq // Hkv, dim=1)
        vv = torch.repeat_interleave(v, Hq // Hkv, dim=1)
        scores = (q @ kk.transpose(-1, -2)) * scale
        if causal:
            mask = torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=Sk - Sq)
            scores = scores.masked_fill(~mask, -math.inf)
        w = torch.softmax(scores, dim=-1).nan_to_num(0.0)
        (w @ vv).backward(go)
        dq, dk, dv = orc.attn_bwd(q.detach(), k.detach(), v.detach(), go, causal=causal, scale=scale)
        for mine, ref in ((dq, q.grad), (dk, k.grad), (dv, v.grad)):
            assert np.allclose(mine, ref.numpy(), rtol=0, atol=1e-11), (B, Hq, Hkv, Sq, Sk)


# ----------------------------------------------------------------------------
# 8. Rotary position embedding.  The rotation of a feature pair by a tabulated
#    (cos, sin) is the product of two complex numbers; the rounding into the
#    storage type is checked against independent roundings; the rotation's
#    defining property -- dot products of rotated rows depend only on the
#    difference of their positions -- is checked on unrounded values.
# ----------------------------------------------------------------------------
def _angles_tables(P, D, base=10000.0):
    ang = np.arange(P, dtype=np.float64)[:, None] * base ** (-np.arange(D // 2) * 2.0 / D)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _interleave_perm(D):
    """perm[j] = feature of the split-halves layout that sits at feature j of the
    interleaved layout: pair i is (i, i + D/2) there and (2i, 2i+1) here."""
    half = D // 2
    perm = np.empty(D, dtype=np.int64)
    perm[0::2] = np.arange(half)
    perm[1::2] = np.arange(half) + half
    return perm


def pin_rope_complex_product(orc):
    """Interleaved pairs (a, b) at position p become (a + ib)(c_p + i s_p) exactly
    (the products are exact in fp64); the split-halves layout is the interleaved
    one on permuted features; row s of a head reads table row s + pos_offset."""
    g = torch.Generator().manual_seed(801)
    rng = _rng(802)
    for dt in (torch.bfloat16, torch.float16):
        B, H, S, D, off = 2, 3, 7, 8, 5
        x = torch.randn(B, H, S, D, generator=g).to(dt)
        # arbitrary (not unit) tables make every entry count
        ct = rng.standard_normal((S + off + 2, D // 2)).astype(np.float32)
        st = rng.standard_normal((S + off + 2, D // 2)).astype(np.float32)
        f1, t1 = orc.rope(x, ct, st, 1, pos_offset=off)
        xd = x.double().numpy()
        z = (xd[..., 0::2] + 1j * xd[..., 1::2]) * (ct[off:off + S].astype(np.float64)
                                                    + 1j * st[off:off + S].astype(np.float64))
        assert np.array_equal(f1[..., 0::2], z.real) and np.array_equal(f1[..., 1::2], z.imag), dt
        # the storage output is the fp64 result rounded once
        name = "bf16" if dt == torch.bfloat16 else "fp16"
        assert np.array_equal(t1.view(torch.int16).numpy().view(np.uint16), orc.round16(f1, name)), dt
        perm = _interleave_perm(D)
        f2, t2 = orc.rope(x, ct, st, 2, pos_offset=off)
        fp, tp = orc.rope(x[..., perm].contiguous(), ct, st, 1, pos_offset=off)
        inv = np.argsort(perm)
        assert np.array_equal(f2, fp[..., inv]), dt
        assert torch.equal(t2.view(torch.int16), tp[..., inv].contiguous().view(torch.int16)), dt


def pin_rope_exact_rotations(orc):
    """Angle 0 is the identity, a quarter turn maps (a, b) to (-b, a) and a half
    turn negates: all exact, in both layouts, after rounding."""
    g = torch.Generator().manual_seed(803)
    for dt in (torch.bfloat16, torch.float16):
        x = torch.randn(1, 2, 4, 16, generator=g).to(dt)
        P = 4
        ones, zeros = np.ones((P, 8), np.float32), np.zeros((P, 8), np.float32)
        for layout in (1, 2):
            perm = _interleave_perm(16) if layout == 2 else np.arange(16)
            _, t = orc.rope(x, ones, zeros, layout)
            assert torch.equal(t.view(torch.int16), x.view(torch.int16)), (dt, layout)
            _, t = orc.rope(x, -ones, zeros, layout)
            assert torch.equal(t.double(), -x.double()), (dt, layout)
            _, t = orc.rope(x, zeros, ones, layout)
            xp, tp = x[..., perm].double(), t[..., perm].double()
            assert torch.equal(tp[..., 0::2], -xp[..., 1::2]), (dt, layout)
            assert torch.equal(tp[..., 1::2], xp[..., 0::2]), (dt, layout)


def pin_rope_relative_position(orc):
    """With the frequency tables of the rotary embedding, the dot product of a
    query rotated at position m with a key rotated at position n depends only on
    m - n, and rotation keeps each row's norm (up to the fp32 tables' rounding)."""
    g = torch.Generator().manual_seed(804)
    D, P = 64, 300
    ct, st = _angles_tables(P, D)
    q = torch.randn(1, 1, 1, D, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 1, 1, D, generator=g).to(torch.bfloat16)
    for layout in (1, 2):
        def dot(m, n):
            fq, _ = orc.rope(q, ct, st, layout, pos_offset=m)
            fk, _ = orc.rope(k, ct, st, layout, pos_offset=n)
            return float((fq * fk).sum())
        for m, n, t in ((3, 1, 100), (50, 70, 200), (0, 0, 299), (200, 10, 50)):
            a, b = dot(m, n), dot(m + t, n + t)
            assert abs(a - b) <= 1e-5 * (1 + abs(a)), (layout, m, n, t, a, b)
        assert abs(dot(7, 0) - dot(0, 7)) > 1e-3      # the sign of m - n matters
        fq, _ = orc.rope(q, ct, st, layout, pos_offset=123)
        nq = float((q.double() ** 2).sum())
        assert abs(float((fq ** 2).sum()) - nq) <= 1e-6 * nq, layout


def _nearest_even_bf16(v):
    """Nearest bf16 to v (ties to an even bit pattern) by searching the bit
    patterns around v's binary32 rounding, decoding each one exactly."""
    f = np.array([v], dtype=np.float64).astype(np.float32)
    top = int(f.view(np.uint32)[0]) >> 16
    best = None
    for cand in range(max(0, (top & 0x7fff) - 2), (top & 0x7fff) + 3):
        for c in (cand, cand | 0x8000):
            val = float(np.array([c << 16], dtype=np.uint32).view(np.float32)[0])
            if not math.isfinite(val):
                continue
            # nearest, then an even last bit, then the sign of v for zeros
            key = (abs(val - v), c & 1, (c >> 15) != (1 if math.copysign(1.0, v) < 0 else 0))
            if best is None or key < best[0]:
                best = (key, c)
    return best[1]


def pin_round16(orc):
    """Rounding fp64 into the storage types: fp16 agrees with numpy's correctly
    rounded float64 -> float16 conversion (normal, subnormal, ties, overflow);
    bf16 agrees with a nearest-even search over decoded neighbours."""
    rng = _rng(805)
    ulp_ties = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -24 * 0.5, 2.0 ** -24 * 1.5,
                         65504.0 + 16.0, 65504.0 + 15.9, -(1.0 + 2.0 ** -11), 2.0 ** -14 * (1 - 2.0 ** -11)])
    x = np.concatenate([rng.standard_normal(20000) * 3, rng.standard_normal(2000) * 1e-6,
                        rng.standard_normal(2000) * 3e4, ulp_ties, [0.0, -0.0, 1e6, -1e6]])
    got = orc.round16(x, "fp16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    bt = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40,
                   -(1.0 + 2.0 ** -8), 3.0e-39, 2.0 ** -133 * 1.5, 2.0 ** -133 * 0.5])
    xb = np.concatenate([rng.standard_normal(3000) * 5, rng.standard_normal(300) * 1e-38, bt])
    got = orc.round16(xb, "bf16")
    for v, gb in zip(xb, got):
        assert int(gb) == _nearest_even_bf16(float(v)), (v, hex(int(gb)))


def pin_rope_bottom_right(orc):
    """Attention with the rotary embedding places query i at position
    i + Sk - Sq: the last Sq query rows of a square causal problem give the same
    outputs as the problem with only those queries."""
    g = torch.Generator().manual_seed(806)
    D, Sk, Sq = 16, 11, 3
    ct, st = _angles_tables(Sk, D, base=50.0)
    q = torch.randn(1, 2, Sk, D, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 1, Sk, D, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 1, Sk, D, generator=g).to(torch.bfloat16)
    for layout in (1, 2):
        of, lf, kf = orc.attn_fwd_rope(q, k, v, ct, st, layout, causal=True)
        qs = q[:, :, Sk - Sq:].contiguous()
        os_, ls, ks = orc.attn_fwd_rope(qs, k, v, ct, st, layout, causal=True)
        assert np.array_equal(os_, of[:, :, Sk - Sq:]) and np.array_equal(ls, lf[:, :, Sk - Sq:])
        assert torch.equal(kf.view(torch.int16), ks.view(torch.int16))
        # and it is attention of the rotated tensors: row 0 of the square problem
        # sees key 0 only, whose rotation at position 0 is the identity
        assert abs(lf[0, 0, 0] - float((q[0, 0, 0].double() * k[0, 0, 0].double()).sum()) / 4.0) < 1e-12


ALL_PINS = [
    pin_bruteforce_decimal,
    pin_hand_examples,
    pin_constant_values,
    pin_uniform_attention,
    pin_causal_boundary_rows,
    pin_empty_rows,
    pin_shift_invariance,
    pin_permutation,
    pin_scale_folding,
    pin_grouped_heads,
    pin_peaky_limit,
    pin_storage_widening,
    pin_torch_sdpa,
    pin_row_subset,
    pin_bwd_finite_differences,
    pin_bwd_special_cases,
    pin_bwd_torch_autograd,
    pin_rope_complex_product,
    pin_rope_exact_rotations,
    pin_rope_relative_position,
    pin_round16,
    pin_rope_bottom_right,
]
