"""fp64 CPU oracle for the fused attention forward and its gradients -- TEST
INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  The product path (the HIP library and its
Python binding) never imports it, and this package imports nothing from the
product.

The arithmetic lives in `attn_oracle.c` (plain C, fp64, two-pass softmax per
row; the rotary embedding of Q and K with one rounding into the storage type);
this module only marshals arrays into it (and, for attention with the rotary
embedding, chains the rotation into the forward).  What it computes: the
multi-head scaled dot-product attention of Equ. 1 on the page "A
Thread-Register Decoupled GPU Execution Model for Efficient Tensor Computation"
(introduction), with the readings listed at the top of `attn_oracle.c`.
"""
import ctypes
import math
import os

import numpy as np

from . import build as _build

_DTYPE_CODE = {"bf16": 0, "fp16": 1, "fp32": 2, "fp64": 3}


def _as_raw(x):
    """Return (contiguous numpy array holding the raw storage bits, dtype name).

    Accepts numpy arrays (float16/32/64) and CPU torch tensors (bfloat16,
    float16, float32, float64).  bf16 has no numpy type, so its bits travel as
    uint16 and the C side widens them exactly.
    """
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16), "bf16"
        if x.dtype == torch.float16:
            return x.view(torch.int16).numpy().view(np.uint16), "fp16"
        if x.dtype == torch.float32:
            return x.numpy(), "fp32"
        if x.dtype == torch.float64:
            return x.numpy(), "fp64"
        raise TypeError("oracle: unsupported torch dtype %s" % x.dtype)
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16), "fp16"
    if x.dtype == np.float32:
        return x, "fp32"
    if x.dtype == np.float64:
        return x, "fp64"
    raise TypeError("oracle: unsupported numpy dtype %s" % x.dtype)


class OracleLib:
    """ctypes view of one build of `attn_oracle.c` (the default build, or a
    deliberately broken copy that the mutation tests compile on the CPU)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_attn_rows.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                         f64, i32, vp, i64, vp, vp, i32]
        lib.oracle_attn_rows.restype = i32
        lib.oracle_widen.argtypes = [vp, i32, i64, vp]
        lib.oracle_widen.restype = i32
        lib.oracle_attn_bwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f64,
                                        i32, vp, vp, vp, i32]
        lib.oracle_attn_bwd.restype = i32
        lib.oracle_round16.argtypes = [vp, i32, i64, vp]
        lib.oracle_round16.restype = i32
        lib.oracle_rope.argtypes = [vp, i32, i64, i32, i32, vp, vp, i32, i32, i32, vp, vp]
        lib.oracle_rope.restype = i32
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i32
        self.lib = lib
        self.path = path

    def widen(self, x) -> np.ndarray:
        """Exact fp64 copy of a bf16/fp16/fp32/fp64 array (same shape)."""
        raw, name = _as_raw(x)
        out = np.empty(raw.shape, dtype=np.float64)
        rc = self.lib.oracle_widen(raw.ctypes.data, _DTYPE_CODE[name], raw.size,
                                   out.ctypes.data)
        if rc:
            raise ValueError("oracle_widen failed (%d)" % rc)
        return out

    def round16(self, x, dtype: str) -> np.ndarray:
        """Round an fp64 array to bf16/fp16 (nearest, ties to even); returns the
        storage bit patterns as uint16, same shape."""
        src = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(src.shape, dtype=np.uint16)
        rc = self.lib.oracle_round16(src.ctypes.data, _DTYPE_CODE[dtype], src.size, out.ctypes.data)
        if rc:
            raise ValueError("oracle_round16 failed (%d)" % rc)
        return out

    def rope(self, x, cos, sin, layout, pos_offset=0):
        """Rotary embedding of x ([..., S, D], bf16 or fp16) with fp32 tables
        cos, sin ([P, D/2]); row s of each head at position s + pos_offset.
        layout 1: pairs (2i, 2i+1); layout 2: pairs (i, i + D/2).
        Returns (fp64 rotated values, storage-typed rotated tensor)."""
        import torch
        xr, xn = _as_raw(x)
        if xn not in ("bf16", "fp16"):
            raise TypeError("oracle: rope takes bf16 or fp16")
        S, D = xr.shape[-2], xr.shape[-1]
        nheads = int(np.prod(xr.shape[:-2])) if xr.ndim > 2 else 1
        ct = np.ascontiguousarray(np.asarray(cos, dtype=np.float32))
        st = np.ascontiguousarray(np.asarray(sin, dtype=np.float32))
        if ct.shape != st.shape or ct.ndim != 2 or ct.shape[1] != D // 2:
            raise ValueError("oracle: rope tables must be [P, D/2]")
        f64 = np.empty(xr.shape, dtype=np.float64)
        bits = np.empty(xr.shape, dtype=np.uint16)
        rc = self.lib.oracle_rope(xr.ctypes.data, _DTYPE_CODE[xn], nheads, S, D, ct.ctypes.data,
                                  st.ctypes.data, ct.shape[0], int(pos_offset), int(layout),
                                  f64.ctypes.data, bits.ctypes.data)
        if rc:
            raise ValueError("oracle_rope failed (%d)" % rc)
        tdt = torch.bfloat16 if xn == "bf16" else torch.float16
        return f64, torch.from_numpy(bits.view(np.int16)).view(tdt)

    def attn_fwd_rope(self, q, k, v, cos, sin, layout, causal=False, scale=None, rows=None,
                      nthreads=0):
        """Attention of the rotated, storage-rounded Q and K: query i at position
        i + Sk - Sq, key j at position j.  Returns (o, lse, k_rot) with o, lse as
        `attn_fwd` and k_rot the rotated K in the storage type."""
        Sq, Sk = q.shape[2], k.shape[2]
        _, q_rot = self.rope(q, cos, sin, layout, pos_offset=Sk - Sq)
        _, k_rot = self.rope(k, cos, sin, layout, pos_offset=0)
        o, lse = self.attn_fwd(q_rot, k_rot, v, causal=causal, scale=scale, rows=rows,
                               nthreads=nthreads)
        return o, lse, k_rot

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def attn_fwd(self, q, k, v, causal=False, scale=None, rows=None, nthreads=0):
        """fp64 attention forward.

        q: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D]; all three of one storage dtype.
        rows: None for every query row, else an int array of flat row indices
              r = (b * Hq + h) * Sq + i.
        Returns (o, lse): with rows=None, o is [B, Hq, Sq, D] and lse [B, Hq, Sq];
        otherwise o is [len(rows), D] and lse [len(rows)].  All float64.
        """
        qr, qn = _as_raw(q)
        kr, kn = _as_raw(k)
        vr, vn = _as_raw(v)
        if not (qn == kn == vn):
            raise TypeError("oracle: q, k, v must share one dtype")
        if qr.ndim != 4 or kr.ndim != 4 or vr.ndim != 4:
            raise ValueError("oracle: q, k, v must be 4-D [B, H, S, D]")
        B, Hq, Sq, D = qr.shape
        Bk, Hkv, Sk, Dk = kr.shape
        if (Bk, Dk) != (B, D) or vr.shape != kr.shape:
            raise ValueError("oracle: shape mismatch q%s k%s v%s"
                             % (qr.shape, kr.shape, vr.shape))
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        total = B * Hq * Sq
        if rows is None:
            nrows, rows_ptr = total, None
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
            nrows, rows_ptr = rows_arr.size, rows_arr.ctypes.data
        o = np.empty((nrows, D), dtype=np.float64)
        lse = np.empty((nrows,), dtype=np.float64)
        rc = self.lib.oracle_attn_rows(qr.ctypes.data, kr.ctypes.data, vr.ctypes.data,
                                       _DTYPE_CODE[qn], B, Hq, Hkv, Sq, Sk, D, float(scale),
                                       int(bool(causal)), rows_ptr, nrows,
                                       o.ctypes.data, lse.ctypes.data, int(nthreads))
        if rc:
            raise ValueError("oracle_attn_rows failed (%d)" % rc)
        if rows is None:
            return o.reshape(B, Hq, Sq, D), lse.reshape(B, Hq, Sq)
        return o, lse


    def attn_bwd(self, q, k, v, do, causal=False, scale=None, nthreads=0):
        """fp64 gradients (dq, dk, dv) of the attention forward for output
        gradient `do` (same shape and storage dtype as q)."""
        qr, qn = _as_raw(q)
        kr, kn = _as_raw(k)
        vr, vn = _as_raw(v)
        gr, gn = _as_raw(do)
        if not (qn == kn == vn == gn):
            raise TypeError("oracle: q, k, v, do must share one dtype")
        B, Hq, Sq, D = qr.shape
        Bk, Hkv, Sk, Dk = kr.shape
        if (Bk, Dk) != (B, D) or vr.shape != kr.shape or gr.shape != qr.shape:
            raise ValueError("oracle: shape mismatch")
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        dq = np.empty(qr.shape, dtype=np.float64)
        dk = np.empty(kr.shape, dtype=np.float64)
        dv = np.empty(kr.shape, dtype=np.float64)
        rc = self.lib.oracle_attn_bwd(qr.ctypes.data, kr.ctypes.data, vr.ctypes.data,
                                      gr.ctypes.data, _DTYPE_CODE[qn], B, Hq, Hkv, Sq, Sk, D,
                                      float(scale), int(bool(causal)), dq.ctypes.data,
                                      dk.ctypes.data, dv.ctypes.data, int(nthreads))
        if rc:
            raise ValueError("oracle_attn_bwd failed (%d)" % rc)
        return dq, dk, dv


_default = None


def default() -> OracleLib:
    """The oracle built from `attn_oracle.c` (rebuilt if the source is newer)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _default = OracleLib(_build.LIB)
    return _default


def attn_fwd(q, k, v, causal=False, scale=None, rows=None, nthreads=0):
    return default().attn_fwd(q, k, v, causal=causal, scale=scale, rows=rows,
                              nthreads=nthreads)


def attn_bwd(q, k, v, do, causal=False, scale=None, nthreads=0):
    return default().attn_bwd(q, k, v, do, causal=causal, scale=scale, nthreads=nthreads)


def round16(x, dtype):
    return default().round16(x, dtype)


def rope(x, cos, sin, layout, pos_offset=0):
    return default().rope(x, cos, sin, layout, pos_offset=pos_offset)


def attn_fwd_rope(q, k, v, cos, sin, layout, causal=False, scale=None, rows=None, nthreads=0):
    return default().attn_fwd_rope(q, k, v, cos, sin, layout, causal=causal, scale=scale,
                                   rows=rows, nthreads=nthreads)


def widen(x) -> np.ndarray:
    return default().widen(x)


def max_threads() -> int:
    return default().max_threads()
