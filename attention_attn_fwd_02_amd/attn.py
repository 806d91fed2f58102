"""Thin Python binding of the C-ABI library `libattn_fwd.so` (include/attn_fwd.h).

Argument marshalling only: every step runs in the HIP kernels behind `attn_fwd`,
`attn_fwd_decode` (and its allocation-free variant), `attn_bwd` and `attn_fwd_rope`.  PyTorch supplies device memory and the stream.  If
the library is missing this module raises; there is no fallback path.
"""
import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn_fwd.so")

# attn_dtype_t
ATTN_BF16, ATTN_FP16, ATTN_FP32 = 0, 1, 2
# attn_rope_layout_t
ATTN_ROPE_INTERLEAVED, ATTN_ROPE_HALVES = 1, 2
# attn_status_t
ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_LAUNCH = 0, 1, 2, 3

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__("attn_fwd failed: %s (%d)" % (attn_status_str(status), status))


def load_library(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libattn_fwd.so is not built (%s); run "
                           "`python -m attention_attn_fwd_02_amd.build`" % path)
    # torch ships its own HIP runtime under another file name; loaded first, it also
    # serves this library (same soname).  Loaded after this library, it would be a
    # second runtime, whose streams and memory this library's kernels cannot use.
    import torch  # noqa: F401  (no GPU access: importing does not initialise a device)
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_status_str.argtypes = [i32]
    lib.attn_status_str.restype = ctypes.c_char_p
    sz = ctypes.c_size_t
    lib.attn_fwd_decode_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.attn_fwd_decode_workspace.restype = i32
    lib.attn_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                    i32, vp, sz, vp]
    lib.attn_fwd_decode.restype = i32
    lib.attn_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                            i32, i32, i32, vp]
    lib.attn_fwd_decode_noalloc.restype = i32
    lib.attn_bwd_workspace.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.attn_bwd_workspace.restype = i32
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                             i32, i32, vp, sz, vp]
    lib.attn_bwd.restype = i32
    lib.attn_fwd_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                  f32, i32, i32, vp]
    lib.attn_fwd_rope.restype = i32
    _lib = lib
    return lib


def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, dtype, stream) -> int:
    """The C entry point with raw integer pointers; returns the status code."""
    return load_library().attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, float(scale),
                                   int(causal), int(dtype), stream)


def attn_fwd_decode_workspace(B, Hq, Hkv, Sq, Sk, D, nsplit):
    """(status, bytes) of the C workspace query."""
    n = ctypes.c_size_t(0)
    st = load_library().attn_fwd_decode_workspace(B, Hq, Hkv, Sq, Sk, D, int(nsplit), ctypes.byref(n))
    return st, n.value


def attn_fwd_decode(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, dtype, nsplit,
                    workspace, workspace_bytes, stream) -> int:
    """The C entry point with raw integer pointers; returns the status code."""
    return load_library().attn_fwd_decode(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, float(scale),
                                          int(causal), int(dtype), int(nsplit), workspace,
                                          int(workspace_bytes), stream)


def attn_fwd_decode_noalloc(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, dtype, nsplit,
                            stream) -> int:
    """The C entry point with raw integer pointers; returns the status code."""
    return load_library().attn_fwd_decode_noalloc(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D,
                                                  float(scale), int(causal), int(dtype),
                                                  int(nsplit), stream)


def attn_bwd_workspace(B, Hq, Hkv, Sq, Sk, D):
    """(status, bytes) of the C workspace query of the backward."""
    n = ctypes.c_size_t(0)
    st = load_library().attn_bwd_workspace(B, Hq, Hkv, Sq, Sk, D, ctypes.byref(n))
    return st, n.value


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, scale, causal, dtype,
             workspace, workspace_bytes, stream) -> int:
    """The C entry point with raw integer pointers; returns the status code."""
    return load_library().attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D,
                                   float(scale), int(causal), int(dtype), workspace,
                                   int(workspace_bytes), stream)


def attn_fwd_rope(q, k, v, o, lse, k_rot, rope_cos, rope_sin, rope_layout, B, Hq, Hkv, Sq, Sk, D,
                  scale, causal, dtype, stream) -> int:
    """The C entry point with raw integer pointers; returns the status code."""
    return load_library().attn_fwd_rope(q, k, v, o, lse, k_rot, rope_cos, rope_sin,
                                        int(rope_layout), B, Hq, Hkv, Sq, Sk, D, float(scale),
                                        int(causal), int(dtype), stream)


def attn_status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def _dtype_code(t):
    import torch
    return {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_FP16, torch.float32: ATTN_FP32}[t]


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None, want_lse=True, stream=None):
    """Attention forward on torch device tensors.

    q: [B, Hq, Sq, D], k and v: [B, Hkv, Sk, D] (contiguous, one dtype: bf16,
    fp16 or fp32).  Returns (o, lse) with o like q and lse [B, Hq, Sq] fp32 (None
    when want_lse is False).  `out` / `lse` may be passed to reuse buffers.  The
    call is asynchronous on `stream` (default: torch's current stream).
    """
    import torch
    B, Hq, Hkv, Sq, Sk, D = _check_inputs(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if want_lse:
        _check_buffer(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                  lse.data_ptr() if want_lse else None,
                  B, Hq, Hkv, Sq, Sk, D, scale, causal, _dtype_code(q.dtype),
                  stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, (lse if want_lse else None)


def _check_inputs(q, k, v):
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch: q%s k%s v%s" % (tuple(q.shape), tuple(k.shape),
                                                          tuple(v.shape)))
    return B, Hq, Hkv, Sq, Sk, D


def _check_buffer(t, name, shape, dtype, device):
    """A caller-supplied output: on q's device, contiguous, of the exact shape and
    dtype the kernels write (they write every element of it and nothing past it)."""
    if not t.is_cuda or t.device != device:
        raise ValueError("%s must be a device tensor on %s" % (name, device))
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError("%s must be %s %s, got %s %s" % (name, list(shape), dtype,
                                                           list(t.shape), t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_workspace(t, device):
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor on %s" % device)


def fwd_decode(q, k, v, causal=False, scale=None, nsplit=0, out=None, lse=None, want_lse=True,
               workspace=None, stream=None):
    """Split-KV attention (few query rows per K/V head group) on torch device tensors.

    Same tensors and result as `fwd` (bf16 or fp16 only; (Hq/Hkv)*Sq <= 32).  The
    workspace (a uint8 device tensor) is allocated here when not given; reuse one
    across calls on the same stream to avoid the allocation.
    """
    import torch
    B, Hq, Hkv, Sq, Sk, D = _check_inputs(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st, need = attn_fwd_decode_workspace(B, Hq, Hkv, Sq, Sk, D, nsplit)
    if st != ATTN_OK:
        raise AttnError(st)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if want_lse:
        _check_buffer(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = attn_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr() if want_lse else None, B, Hq, Hkv, Sq, Sk, D, scale,
                         causal, _dtype_code(q.dtype), nsplit, workspace.data_ptr(),
                         workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, (lse if want_lse else None)


def fwd_decode_noalloc(q, k, v, causal=False, scale=None, nsplit=0, out=None, lse=None,
                       want_lse=True, stream=None):
    """`fwd_decode` through the allocation-free entry point: the partial results go
    to the library's static 16 MiB device scratch instead of a workspace.  With
    `out` (and `lse`) given, nothing is allocated here either."""
    import torch
    B, Hq, Hkv, Sq, Sk, D = _check_inputs(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if want_lse:
        _check_buffer(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = attn_fwd_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if want_lse else None, B, Hq, Hkv, Sq, Sk, D,
                                 scale, causal, _dtype_code(q.dtype), nsplit, stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, (lse if want_lse else None)


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None,
        workspace=None, stream=None):
    """Gradients (dq, dk, dv) of `fwd` on torch device tensors (bf16 or fp16).

    o and lse are `fwd`'s outputs for q, k, v; dout is the gradient of the loss
    with respect to o.  The workspace (uint8 device tensor) is allocated here when
    not given.
    """
    import torch
    B, Hq, Hkv, Sq, Sk, D = _check_inputs(q, k, v)
    if o.shape != q.shape or dout.shape != q.shape or o.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("o and dout must match q")
    if lse is None or tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be the forward's [B, Hq, Sq] fp32 log-sum-exp")
    if not (o.is_contiguous() and dout.is_contiguous() and lse.is_contiguous()):
        raise ValueError("o, lse, dout must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st, need = attn_bwd_workspace(B, Hq, Hkv, Sq, Sk, D)
    if st != ATTN_OK:
        raise AttnError(st)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name, like in ((o, "o", q), (dout, "dout", q), (lse, "lse", None), (dq, "dq", q),
                          (dk, "dk", k), (dv, "dv", v)):
        if like is None:
            _check_buffer(t, name, (B, Hq, Sq), torch.float32, q.device)
        else:
            _check_buffer(t, name, like.shape, like.dtype, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                  dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                  B, Hq, Hkv, Sq, Sk, D, scale, causal, _dtype_code(q.dtype),
                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                  stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return dq, dk, dv


def fwd_rope(q, k, v, rope_cos, rope_sin, layout=ATTN_ROPE_INTERLEAVED, causal=False, scale=None,
             out=None, lse=None, want_lse=True, k_rot=None, stream=None):
    """Attention with the rotary embedding applied to Q and K (bf16 or fp16).

    rope_cos, rope_sin: [P, D/2] fp32 device tables with P >= Sk (position p in
    row p); key j sits at position j and query i at i + Sk - Sq (Sq <= Sk).
    Returns (o, lse, k_rot): k_rot is the rotated K (allocated here unless given).
    """
    import torch
    B, Hq, Hkv, Sq, Sk, D = _check_inputs(q, k, v)
    for t in (rope_cos, rope_sin):
        if not t.is_cuda or t.device != q.device or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("rope tables must be contiguous fp32 tensors on q's device")
        if t.dim() != 2 or t.shape[1] != D // 2 or t.shape[0] < Sk:
            raise ValueError("rope tables must be [P >= Sk, D/2]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if want_lse:
        _check_buffer(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    if k_rot is None:
        k_rot = torch.empty_like(k)
    _check_buffer(k_rot, "k_rot", k.shape, k.dtype, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = attn_fwd_rope(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       lse.data_ptr() if want_lse else None, k_rot.data_ptr(),
                       rope_cos.data_ptr(), rope_sin.data_ptr(), layout, B, Hq, Hkv, Sq, Sk, D,
                       scale, causal, _dtype_code(q.dtype), stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, (lse if want_lse else None), k_rot
