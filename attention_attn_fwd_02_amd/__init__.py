"""MI355X-native fused attention forward: a C-ABI HIP library and its binding.

    from attention_attn_fwd_02_amd import fwd, fwd_decode
    o, lse = fwd(q, k, v, causal=True)          # prefill
    o, lse = fwd_decode(q1, k, v)               # few query rows: split-KV
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)   # gradients
    o, lse, k_rot = fwd_rope(q, k, v, cos, sin, causal=True)   # rotary embedding on Q, K

The library is loaded on first use (`attn.load_library`); importing the package
does not touch the GPU.
"""
from .attn import (ATTN_BF16, ATTN_FP16, ATTN_FP32, ATTN_OK, ATTN_ERR_INVALID_ARG,
                   ATTN_ERR_UNSUPPORTED, ATTN_ERR_LAUNCH, ATTN_ROPE_INTERLEAVED, ATTN_ROPE_HALVES,
                   AttnError, attn_bwd, attn_bwd_workspace, attn_fwd, attn_fwd_decode,
                   attn_fwd_decode_noalloc, attn_fwd_decode_workspace, attn_fwd_rope,
                   attn_status_str, bwd, fwd, fwd_decode, fwd_decode_noalloc, fwd_rope,
                   load_library)

__all__ = ["ATTN_BF16", "ATTN_FP16", "ATTN_FP32", "ATTN_OK", "ATTN_ERR_INVALID_ARG",
           "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_LAUNCH", "ATTN_ROPE_INTERLEAVED", "ATTN_ROPE_HALVES",
           "AttnError", "attn_bwd", "attn_bwd_workspace", "attn_fwd", "attn_fwd_decode",
           "attn_fwd_decode_noalloc", "attn_fwd_decode_workspace", "attn_fwd_rope",
           "attn_status_str", "bwd", "fwd", "fwd_decode", "fwd_decode_noalloc", "fwd_rope",
           "load_library"]
