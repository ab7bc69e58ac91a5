"""Fused exact scaled-dot-product attention for AMD Instinct MI355X (gfx950).

    import exact_attention_125_amd as fa
    o, lse = fa.fwd(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1))
    dq, dk, dv = fa.bwd(do, q, k, v, o, lse, ...)
    o = fa.attention(q, k, v, causal=True)           # autograd-aware
    o, lse = fa.fwd_kv(q, k, v, causal=True)         # N_q != N_k, any strides
    dq, dk, dv = fa.bwd_kv(do, q, k, v, o, lse, causal=True)
    o = fa.attention_kv(q, k, v, causal=True, alibi_slopes=s, dropout_p=0.1, block_mask=m)

q, k, v: contiguous [batch, heads, seqlen, head_dim] float16 / bfloat16 GPU tensors,
head_dim 64 or 128.  The work runs in the HIP kernels of ``libfa.so`` (C ABI in
include/fa.h); importing this package fails if that library has not been built.
"""
from ._lib import (FaError, bwd, bwd_kv, bwd_noalloc, bwd_packed, bwd_workspace_size,  # noqa: F401
                   fwd, fwd_fp8, fwd_kv, fwd_kv_fp8, fwd_kv_workspace_size, fwd_packed, lib)
from .autograd import attention, attention_kv  # noqa: F401

__all__ = ["fwd", "bwd", "attention", "attention_kv", "bwd_workspace_size", "fwd_kv",
           "fwd_kv_workspace_size", "fwd_kv_fp8", "fwd_fp8", "fwd_packed", "bwd_packed",
           "bwd_kv", "bwd_noalloc",
           "FaError", "lib"]
