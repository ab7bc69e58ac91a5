"""torch.autograd wrapper: forward saves (q, k, v, o, lse); backward recomputes P."""
from __future__ import annotations

import torch

from . import _lib


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, softmax_scale, causal, window_size, seqlens):
        o, lse = _lib.fwd(q, k, v, softmax_scale, causal, window_size, seqlens=seqlens)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (softmax_scale, causal, window_size)
        ctx.seqlens = seqlens
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = _lib.bwd(do.contiguous(), q, k, v, o, lse, *ctx.cfg, seqlens=ctx.seqlens)
        return dq, dk, dv, None, None, None, None


def attention(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1), seqlens=None):
    """softmax(scale * q k^T + mask) v with the library's fused kernels (differentiable).
    ``seqlens`` (int32 [B] on the device) makes it a padded batch: sample b is its first
    seqlens[b] rows, the other rows give zero outputs and zero gradients."""
    return _Attention.apply(q, k, v, softmax_scale, causal, tuple(window_size), seqlens)
