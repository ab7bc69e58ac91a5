"""torch.autograd wrapper: forward saves (q, k, v, o, lse); backward recomputes P."""
from __future__ import annotations

import torch

from . import _lib


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, softmax_scale, causal, window_size):
        o, lse = _lib.fwd(q, k, v, softmax_scale, causal, window_size)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (softmax_scale, causal, window_size)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = _lib.bwd(do.contiguous(), q, k, v, o, lse, *ctx.cfg)
        return dq, dk, dv, None, None, None


def attention(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1)):
    """softmax(scale * q k^T + mask) v with the library's fused kernels (differentiable)."""
    return _Attention.apply(q, k, v, softmax_scale, causal, tuple(window_size))
