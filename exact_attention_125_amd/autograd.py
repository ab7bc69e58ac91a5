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


class _AttentionKv(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, softmax_scale, causal, window_size, alibi_slopes, dropout_p,
                dropout_seed, dropout_offset, block_mask, key_padding_mask):
        extra = dict(alibi_slopes=alibi_slopes, dropout_p=dropout_p, dropout_seed=dropout_seed,
                     dropout_offset=dropout_offset, block_mask=block_mask,
                     key_padding_mask=key_padding_mask)
        o, lse = _lib.fwd_kv(q, k, v, softmax_scale, causal, window_size, **extra)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (softmax_scale, causal, window_size)
        ctx.extra = extra
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        if do.stride(-1) != 1:
            do = do.contiguous()
        dq, dk, dv = _lib.bwd_kv(do, q, k, v, o, lse, *ctx.cfg, **ctx.extra)
        return (dq, dk, dv) + (None,) * 9


def attention_kv(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1),
                 alibi_slopes=None, dropout_p=0.0, dropout_seed=0, dropout_offset=0,
                 block_mask=None, key_padding_mask=None):
    """Differentiable ``fa_fwd_kv`` / ``fa_bwd_kv``: q [B, H, N_q, d] over k, v [B, H, N_k, d]
    (the queries being the last N_q key positions), any strides with a contiguous last
    dimension, optional ALiBi slopes, attention dropout (Philox masks from ``dropout_seed`` and
    ``dropout_offset``; the backward replays the same masks), a block-sparse mask and a key
    padding mask ([B, N_k], True where a key is padding).  k and v must not share rows (a head
    stride of 0 would make their gradients overlap)."""
    return _AttentionKv.apply(q, k, v, softmax_scale, causal, tuple(window_size), alibi_slopes,
                              float(dropout_p), int(dropout_seed), int(dropout_offset), block_mask,
                              key_padding_mask)
