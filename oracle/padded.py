"""Padded batches: each sample is attention over its own first L_b rows — test infrastructure.

Sources: "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型（含A100环境配置）" ([A100])
§6 hands a length-grouped attention each sample's actual length; "Flash Attention 3.7 核心原理
与实战：加速Transformer模型训练与推理" ([FA37]) §4.2 hides padded keys with a key padding mask
(-inf before the softmax).

Reading, over one padded [B, H, N, d] array with lengths L_b (values clamped to [0, N]):
  * sample b is rows 0 .. L_b - 1 of every head of batch b; it is the definition of
    ``attention`` over those rows alone (so keys past L_b are hidden from every query);
  * rows past L_b do not exist: they are written as O = 0, LSE = -inf, and their
    gradients dQ, dK, dV as 0; their Q, K, V and dO values never matter.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_backward, attention_forward


def clamp_lengths(seqlens, n: int):
    """Lengths as the padded call reads them: below 0 counts as 0, above N as N."""
    return [min(max(int(x), 0), n) for x in seqlens]


def padded_forward_bh(q, k, v, seqlens, scale, causal=False, window=(-1, -1)):
    """[B, H, N, d] float64 arrays and B lengths -> (O [B, H, N, d], LSE [B, H, N])."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, H, N), -np.inf, dtype=np.float64)
    for b, L in enumerate(clamp_lengths(seqlens, N)):
        if L == 0:
            continue
        for h in range(H):
            o[b, h, :L], lse[b, h, :L] = attention_forward(q[b, h, :L], k[b, h, :L], v[b, h, :L],
                                                           scale, causal, window)
    return o, lse


def padded_backward_bh(q, k, v, do, seqlens, scale, causal=False, window=(-1, -1)):
    """[B, H, N, d] float64 arrays and B lengths -> (dQ, dK, dV), zero past each length."""
    B, H, N, d = q.shape
    dq, dk, dv = (np.zeros(t.shape, dtype=np.float64) for t in (q, k, v))
    for b, L in enumerate(clamp_lengths(seqlens, N)):
        if L == 0:
            continue
        for h in range(H):
            dq[b, h, :L], dk[b, h, :L], dv[b, h, :L] = attention_backward(
                q[b, h, :L], k[b, h, :L], v[b, h, :L], do[b, h, :L], scale, causal, window)
    return dq, dk, dv
