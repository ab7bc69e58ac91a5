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


# ---------------------------------------------------------------------------- packed batches
# Packed batches carry the same sequences without padding: per head, the rows of every sequence
# concatenated ([H, total, d]), sequence b being rows cu[b] .. cu[b+1] - 1.  Reading: each
# sequence is attention over its own rows alone, as for a padded batch; rows no sequence covers
# belong to no sequence (returned as NaN here: the library neither reads nor writes them).
# Offsets are taken as the kernels read them: each clamped to [0, total], each sequence to
# [cu[b], cu[b+1]) and to at most max_seqlen rows.

def packed_ranges(cu, total: int, max_seqlen: int):
    """(start, stop) row range of every sequence, as the packed call reads the offsets."""
    out = []
    for b in range(len(cu) - 1):
        c0 = min(max(int(cu[b]), 0), total)
        c1 = min(max(int(cu[b + 1]), c0), total)
        out.append((c0, c0 + min(c1 - c0, max_seqlen)))
    return out


def packed_forward(q, k, v, cu, max_seqlen, scale, causal=False, window=(-1, -1)):
    """[H, total, d] float64 arrays -> (O [H, total, d], LSE [H, total]), NaN outside every
    sequence."""
    H, total, _ = q.shape
    o = np.full((H, total, v.shape[-1]), np.nan)
    lse = np.full((H, total), np.nan)
    for r0, r1 in packed_ranges(cu, total, max_seqlen):
        if r1 == r0:
            continue
        for h in range(H):
            o[h, r0:r1], lse[h, r0:r1] = attention_forward(q[h, r0:r1], k[h, r0:r1], v[h, r0:r1],
                                                           scale, causal, window)
    return o, lse


def packed_backward(q, k, v, do, cu, max_seqlen, scale, causal=False, window=(-1, -1)):
    """[H, total, d] float64 arrays -> (dQ, dK, dV), NaN outside every sequence."""
    H, total, _ = q.shape
    dq, dk, dv = (np.full(t.shape, np.nan) for t in (q, k, v))
    for r0, r1 in packed_ranges(cu, total, max_seqlen):
        if r1 == r0:
            continue
        for h in range(H):
            dq[h, r0:r1], dk[h, r0:r1], dv[h, r0:r1] = attention_backward(
                q[h, r0:r1], k[h, r0:r1], v[h, r0:r1], do[h, r0:r1], scale, causal, window)
    return dq, dk, dv
