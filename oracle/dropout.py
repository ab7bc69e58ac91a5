"""Attention dropout with a counter-based generator — test infrastructure.

Sources: the ``dropout_p`` argument of the attention call in [A100] §4.2 and of the SDPA call
in [FA37] §3.2, and the ``StandardMultiHeadAttention`` module of [FA37] §4.2, which applies
``F.dropout`` to the softmax weights before multiplying by V.  Reading: each weight P_ij is
kept with probability r (about 1 - p) and scaled by 1 / r, or zeroed, so that the expected
weight is P_ij itself (the unbiased drop that ``F.dropout`` performs):

    O = (P * M / r) V,     M_ij in {0, 1},  P(M_ij = 1) = r

The LSE is that of the softmax before dropout (dropout acts on the weights, after the
normalisation).  The pages fix no generator; M must be reproducible by the GPU and by this
oracle, so it comes from Philox4x32-10, the counter-based generator of J. K. Salmon,
M. A. Moraes, R. O. Dror and D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
(SC 2011), written here from its definition:
  * a round maps counter (c0, c1, c2, c3) and key (k0, k1) to
      (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
    with M0 = 0xD2511F53, M1 = 0xCD9E8D57 and 32x32 -> 64-bit products;
  * between rounds the key is bumped by (0x9E3779B9, 0xBB67AE85); 10 rounds.
Counter layout (this library's choice): one call covers 2 queries x 4 keys of one
(batch, head), 16 random bits per (query, key) pair:
    counter = (j >> 2, i >> 1, b * H + h, offset),  key = (seed mod 2^32, seed >> 32),
    half-word index t = 4 (i & 1) + (j & 3),  u = bits 16 (t & 1) .. 16 (t & 1) + 15 of word t >> 1
for query index i and key index j.  Pair (i, j) is kept iff u >= floor(p 2^16), which happens
with probability r = (2^16 - floor(p 2^16)) / 2^16 (1 - p quantised to 2^-16); kept weights are
scaled by 1 / r = 2^16 / (2^16 - floor(p 2^16)), the inverse of that probability, so the mean
of M / r is exactly 1.
"""
from __future__ import annotations

import math

import numpy as np

from .cross import _scores

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 over arrays of counters (uint32-valued, any broadcastable shapes) with
    one key; returns the four output words as uint64 arrays holding 32-bit values."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    k = [np.uint64(int(k0) & 0xFFFFFFFF), np.uint64(int(k1) & 0xFFFFFFFF)]
    for r in range(10):
        p0 = np.uint64(M0) * c[0]          # < 2^64: exact in uint64
        p1 = np.uint64(M1) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k[0], p1 & _MASK32,
             (p0 >> np.uint64(32)) ^ c[3] ^ k[1], p0 & _MASK32]
        if r < 9:
            k = [(k[0] + np.uint64(W0)) & _MASK32, (k[1] + np.uint64(W1)) & _MASK32]
    return c


def keep_threshold(p: float) -> int:
    """floor(p 2^16) for 0 <= p < 1: a 16-bit draw at or above it keeps its pair."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(math.floor(p * 65536.0))


def keep_scale(p: float) -> float:
    """Factor of kept weights: 1 / r with r = (2^16 - floor(p 2^16)) / 2^16 the probability that
    a pair is kept (1 for p = 0)."""
    return 65536.0 / (65536 - keep_threshold(p))


def dropout_keep(n_q: int, n_k: int, bh: int, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """Boolean [n_q, n_k] keep mask of (batch, head) number bh = b * H + h."""
    i = np.arange(n_q, dtype=np.uint64)[:, None]
    j = np.arange(n_k, dtype=np.uint64)[None, :]
    one, two, three = np.uint64(1), np.uint64(2), np.uint64(3)
    words = philox4x32_10(j >> two, i >> one, np.uint64(bh), np.uint64(offset),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    t = np.broadcast_to(np.uint64(4) * (i & one) + (j & three), (n_q, n_k))
    w = np.choose((t >> one).astype(np.int64), [np.broadcast_to(x, (n_q, n_k)) for x in words])
    u = (w >> (np.uint64(16) * (t & one))) & np.uint64(0xFFFF)
    return u >= np.uint64(keep_threshold(p))


def _probs(q, k, scale, causal, window, slope, key_mask=None):
    s = _scores(q, k, scale, causal, window, slope, key_mask=key_mask)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    e = np.exp(s - np.where(live, m, 0.0)[:, None])
    l = e.sum(axis=1)
    p = e / np.where(live, l, 1.0)[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return p, lse


def dropout_forward(q, k, v, scale, causal, window, slope, p_drop, keep, key_mask=None):
    """One (batch, head) with the keep mask ``keep`` [N_q, N_k]: (O, LSE) with
    O = (P * keep / r) V (1 / r = ``keep_scale(p_drop)``) and LSE of the softmax before
    dropout; ``key_mask`` [N_k] hides padding keys as in ``cross_forward``."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    p, lse = _probs(q, k, scale, causal, window, slope, key_mask)
    return (p * keep * keep_scale(p_drop)) @ v, lse


def dropout_backward(q, k, v, do, scale, causal, window, slope, p_drop, keep, key_mask=None):
    """Gradients (dQ, dK, dV) of <dO, O> for ``dropout_forward`` with a fixed mask:
        dV = (P * keep / r)^T dO,   dP = (dO V^T) * keep / r,
        dS = P * (dP - rowsum(P * dP)),   dQ = scale dS K,   dK = scale dS^T Q."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    p, _ = _probs(q, k, scale, causal, window, slope, key_mask)
    f = keep * keep_scale(p_drop)
    dv = (p * f).T @ do
    dp = (do @ v.T) * f
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ q), dv


def dropout_forward_bh(q, k, v, scale, causal, window, p_drop, seed, offset=0, slopes=None,
                       key_padding_mask=None):
    """[B, H, N_q, d] / [B, H, N_k, d] arrays -> (O, LSE), masks from ``dropout_keep``;
    ``key_padding_mask`` [B, N_k] or None."""
    B, H, n_q, _ = q.shape
    n_k = k.shape[2]
    o = np.empty((B, H, n_q, v.shape[-1]))
    lse = np.empty((B, H, n_q))
    for b in range(B):
        for h in range(H):
            keep = dropout_keep(n_q, n_k, b * H + h, p_drop, seed, offset)
            o[b, h], lse[b, h] = dropout_forward(q[b, h], k[b, h], v[b, h], scale, causal, window,
                                                 0.0 if slopes is None else float(slopes[h]),
                                                 p_drop, keep,
                                                 None if key_padding_mask is None
                                                 else key_padding_mask[b])
    return o, lse


def dropout_backward_bh(q, k, v, do, scale, causal, window, p_drop, seed, offset=0, slopes=None,
                        key_padding_mask=None):
    B, H, n_q, _ = q.shape
    n_k = k.shape[2]
    dq, dk, dv = (np.empty(t.shape) for t in (q, k, v))
    for b in range(B):
        for h in range(H):
            keep = dropout_keep(n_q, n_k, b * H + h, p_drop, seed, offset)
            dq[b, h], dk[b, h], dv[b, h] = dropout_backward(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, window,
                0.0 if slopes is None else float(slopes[h]), p_drop, keep,
                None if key_padding_mask is None else key_padding_mask[b])
    return dq, dk, dv
