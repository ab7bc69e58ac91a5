"""Attention with N_q queries over N_k keys (N_q != N_k allowed) — test infrastructure.

Sources: the definition of ``attention`` (the formula softmax(QK^T/sqrt(d_k))V of [PT29],
scale, -inf mask and safe softmax as there); the inference use the pages name — LLM inference
([FA37] §1.3) and the KV cache that PagedAttention pages through memory ([PT29], closing section
"写在最后") — where a step's new queries attend to every cached key; the ``causal`` / ``window_size`` switches of
[A100] §4.2.  The (batch, num_heads, seq_len, head_dim) tensors of [FA37] §3.2 may come as
views of (batch, seq_len, num_heads, head_dim) memory (the ``view(...).transpose(1, 2)`` of
its §4.2 module, the (batch, seq, heads * head_dim) layout of its §3.3): the layout is a
matter of addressing only and does not enter this definition.

Reading where the pages are silent (they never define a mask for N_q != N_k):
  * the queries are the LAST N_q positions of the key sequence: query i sits at position
      p_i = i + (N_k - N_q)
    and key j is allowed for it iff
      (not causal or j <= p_i) and (left < 0 or j >= p_i - left) and (right < 0 or j <= p_i + right)
    (inclusive bounds, -1 unbounded, causal AND window, as in ``attention``).  A decode step
    (N_q = 1) then sees every cached key, and a block of new queries sees the cache plus its own
    causal prefix.  With N_q = N_k this is ``attention`` itself.
  * a row with no allowed key (N_q > N_k under causal, or a window that misses every key) has
    O = 0 and LSE = -inf.

ALiBi: [A100] §4.2 lists ``alibi_slopes`` ("linear bias coefficients") among the switches of
its attention call and [FA37] §6 names ALiBi as the relative position encoding for very long
sequences; neither page writes the bias out.  Reading: head h adds -slope_h * |p_i - j| to
the scaled score of query i and key j (a penalty linear in the distance between their
positions), before the mask and the softmax:
      S_ij = scale * <q_i, k_j> - slope * |p_i - j|
With slope = 0 this is the definition above.

Block-sparse attention: [A100] §6 lists block-sparse FlashAttention (90% sparsity on 64k-token
texts) among the next steps and [FA37] §6 names sparse attention for very long sequences;
neither fixes the pattern.  Reading: a boolean mask over blocks of BLOCK = 64 queries x 64
keys (query index i // 64, key index j // 64) selects the blocks that are computed; a pair
outside the selected blocks is hidden like any masked pair (its score is -inf), so it takes
no part in the softmax.

Key padding mask: the reference attention module of [FA37] §4.2 takes a ``key_padding_mask``
of shape (batch, seq_len), True where a key is padding, and sets the scores of those keys to
-inf before the softmax, broadcast over heads and queries ([PT29], section "如何集成
FlashAttention：从安装到应用", names the same argument among those the replacement layer keeps):
a padding key is hidden from every query of its batch entry, in every head.  Reading: the mask may mark any keys
(holes anywhere, not only a padded tail), it combines with the other masks by AND of the
visible pairs, and a row left with no visible key follows the rule above (O = 0, LSE = -inf)
where the page's softmax over a row of -inf would give NaN.
"""
from __future__ import annotations

import numpy as np


def cross_allowed_mask(n_q: int, n_k: int, causal: bool, window=(-1, -1)) -> np.ndarray:
    """Boolean [n_q, n_k]: True where key j is visible to query i (reading above)."""
    left, right = int(window[0]), int(window[1])
    p = (np.arange(n_q, dtype=np.int64) + (n_k - n_q))[:, None]
    j = np.arange(n_k, dtype=np.int64)[None, :]
    ok = np.ones((n_q, n_k), dtype=bool)
    if causal:
        ok &= j <= p
    if left >= 0:
        ok &= j >= p - left
    if right >= 0:
        ok &= j <= p + right
    return ok


def cross_allowed_pairs(n_q: int, n_k: int, causal: bool, window=(-1, -1)) -> int:
    """Number of (query, key) pairs the mask allows for one (batch, head)."""
    return int(cross_allowed_mask(n_q, n_k, causal, window).sum())


def alibi_bias(n_q: int, n_k: int, slope: float) -> np.ndarray:
    """[n_q, n_k] float64: -slope * |p_i - j| with p_i = i + (n_k - n_q)."""
    p = (np.arange(n_q, dtype=np.float64) + (n_k - n_q))[:, None]
    j = np.arange(n_k, dtype=np.float64)[None, :]
    return -float(slope) * np.abs(p - j)


BLOCK = 64   # queries and keys per block of a block-sparse mask


def block_allowed(n_q: int, n_k: int, block_mask) -> np.ndarray:
    """[n_q, n_k] bool: True where the pair's (query block, key block) is selected."""
    bm = np.asarray(block_mask, dtype=bool)
    return bm[np.arange(n_q)[:, None] // BLOCK, np.arange(n_k)[None, :] // BLOCK]


def _scores(q, k, scale, causal, window, slope, block_mask=None, key_mask=None):
    ok = cross_allowed_mask(q.shape[0], k.shape[0], causal, window)
    if block_mask is not None:
        ok &= block_allowed(q.shape[0], k.shape[0], block_mask)
    if key_mask is not None:     # True = a padding key, hidden from every query
        ok &= ~np.asarray(key_mask, dtype=bool)[None, :]
    s = scale * (q @ k.T)
    if slope:
        s = s + alibi_bias(q.shape[0], k.shape[0], slope)
    return np.where(ok, s, -np.inf)


def cross_forward(q, k, v, scale: float, causal: bool = False, window=(-1, -1),
                  slope: float = 0.0, block_mask=None, key_mask=None):
    """One (batch, head): q float64 [N_q, d], k, v [N_k, d] -> (O [N_q, d], LSE [N_q]).

    S = scale * Q K^T (minus the ALiBi distance penalty when slope != 0) is materialised in
    full, masked with -inf (also outside the selected blocks of ``block_mask``
    [ceil(N_q / 64), ceil(N_k / 64)], if given, and at the keys where ``key_mask`` [N_k] is
    True), and put through the max-shifted softmax; O = P V, LSE = rowmax + ln(rowsum).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = _scores(q, k, scale, causal, window, slope, block_mask, key_mask)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    e = np.exp(s - np.where(live, m, 0.0)[:, None])     # exp(-inf) = 0 at hidden entries
    l = e.sum(axis=1)
    p = e / np.where(live, l, 1.0)[:, None]
    o = np.where(live[:, None], p @ v, 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse


def cross_forward_bh(q, k, v, scale, causal=False, window=(-1, -1), slopes=None,
                     block_mask=None, key_padding_mask=None):
    """q [B, H, N_q, d], k, v [B, H, N_k, d] -> (O [B, H, N_q, d], LSE [B, H, N_q]);
    ``slopes``: the H ALiBi slopes, or None; ``block_mask``: [H, n_qb, n_kb] or None;
    ``key_padding_mask``: [B, N_k] (True = padding key) or None."""
    B, H, n_q, _ = q.shape
    o = np.empty((B, H, n_q, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, n_q), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = cross_forward(q[b, h], k[b, h], v[b, h], scale, causal, window,
                                               0.0 if slopes is None else float(slopes[h]),
                                               None if block_mask is None else block_mask[h],
                                               None if key_padding_mask is None
                                               else key_padding_mask[b])
    return o, lse


def cross_backward(q, k, v, do, scale: float, causal: bool = False, window=(-1, -1),
                   slope: float = 0.0, block_mask=None, key_mask=None):
    """One (batch, head): gradients (dQ [N_q, d], dK, dV [N_k, d]) of <dO, O> for
    ``cross_forward``, the ordinary derivative of that definition:

        dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(P * dP)),
        dQ = scale * dS K,   dK = scale * dS^T Q

    with P recomputed from Q and K; rows without a visible key have P = 0 and contribute
    nothing.  The ALiBi penalty does not depend on Q or K, so it enters only through P.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    s = _scores(q, k, scale, causal, window, slope, block_mask, key_mask)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    e = np.exp(s - np.where(live, m, 0.0)[:, None])
    p = e / np.where(live, e.sum(axis=1), 1.0)[:, None]
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ q), dv


def cross_backward_bh(q, k, v, do, scale, causal=False, window=(-1, -1), slopes=None,
                      block_mask=None, key_padding_mask=None):
    """[B, H, N_q, d] q and dO, [B, H, N_k, d] k and v -> (dQ, dK, dV), one head at a time."""
    B, H = q.shape[:2]
    dq, dk, dv = (np.empty(t.shape, dtype=np.float64) for t in (q, k, v))
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = cross_backward(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, window,
                0.0 if slopes is None else float(slopes[h]),
                None if block_mask is None else block_mask[h],
                None if key_padding_mask is None else key_padding_mask[b])
    return dq, dk, dv
