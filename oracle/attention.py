"""The definition of masked scaled-dot-product attention, in float64 — test infrastructure.

What is computed (one (batch, head) slice, queries i and keys j in 0..N-1):

    S   = scale * Q K^T                          (the N x N score matrix, materialised)
    S_ij = -inf where key j is not allowed for query i
    P   = softmax over j of S  (max-shifted: exp(S - rowmax) / rowsum)
    O   = P V,     LSE_i = rowmax_i + ln(rowsum_i)

Sources: the formula softmax(QK^T/sqrt(d_k))V ([PT29], section "FlashAttention：不只是
更快的 Attention"); the three-step S -> P -> O computation ([A100] §1; [FA37] §3.1;
[VRAM] §三 ``traditional_attention``); the max-subtracted ("safe") softmax ([A100]
§2.2 ``safe_softmax``); scale first, then an additive -inf mask, then softmax, as in the
``StandardMultiHeadAttention`` module of [FA37] §4.2; default scale head_dim**-0.5
([FA37] §3.2; [A100] §4.2 ``softmax_scale=None``); the ``causal`` and
``window_size=(-1, -1)`` switches ([A100] §4.2).

Readings where the pages are silent:
  * mask bounds are inclusive: key j is allowed for query i iff
      (not causal or j <= i) and (left < 0 or j >= i - left) and (right < 0 or j <= i + right)
    with -1 meaning unbounded; causal and window combine as an AND;
  * LSE is the natural logarithm of sum_j exp(S_ij) over the allowed keys, in the units
    of the scaled scores (the "normalisation factor" [A100] §2.2 says is kept for backward);
  * a row with no allowed key has no defined softmax; with equal query/key lengths and
    window bounds >= 0 or -1 the diagonal is always allowed, so this never happens; if it
    is asked for anyway, O = 0 and LSE = -inf;
  * the backward is the ordinary derivative of this definition (the pages say only that
    it recomputes instead of storing, [PT29] "3. 重计算策略（Recomputation）").
"""
from __future__ import annotations

import numpy as np


def allowed_mask(n: int, causal: bool, window=(-1, -1), rows=None) -> np.ndarray:
    """Boolean [len(rows), n]: True where key j is visible to query i (reading above)."""
    left, right = int(window[0]), int(window[1])
    i = (np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    j = np.arange(n)[None, :]
    ok = np.ones((i.shape[0], n), dtype=bool)
    if causal:
        ok &= j <= i
    if left >= 0:
        ok &= j >= i - left
    if right >= 0:
        ok &= j <= i + right
    return ok


def allowed_pairs(n: int, causal: bool, window=(-1, -1)) -> int:
    """Number of (query, key) pairs the mask allows for one (batch, head)."""
    return int(allowed_mask(n, causal, window).sum())


def score_matrix_nbytes(n: int, itemsize: int) -> int:
    """Bytes the definition materialises for S of one (batch, head): N x N elements."""
    return n * n * itemsize


def _scores(q, k, scale, ok):
    s = scale * (q @ k.T)
    return np.where(ok, s, -np.inf)


def _softmax_rows(s):
    """Row softmax with the row maximum subtracted first ([A100] §2.2 ``safe_softmax``).

    Returns (P, m, l): probabilities, row max and row sum of exp(S - m).
    Fully masked rows give P = 0, m = -inf, l = 0.
    """
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])            # exp(-inf) = 0 at masked entries
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l[:, None] > 0, e / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return p, m, l


def attention_forward(q, k, v, scale: float, causal: bool = False, window=(-1, -1)):
    """One (batch, head): q, k, v float64 [N, d] -> (O [N, d], LSE [N]).

    S and P are materialised in full, exactly as the naive three-pass computation of
    [A100] §1 does.
    """
    return attention_forward_rows(q, k, v, scale, causal, window, rows=None)


def attention_forward_rows(q, k, v, scale: float, causal: bool = False, window=(-1, -1),
                           rows=None):
    """The definition restricted to the query rows ``rows`` (absolute indices).

    ``q`` holds all N query rows; only the selected rows are evaluated, each one from the
    full key set.  Used to check sampled outputs of large workloads one row at a time.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[0]
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    ok = allowed_mask(n, causal, window, rows=idx)
    s = _scores(q[idx], k, scale, ok)
    p, m, l = _softmax_rows(s)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool = False, window=(-1, -1)):
    """One (batch, head): gradients (dQ, dK, dV) of <dO, O> for the definition above.

        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))        (softmax Jacobian applied row by row)
        dQ = scale * dS K,   dK = scale * dS^T Q

    P is recomputed from Q and K here too; nothing from a forward call is reused.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = k.shape[0]
    ok = allowed_mask(n, causal, window)
    p, _, _ = _softmax_rows(_scores(q, k, scale, ok))
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_forward_bh(q, k, v, scale, causal=False, window=(-1, -1)):
    """[B, H, N, d] arrays -> (O [B, H, N, d], LSE [B, H, N]), one head at a time."""
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_forward(q[b, h], k[b, h], v[b, h], scale, causal, window)
    return o, lse


def attention_backward_bh(q, k, v, do, scale, causal=False, window=(-1, -1)):
    """[B, H, N, d] arrays -> (dQ, dK, dV), one head at a time."""
    B, H = q.shape[:2]
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = attention_backward(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, window)
    return dq, dk, dv
