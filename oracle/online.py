"""The tiled forward with a running max and running sum — test infrastructure.

Follows the tiling of [A100] §2.1 (S_ij = Q_i K_j^T per tile, O_i accumulated tile by
tile) with the running-max / running-sum update of [A100] §2.2, and [FA37] §3.1's
description: load one query block, loop over the key/value blocks, update the output
and the normalisation factors, write only the result.

Readings (the printed update lost its operators in extraction, and the printed tile
loop omits the rescaling):
  m_new   = max(m_old, max_j s_j)
  alpha   = exp(m_old - m_new)                      (0 when m_old = -inf)
  l_new   = alpha * l_old + sum_j exp(s_j - m_new)
  acc_new = alpha * acc_old + sum_j exp(s_j - m_new) v_j
  O = acc / l and LSE = m + ln(l) once, after the last tile.
The query-block-outer / key-block-inner order is used (the key-outer order printed
in [A100] §2.1 yields the same numbers).  Key blocks that the mask hides entirely
are skipped; partly hidden blocks get -inf where hidden.  All arithmetic in float64.
"""
from __future__ import annotations

import numpy as np


def _block_visible(i0, i1, j0, j1, causal, left, right):
    """Whether any (i, j) with i0 <= i < i1, j0 <= j < j1 is allowed."""
    if causal and j0 > i1 - 1:
        return False
    if left >= 0 and j1 - 1 < i0 - left:
        return False
    if right >= 0 and j0 > i1 - 1 + right:
        return False
    return True


def attention_forward_online(q, k, v, scale: float, causal: bool = False, window=(-1, -1),
                             block_q: int = 64, block_k: int = 64, return_visits: bool = False):
    """One (batch, head): float64 [N, d] arrays -> (O, LSE) by the tiled recurrence.

    With ``return_visits`` also returns the list of (query block, key block) pairs that
    were processed, so tile-skipping can be checked.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[0]
    left, right = int(window[0]), int(window[1])
    o = np.zeros((q.shape[0], v.shape[1]))
    lse = np.full(q.shape[0], -np.inf)
    visits = []
    for i0 in range(0, n, block_q):
        i1 = min(i0 + block_q, n)
        ii = np.arange(i0, i1)[:, None]
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        acc = np.zeros((i1 - i0, v.shape[1]))
        for j0 in range(0, n, block_k):
            j1 = min(j0 + block_k, n)
            if not _block_visible(i0, i1, j0, j1, causal, left, right):
                continue
            visits.append((i0 // block_q, j0 // block_k))
            jj = np.arange(j0, j1)[None, :]
            s = scale * (q[i0:i1] @ k[j0:j1].T)
            hide = np.zeros(s.shape, dtype=bool)
            if causal:
                hide |= jj > ii
            if left >= 0:
                hide |= jj < ii - left
            if right >= 0:
                hide |= jj > ii + right
            s = np.where(hide, -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            # rows still without any visible key keep m = -inf; shift by 0 there
            shift = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - shift), 0.0)
            p = np.exp(s - shift[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[j0:j1]
            m = m_new
        seen = l > 0
        o[i0:i1] = np.where(seen[:, None], acc / np.where(seen, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            lse[i0:i1] = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return (o, lse, visits) if return_visits else (o, lse)
