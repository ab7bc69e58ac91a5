"""Scalar brute-force attention on tiny shapes — test infrastructure.

Pure-Python floats and explicit loops; no numpy arithmetic.  It evaluates the
softmax as written in the formula softmax(QK^T/sqrt(d_k))V ([PT29], section
"FlashAttention：不只是更快的 Attention") *without* the row-maximum shift:

    w_ij = exp(s_ij) / sum_{j' allowed} exp(s_ij'),    s_ij = scale * sum_c q_ic k_jc
    O_i  = sum_j w_ij v_j,      LSE_i = ln(sum_j exp(s_ij))

Because it skips the shift it only works where exp does not overflow (tiny |s|);
that is the point: agreement with the shifted definition pins the claim of [A100]
§2.2 that subtracting the maximum leaves the softmax unchanged.  Sums use math.fsum.
Mask reading: inclusive bounds, -1 unbounded, causal AND window.
"""
from __future__ import annotations

import math


def _visible(i: int, j: int, causal: bool, left: int, right: int) -> bool:
    if causal and j > i:
        return False
    if left >= 0 and j < i - left:
        return False
    if right >= 0 and j > i + right:
        return False
    return True


def attention_forward_brute(q, k, v, scale: float, causal: bool = False, window=(-1, -1)):
    """q, k, v: nested lists (or arrays) [N][d]. Returns (O as list [N][dv], LSE list [N])."""
    n = len(k)
    left, right = int(window[0]), int(window[1])
    out, lse = [], []
    for i in range(n):
        js = [j for j in range(n) if _visible(i, j, causal, left, right)]
        if not js:
            out.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        e = {}
        for j in js:
            s = scale * math.fsum(float(q[i][c]) * float(k[j][c]) for c in range(len(q[i])))
            e[j] = math.exp(s)
        z = math.fsum(e.values())
        row = [math.fsum(e[j] / z * float(v[j][c]) for j in js) for c in range(len(v[0]))]
        out.append(row)
        lse.append(math.log(z))
    return out, lse
