"""Decode steps over an FP8 key/value cache — test infrastructure.

Sources: FP8 support is among the next steps the A100 page lists (§6, future directions); the
cache a decode step reads is the KV cache of LLM inference named by the FA3.7 page (§1.3) and
paged through memory by PagedAttention (closing section of the PyTorch-CUDA-v2.9 page).  The
pages fix no 8-bit format.  Reading: keys and values are stored as E4M3 codes of the OCP 8-bit
floating-point specification (the FP8 of current accelerators): bit 7 the sign, bits 6..3 the
exponent e with bias 7, bits 2..0 the mantissa m,
    value = (-1)^sign * 2^(e - 7) * (1 + m / 8)   for e > 0,
    value = (-1)^sign * 2^(-6) * (m / 8)          for e = 0 (subnormal),
no infinities, and e = 15 with m = 7 is NaN (largest finite magnitude 448).  Each tensor has
one descale factor: key element = k_descale * value(code), value element = v_descale *
value(code).  The attention over those exact values is ``cross_forward`` (queries at the last
N_q key positions).

The FP8 forward (``fp8_forward``) reads queries, keys and values as E4M3 codes, each tensor with
its own descale: element = descale * value(code).  Its result is the attention of
``attention.attention_forward`` over those exact values, with the usual masks: the definition
fixes no intermediate format, so how a kernel rounds the probabilities before the product with V
is part of its error, not of the reference.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_forward, attention_forward_rows
from .cross import cross_forward


def e4m3_value(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8 array-like) from the definition above."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def fp8_cache_forward(q, k_codes, v_codes, scale, k_descale, v_descale, causal=False,
                      window=(-1, -1), key_mask=None):
    """One (batch, head): q float64 [N_q, d], k_codes / v_codes uint8 [N_k, d] ->
    (O [N_q, d], LSE [N_q]) over K = k_descale * value(k_codes), V = v_descale * value(v_codes);
    ``key_mask`` [N_k] (True = padding key) as in ``cross_forward``."""
    k = float(k_descale) * e4m3_value(k_codes)
    v = float(v_descale) * e4m3_value(v_codes)
    return cross_forward(q, k, v, scale, causal, window, key_mask=key_mask)


def fp8_cache_forward_bh(q, k_codes, v_codes, scale, k_descale, v_descale, causal=False,
                         window=(-1, -1), key_padding_mask=None):
    """[B, H, N_q, d] q, [B, H, N_k, d] codes -> (O [B, H, N_q, d], LSE [B, H, N_q]);
    ``key_padding_mask`` [B, N_k] or None."""
    B, H, n_q, d = q.shape
    o = np.empty((B, H, n_q, d))
    lse = np.empty((B, H, n_q))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = fp8_cache_forward(
                q[b, h], k_codes[b, h], v_codes[b, h], scale, k_descale, v_descale, causal, window,
                None if key_padding_mask is None else key_padding_mask[b])
    return o, lse


def fp8_forward(q_codes, k_codes, v_codes, scale, q_descale, k_descale, v_descale, causal=False,
                window=(-1, -1), rows=None):
    """One (batch, head) of the FP8 forward: codes [N, d] (uint8) -> (O [N, d], LSE [N]) of the
    attention over Q = q_descale value(q_codes), K = k_descale value(k_codes),
    V = v_descale value(v_codes); ``rows`` restricts it to those query rows."""
    q = float(q_descale) * e4m3_value(q_codes)
    k = float(k_descale) * e4m3_value(k_codes)
    v = float(v_descale) * e4m3_value(v_codes)
    if rows is None:
        return attention_forward(q, k, v, scale, causal, window)
    return attention_forward_rows(q, k, v, scale, causal, window, rows=rows)
