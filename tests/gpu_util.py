"""Helpers for the GPU parity tests: run the library, run the oracle, compare.

Tolerances (fixed before any GPU run):
  O     max |O_gpu - O_oracle| <= 2e-3 (fp16), 1e-2 (bf16)
  LSE   max |LSE_gpu - LSE_oracle| <= 1e-3
  grads ||g_gpu - g_oracle||_2 / ||g_oracle||_2 <= 2e-2 for each of dQ, dK, dV
The oracle is float64 on exactly the rounded fp16/bf16 input values.
"""
from __future__ import annotations

import sys

import numpy as np

O_TOL = {"f16": 2e-3, "bf16": 1e-2}
LSE_TOL = 1e-3
GRAD_REL_L2 = 2e-2


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def torch_dtype(name):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16}[name]


def to_dev(t):
    return t.to("cuda")


def to64(t):
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_forward(o_gpu, lse_gpu, q64, k64, v64, scale, causal, window, dtype, heads=None,
                  rows=None, label=""):
    """Compare GPU outputs to the oracle on the listed heads ((b, h) pairs) and rows
    (None = all).  Returns (max |dO|, max |dLSE|)."""
    import oracle
    B, H, N, _ = q64.shape
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    o = to64(o_gpu)
    lse = lse_gpu.detach().to("cpu").numpy().astype(np.float64) if lse_gpu is not None else None
    worst_o = worst_l = 0.0
    for b, h in heads:
        r = np.arange(N) if rows is None else np.asarray(rows(b, h) if callable(rows) else rows)
        ro, rl = oracle.attention_forward_rows(q64[b, h], k64[b, h], v64[b, h], scale, causal,
                                               window, rows=r)
        do = np.abs(o[b, h][r] - ro)
        worst_o = max(worst_o, float(do.max()))
        if lse is not None:
            worst_l = max(worst_l, float(np.abs(lse[b, h][r] - rl).max()))
        if do.max() > O_TOL[dtype]:
            i, c = np.unravel_index(np.argmax(do), do.shape)
            raise AssertionError(
                f"{label} O mismatch at b={b} h={h} row={r[i]} col={c}: gpu={o[b, h][r[i], c]} "
                f"oracle={ro[i, c]} |d|={do.max():.3e} > {O_TOL[dtype]}")
    assert worst_l <= LSE_TOL, f"{label} LSE mismatch {worst_l:.3e} > {LSE_TOL}"
    return worst_o, worst_l


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
