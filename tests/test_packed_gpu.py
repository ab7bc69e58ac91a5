"""Packed batches on the GPU: fa_fwd_packed / fa_bwd_packed ([H, total, d], sequences concatenated
per head, offsets cu_seqlens) through the C ABI.

  * bit-identical to fa_fwd_varlen / fa_bwd_varlen on the same sequences laid out padded (the
    padded path is checked against the oracle in test_varlen_gpu.py);
  * against the float64 packed-batch oracle (oracle.packed_forward / packed_backward) at the
    fixed tolerances;
  * rows no sequence covers keep what the caller put there, in every output.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import GRAD_REL_L2, LSE_TOL, O_TOL, rel_l2, say, to64, to_dev

pytestmark = pytest.mark.gpu

GAP = 5          # rows after the last sequence that no sequence covers
SENTINEL = 7.0


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_125_amd as fa
    return fa


def _pack(x, lens):
    """[B, H, N, d] -> [H, total + GAP, d]: each sample's first L_b rows, concatenated."""
    import torch
    parts = [x[b, :, :L] for b, L in enumerate(lens)]
    gap = torch.full((x.shape[1], GAP, x.shape[3]), float("nan"), dtype=x.dtype, device=x.device)
    return torch.cat(parts + [gap], dim=1).contiguous()


def _run_case(fa, lens, d, dtype, causal, window, seed):
    import torch
    B, H, N = len(lens), 3, max(lens)
    inp = W.random_case((B, H, N, d), dtype, seed=seed, with_grad=True)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    po, plse = fa.fwd(q, k, v, scale, causal, window, seqlens=sl)
    pg = fa.bwd(do, q, k, v, po, plse, scale, causal, window, seqlens=sl)
    cu_list = [0] + list(np.cumsum(lens))
    cu = torch.tensor(cu_list, dtype=torch.int32, device="cuda")
    qp, kp, vp, dop = (_pack(t, lens) for t in (q, k, v, do))
    total = qp.shape[1]
    o = torch.full_like(qp, SENTINEL)
    lse = torch.full((H, total), SENTINEL, dtype=torch.float32, device="cuda")
    fa.fwd_packed(qp, kp, vp, cu, N, scale, causal, window, out=o, lse=lse)
    grads = [torch.full_like(qp, SENTINEL) for _ in range(3)]
    fa.bwd_packed(dop, qp, kp, vp, o, lse, cu, N, scale, causal, window, dq=grads[0],
                  dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    label = f"packed lens={lens} d={d} {dtype} causal={causal} window={window}"
    # bit-identical to the padded call on every covered row; the gap keeps the sentinel
    for b, L in enumerate(lens):
        r = slice(cu_list[b], cu_list[b + 1])
        assert torch.equal(o[:, r], po[b, :, :L]), f"{label}: O differs from the padded call"
        assert torch.equal(lse[:, r], plse[b, :, :L]), f"{label}: LSE differs from the padded call"
        for g, gp in zip(grads, pg):
            assert torch.equal(g[:, r], gp[b, :, :L]), f"{label}: gradient differs"
    for t in [o, lse] + grads:
        assert bool((t[:, total - GAP:] == SENTINEL).all()), f"{label}: a row outside wrote"
    # against the oracle
    q64, k64, v64, do64 = (np.concatenate([inp[n + "64"][b, :, :L] for b, L in enumerate(lens)],
                                          axis=1) for n in ("q", "k", "v", "do"))
    cu_h = cu_list
    ro, rl = oracle.packed_forward(q64, k64, v64, cu_h, N, scale, causal, window)
    rg = oracle.packed_backward(q64, k64, v64, do64, cu_h, N, scale, causal, window)
    n = total - GAP
    d_o = float(np.abs(to64(o[:, :n]) - ro).max())
    d_l = float(np.abs(lse[:, :n].cpu().numpy().astype(np.float64) - rl).max())
    say(f"{label}: max|dO|={d_o:.2e} max|dLSE|={d_l:.2e}")
    assert d_o <= O_TOL[dtype] and d_l <= LSE_TOL, label
    floor = 1e-3 * float(np.linalg.norm(do64))
    for name, g, r in zip(("dq", "dk", "dv"), grads, rg):
        e = rel_l2(to64(g[:, :n]), r, floor)
        assert e <= GRAD_REL_L2, f"{label} {name} rel L2 {e:.3e}"


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (-1, -1)), (True, (64, 0)),
                                           (False, (33, 17))])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16"), (64, "f16"), (128, "bf16")])
def test_packed_matches_padded_and_oracle(fa, d, dtype, causal, window):
    _run_case(fa, [37, 0, 1, 300, 129, 64, 257], d, dtype, causal, window, seed=3100 + d)


def test_packed_many_sequences(fa):
    # grids of many short and a few long sequences (tile pairing off and on)
    rng = np.random.default_rng(3200)
    lens = [int(x) for x in rng.integers(1, 700, size=24)]
    _run_case(fa, lens, 64, "bf16", True, (-1, -1), seed=3201)


def test_packed_empty_and_errors(fa):
    import torch
    z = torch.empty((3, 0, 64), device="cuda", dtype=torch.bfloat16)
    cu = torch.zeros(5, dtype=torch.int32, device="cuda")
    o, lse = fa.fwd_packed(z, z, z, cu, 0)
    assert o.shape == (3, 0, 64) and lse.shape == (3, 0)
    x = torch.zeros((2, 10, 96), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(fa.FaError, match="UNSUPPORTED_HEAD_DIM"):
        fa.fwd_packed(x, x, x, torch.tensor([0, 10], dtype=torch.int32, device="cuda"), 10)


def test_packed_stages_match_single_call(fa):
    """A packed batch's backward in one call (the dQ kernel forming the row statistics) and as
    three separate stages give the same gradients, bit for bit."""
    import torch
    lens = [37, 0, 1, 300, 129]
    B, H, N, d = len(lens), 3, max(lens), 64
    inp = W.random_case((B, H, N, d), "bf16", seed=251, with_grad=True)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda")
    qp, kp, vp, dop = (_pack(t, lens) for t in (q, k, v, do))
    o, lse = fa.fwd_packed(qp, kp, vp, cu, N, None, True)
    one = [torch.zeros_like(qp) for _ in range(3)]
    fa.bwd_packed(dop, qp, kp, vp, o, lse, cu, N, None, True, dq=one[0], dk=one[1], dv=one[2])
    split = [torch.zeros_like(qp) for _ in range(3)]
    ws = torch.empty(fa.bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    for st in (fa._lib.BWD_DELTA, fa._lib.BWD_DKDV, fa._lib.BWD_DQ):
        fa.bwd_packed(dop, qp, kp, vp, o, lse, cu, N, None, True, dq=split[0], dk=split[1], dv=split[2],
                      workspace=ws, stages=st)
    torch.cuda.synchronize()
    for x, y in zip(one, split):
        assert torch.equal(x, y)
