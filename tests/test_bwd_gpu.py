"""Backward parity on the GPU: dQ, dK, dV from the recomputing kernels (C ABI) against the
float64 oracle's derivative, each within 2e-2 relative L2 per tensor."""
import math
import os

import numpy as np
import pytest

import workloads as W
from gpu_util import GRAD_REL_L2, rel_l2, say, to64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_125_amd as fa
    return fa


def run(fa, inp, scale, causal, window, stages=None, kernel=None):
    """Forward then backward through the C ABI.  ``kernel`` ("main" / "basic") forces the
    library's dK/dV and dQ kernels through its FA_BWD_KERNEL knob; None keeps the default."""
    import torch
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, scale, causal, window)
    old = os.environ.get("FA_BWD_KERNEL")
    if kernel is not None:
        os.environ["FA_BWD_KERNEL"] = kernel
    try:
        if stages is None:
            grads = fa.bwd(do, q, k, v, o, lse, scale, causal, window)
        else:
            dq, dk, dv = (torch.empty_like(q) for _ in range(3))
            ws = torch.empty(max(fa.bwd_workspace_size(*q.shape), 16), device="cuda",
                             dtype=torch.uint8)
            for st in stages:
                fa.bwd(do, q, k, v, o, lse, scale, causal, window, dq=dq, dk=dk, dv=dv,
                       workspace=ws, stages=st)
            grads = (dq, dk, dv)
        torch.cuda.synchronize()
    finally:
        if kernel is not None:
            if old is None:
                os.environ.pop("FA_BWD_KERNEL", None)
            else:
                os.environ["FA_BWD_KERNEL"] = old
    return grads


KERNELS = ["main", "basic"]   # the two kernel sets (dK/dV, dQ); the default is covered too


def check_grads(grads, inp, scale, causal, window, heads=None, label=""):
    import oracle
    B, H = inp["q64"].shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    got = [to64(g) for g in grads]
    ref = [[], [], []]
    mine = [[], [], []]
    do_norm = float(np.linalg.norm(np.stack([inp["do64"][b, h] for b, h in heads])))
    for b, h in heads:
        r = oracle.attention_backward(inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h],
                                      inp["do64"][b, h], scale, causal, window)
        for t in range(3):
            ref[t].append(r[t])
            mine[t].append(got[t][b, h])
    errs = [rel_l2(np.stack(mine[t]), np.stack(ref[t]), floor=1e-3 * do_norm) for t in range(3)]
    say(f"{label}: rel L2 dQ={errs[0]:.2e} dK={errs[1]:.2e} dV={errs[2]:.2e}")
    for name, e in zip(("dQ", "dK", "dV"), errs):
        assert e <= GRAD_REL_L2, f"{label} {name} rel L2 {e:.3e} > {GRAD_REL_L2}"
    return errs


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiny_workload_backward(fa, dtype):
    w = W.TINY
    inp = W.make_inputs(w, dtype=dtype, with_grad=True)
    grads = run(fa, inp, w.softmax_scale, w.causal, w.window)
    check_grads(grads, inp, w.softmax_scale, w.causal, w.window, label=f"tiny {dtype}")


def test_train_workload_backward_basic_kernels(fa):
    """The full fwd+bwd workload (B=8, H=16, N=4096, d=64, causal, bf16) through the four-wave
    backward kernels, last head against the oracle (the default kernels are checked on every
    head in test_full_size_gpu.py)."""
    w = W.TRAIN
    inp = W.make_inputs(w)
    say(f"[train] {w.name} basic kernels")
    B, H = w.B, w.H
    basic = run(fa, inp, w.softmax_scale, w.causal, w.window, kernel="basic")
    check_grads(basic, inp, w.softmax_scale, w.causal, w.window, heads=[(B - 1, H - 1)],
                label=w.name + " basic kernels")


# (False, (-1, 64)) and (False, (128, 32)) put band edges on multiples of 32, the case the
# kernels mask with constant lane masks away from the causal diagonal
MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (0, 0)), (False, (7, 3)),
         (True, (50, -1)), (False, (0, 40)), (True, (1024, 0)), (False, (-1, 64)),
         (False, (128, 32))]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("n", [1, 17, 64, 65, 129, 200, 513])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_edge_shapes_backward(fa, n, d, dtype, kernel):
    B, H = (1, 3) if n % 2 else (2, 4)
    inp = W.random_case((B, H, n, d), dtype, seed=2000 + n + d, with_grad=True)
    scale = 1.0 / math.sqrt(d)
    for causal, window in MASKS:
        grads = run(fa, inp, scale, causal, window, kernel=kernel)
        check_grads(grads, inp, scale, causal, window,
                    label=f"{kernel} n={n} d={d} {dtype} causal={causal} window={window}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("scale", [0.0, -0.25, 0.6])
def test_scales_backward(fa, scale, kernel):
    inp = W.random_case((1, 2, 300, 64), "bf16", seed=90, with_grad=True)
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (False, (20, 9))]:
        grads = run(fa, inp, scale, causal, window, kernel=kernel)
        check_grads(grads, inp, scale, causal, window, label=f"{kernel} scale={scale}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("d", [64, 128])
def test_many_key_tiles_backward(fa, d, kernel):
    """Sequences spanning many key and query tiles of either kernel set, with a
    ragged tail, under each mask family."""
    inp = W.random_case((1, 2, 1500, d), "bf16", seed=95 + d, with_grad=True)
    scale = 1.0 / math.sqrt(d)
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (False, (300, 77)),
                           (True, (700, -1))]:
        grads = run(fa, inp, scale, causal, window, kernel=kernel)
        check_grads(grads, inp, scale, causal, window,
                    label=f"{kernel} n=1500 d={d} causal={causal} window={window}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("d", [64, 128])
def test_stages_match_single_call_and_are_deterministic(fa, d, kernel):
    import torch
    inp = W.random_case((2, 4, 333, d), "bf16", seed=91, with_grad=True)
    a = run(fa, inp, None, True, (-1, -1), kernel=kernel)
    b = run(fa, inp, None, True, (-1, -1), kernel=kernel)
    c = run(fa, inp, None, True, (-1, -1), stages=[1, 2, 4], kernel=kernel)
    d = run(fa, inp, None, True, (-1, -1), stages=[1, 6], kernel=kernel)
    for x, y, z, u in zip(a, b, c, d):
        assert torch.equal(x, y) and torch.equal(x, z) and torch.equal(x, u)


def test_autograd_wrapper(fa):
    import torch
    inp = W.random_case((1, 4, 200, 64), "f16", seed=92, with_grad=True)
    q, k, v, do = (to_dev(inp[n]).requires_grad_(n != "do") for n in ("q", "k", "v", "do"))
    o = fa.attention(q, k, v, causal=True)
    o.backward(do)
    ref = run(fa, inp, None, True, (-1, -1))
    for g, r in zip((q.grad, k.grad, v.grad), ref):
        assert torch.equal(g, r)
    check_grads((q.grad, k.grad, v.grad), inp, 1 / 8, True, (-1, -1), label="autograd")


def test_guard_bands_backward(fa):
    import torch
    B, H, N, d = 1, 3, 130, 64
    inp = W.random_case((B, H, N, d), "f16", seed=93, with_grad=True)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, None, True)
    pad, size = 4096, B * H * N * d
    bufs = [torch.full((pad + size + pad,), 5.0, device="cuda", dtype=torch.float16)
            for _ in range(3)]
    views = [b[pad:pad + size].view(B, H, N, d) for b in bufs]
    fa.bwd(do, q, k, v, o, lse, None, True, dq=views[0], dk=views[1], dv=views[2])
    torch.cuda.synchronize()
    for b in bufs:
        assert (b[:pad] == 5).all() and (b[-pad:] == 5).all()
    check_grads(views, inp, 1 / 8, True, (-1, -1), label="guard")


@pytest.mark.parametrize("d", [64, 128])
def test_causal_tile_pairing_backward(fa, d):
    """Grids large enough that the causal dK/dV and dQ kernels pair tile t with tile
    n_tiles-1-t (96 heads, N=1100: 5 key tiles of 256 at d=64, 9 of 128 at d=128, so the middle
    tile pairs with itself); heads at both ends and inside against the oracle."""
    import torch
    inp = W.random_case((1, 96, 1100, d), "bf16", seed=97 + d, with_grad=True)
    grads = run(fa, inp, None, True, (-1, -1))
    for g in grads:
        assert torch.isfinite(g).all()
    check_grads(grads, inp, 1 / math.sqrt(d), True, (-1, -1), heads=[(0, 0), (0, 47), (0, 95)],
                label=f"pairing d={d}")
