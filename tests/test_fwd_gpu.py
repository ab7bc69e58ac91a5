"""Forward parity on the GPU: the HIP kernels through the C ABI against the float64 oracle."""
import math
import os

import numpy as np
import pytest

import workloads as W
from gpu_util import (LSE_TOL, O_TOL, check_forward, say, to64, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_125_amd as fa
    return fa


def run(fa, inp, scale, causal, window, return_lse=True, kernel=None):
    """Forward through the C ABI.  ``kernel`` ("main" / "basic" / "split") forces the
    library's kernel choice through its FA_FWD_KERNEL knob; None keeps its own heuristic."""
    import torch
    q, k, v = (to_dev(inp[n]) for n in "qkv")
    old = os.environ.get("FA_FWD_KERNEL")
    if kernel is not None:
        os.environ["FA_FWD_KERNEL"] = kernel
    try:
        o, lse = fa.fwd(q, k, v, scale, causal, window, return_lse=return_lse)
        torch.cuda.synchronize()
    finally:
        if kernel is not None:
            if old is None:
                os.environ.pop("FA_FWD_KERNEL", None)
            else:
                os.environ["FA_FWD_KERNEL"] = old
    return o, lse


KERNELS = ["main", "basic", "split"]   # the three forward kernels; the default choice too


def sampled_rows(n, rng, extra=8):
    base = {0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, n // 2, n - 130, n - 129, n - 2, n - 1}
    base |= set(rng.integers(0, n, extra).tolist())
    return sorted(r for r in base if 0 <= r < n)


# --------------------------------------------------------------------------- the workloads
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiny_workload(fa, dtype):
    w = W.TINY
    inp = W.make_inputs(w, dtype=dtype)
    say(f"[tiny] {w.name} as {dtype}")
    o, lse = run(fa, inp, w.softmax_scale, w.causal, w.window)
    err = check_forward(o, lse, inp["q64"], inp["k64"], inp["v64"], w.softmax_scale, w.causal,
                        w.window, dtype, label=w.name)
    say(f"[tiny] max|dO|={err[0]:.3e} max|dLSE|={err[1]:.3e}")


@pytest.mark.parametrize("kernel", [None] + KERNELS)
def test_bert_workload(fa, kernel):
    w = W.BERT
    inp = W.make_inputs(w)
    say(f"[bert] {w.name} kernel={kernel or 'default'}")
    o, lse = run(fa, inp, w.softmax_scale, w.causal, w.window, kernel=kernel)
    err = check_forward(o, lse, inp["q64"], inp["k64"], inp["v64"], w.softmax_scale, w.causal,
                        w.window, w.dtype, label=w.name)
    say(f"[bert] max|dO|={err[0]:.3e} max|dLSE|={err[1]:.3e}")


# The large workloads (every row of every head) are checked in test_full_size_gpu.py.


# --------------------------------------------------------------------------- edge cases
EDGE_MASKS = [
    (False, (-1, -1)), (True, (-1, -1)), (False, (0, 0)), (True, (0, 0)), (False, (3, 5)),
    (True, (40, -1)), (False, (0, 70)), (False, (100, 0)), (True, (1024, 0)),
    (False, (5000, 5000)),
]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("n", [1, 17, 63, 64, 65, 127, 128, 129, 200, 257, 513, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_edge_shapes(fa, n, d, dtype, kernel):
    B, H = (1, 3) if n % 2 else (2, 4)       # n_bh = 3 (not a multiple of 8) or 8
    inp = W.random_case((B, H, n, d), dtype, seed=1000 + n + d)
    scale = 1.0 / math.sqrt(d)
    for causal, window in EDGE_MASKS:
        say(f"[edge] {kernel} n={n} d={d} {dtype} causal={causal} window={window}")
        o, lse = run(fa, inp, scale, causal, window, kernel=kernel)
        check_forward(o, lse, inp["q64"], inp["k64"], inp["v64"], scale, causal, window, dtype,
                      label=f"{kernel} n={n} d={d} {dtype} causal={causal} window={window}",
                      rounding="edge")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("scale", [0.0, -0.125, None, -0.3, 0.5])
def test_scales(fa, scale, kernel):
    # |scale| above 1/sqrt(d) sharpens the softmax beyond the workloads' statistics: those
    # cases are checked against the derived rounding bound (tests/gpu_util.py)
    inp = W.random_case((1, 2, 300, 64), "bf16", seed=77)
    s = 1 / 8 if scale is None else scale
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (False, (20, 9))]:
        o, lse = run(fa, inp, scale, causal, window, kernel=kernel)
        check_forward(o, lse, inp["q64"], inp["k64"], inp["v64"], s, causal, window, "bf16",
                      label=f"{kernel} scale={scale}", derived_bound=abs(s) > 1 / 8)


@pytest.mark.parametrize("kernel", KERNELS)
def test_peaked_scores(fa, kernel):
    # large |q.k| (near one-hot softmax rows) stresses the running-max rescaling
    inp = W.random_case((1, 2, 500, 128), "f16", seed=78)
    import torch
    q = inp["q"] * 6
    inp2 = dict(inp, q=q, q64=q.to(torch.float64).numpy())
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (True, (64, 0))]:
        o, lse = run(fa, inp2, 0.25, causal, window, kernel=kernel)
        check_forward(o, lse, inp2["q64"], inp2["k64"], inp2["v64"], 0.25, causal, window, "f16",
                      label=f"{kernel} peaked", derived_bound=True)


def test_q_equals_k_equals_v(fa):
    # the demo configuration of "显存神技：必学FlashAttention！" §三 (k and v cloned from q)
    inp = W.random_case((2, 8, 512, 64), "f16", seed=79)
    same = dict(q=inp["q"], k=inp["q"], v=inp["q"], q64=inp["q64"], k64=inp["q64"],
                v64=inp["q64"])
    o, lse = run(fa, same, None, False, (-1, -1))
    check_forward(o, lse, same["q64"], same["k64"], same["v64"], 1 / 8, False, (-1, -1), "f16",
                  label="q=k=v")


@pytest.mark.parametrize("kernel", KERNELS)
def test_deterministic_and_lse_optional(fa, kernel):
    import torch
    inp = W.random_case((2, 8, 777, 128), "bf16", seed=80)
    o1, l1 = run(fa, inp, None, True, (100, 0), kernel=kernel)
    o2, l2 = run(fa, inp, None, True, (100, 0), kernel=kernel)
    o3, none = run(fa, inp, None, True, (100, 0), return_lse=False, kernel=kernel)
    assert none is None
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o3)


def test_causal_pairing_and_many_tiles(fa):
    """A causal launch large enough for the main kernel to pair query tiles (and a windowed
    one, which it does not pair), checked on rows of every query tile of several heads."""
    import numpy as np
    for (B, H, N, d, causal, window, seed) in [(2, 64, 1536, 64, True, (-1, -1), 82),
                                               (2, 64, 1536, 128, True, (300, 0), 83),
                                               (1, 128, 1100, 64, False, (-1, -1), 84)]:
        inp = W.random_case((B, H, N, d), "bf16", seed=seed)
        o, lse = run(fa, inp, None, causal, window)
        rows = sorted(set(list(range(0, N, 97)) + [N - 1, 255, 256, 511, 512]))
        heads = [(0, 0), (B - 1, H - 1), (0, H // 2), (B - 1, 3)]
        check_forward(o, lse, inp["q64"], inp["k64"], inp["v64"], 1 / math.sqrt(d), causal, window,
                      "bf16", heads=heads, rows=rows, label=f"pairing N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rem", [0, 1, 2, 3])
def test_key_tile_count_remainders(fa, d, rem):
    """The main kernel's key loop runs in groups of four tiles and then 0-3 single tiles before
    the last one: sequences whose tile count leaves each remainder, with a ragged last tile,
    without and with a causal mask."""
    bc = 64 if d == 64 else 32                      # keys per tile of the main kernel
    n = bc * (4 * 2 + rem + 1) - 5
    inp = W.random_case((1, 2, n, d), "bf16", seed=300 + 10 * d + rem)
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (False, (2 * bc + 3, 0))]:
        o, lse = run(fa, inp, None, causal, window, kernel="main")
        check_forward(o, lse, inp["q64"], inp["k64"], inp["v64"], 1 / math.sqrt(d), causal, window,
                      "bf16", label=f"remainder {rem} n={n} d={d} causal={causal} window={window}")


def test_guard_bands_untouched(fa):
    import torch
    B, H, N, d = 1, 3, 130, 64
    inp = W.random_case((B, H, N, d), "f16", seed=81)
    q, k, v = (to_dev(inp[n]) for n in "qkv")
    pad = 4096
    obuf = torch.full((pad + B * H * N * d + pad,), 7.0, device="cuda", dtype=torch.float16)
    lbuf = torch.full((pad + B * H * N + pad,), 7.0, device="cuda", dtype=torch.float32)
    o = obuf[pad:pad + B * H * N * d].view(B, H, N, d)
    lse = lbuf[pad:pad + B * H * N].view(B, H, N)
    fa.fwd(q, k, v, None, True, (-1, -1), out=o, lse=lse)
    torch.cuda.synchronize()
    assert (obuf[:pad] == 7).all() and (obuf[-pad:] == 7).all()
    assert (lbuf[:pad] == 7).all() and (lbuf[-pad:] == 7).all()
    check_forward(o, lse, inp["q64"], inp["k64"], inp["v64"], 1 / 8, True, (-1, -1), "f16",
                  label="guard")


def test_empty(fa):
    import torch
    q = torch.empty((2, 3, 0, 64), device="cuda", dtype=torch.float16)
    o, lse = fa.fwd(q, q, q)
    assert o.shape == q.shape and lse.shape == (2, 3, 0)


def test_errors_surface(fa):
    import torch
    q = torch.zeros((1, 1, 8, 96), device="cuda", dtype=torch.float16)
    with pytest.raises(fa.FaError, match="UNSUPPORTED_HEAD_DIM"):
        fa.fwd(q, q, q)
    q = torch.zeros((1, 1, 8, 64), device="cuda", dtype=torch.float16)
    with pytest.raises(fa.FaError, match="BAD_WINDOW"):
        fa.fwd(q, q, q, window_size=(-3, 0))
