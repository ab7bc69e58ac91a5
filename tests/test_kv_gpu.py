"""N_q queries over N_k keys on the GPU: fa_fwd_kv through the C ABI against the float64 oracle
(oracle/cross.py), with the fixed tolerances (max |dO| 2e-3 fp16 / 1e-2 bf16, |dLSE| 1e-3).

Covers the few-query kernel (N_q <= 4) and the MFMA kernel, with and without key splits,
every mask mode, rows that see no key, strided operands ([B, N, H, d] memory, a key/value
head shared by every head), and sampled rows of the decode workloads at full size."""
import math

import numpy as np
import pytest

import workloads as W
from gpu_util import GRAD_REL_L2, LSE_TOL, O_TOL, UNIT_ROUNDOFF, rel_l2, say, to64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_125_amd as fa
    return fa


def compare(o, lse, inp, scale, causal, window, dtype, label, heads=None, slopes=None,
            block_mask=None, edge=False):
    """``edge``: the edge-shape rule of gpu_util (an element over the fixed tolerance passes
    if it is within the derived rounding bound and one step of the output type from the
    correctly rounded oracle value), for rows whose weight sits on a few keys."""
    import oracle
    from gpu_util import ulp_distance
    q64, k64, v64 = inp["q64"], inp["k64"], inp["v64"]
    B, H = q64.shape[:2]
    o64 = to64(o)
    l64 = lse.detach().cpu().numpy().astype(np.float64)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    worst_o = worst_l = 0.0
    n_edge = 0
    for b, h in heads:
        slope = 0.0 if slopes is None else float(slopes[h])
        bm = None if block_mask is None else block_mask[h]
        ro, rl = oracle.cross_forward(q64[b, h], k64[b, h], v64[b, h], scale, causal, window,
                                      slope, bm)
        empty = np.isneginf(rl)
        assert np.array_equal(np.isneginf(l64[b, h]), empty), f"{label}: rows without keys differ"
        assert np.all(o64[b, h][empty] == 0.0), f"{label}: O of a row without keys is not 0"
        diff = np.abs(o64[b, h] - ro)
        over = diff > O_TOL[dtype]
        if edge and over.any():
            wabs, _ = oracle.cross_forward(q64[b, h], k64[b, h], np.abs(v64[b, h]), scale, causal,
                                           window, slope, bm)
            derived = UNIT_ROUNDOFF[dtype] * (wabs + np.abs(ro)) + 1e-5
            ok = over & (diff <= derived) & (ulp_distance(o64[b, h], ro, dtype) <= 1)
            n_edge += int(ok.sum())
            diff = np.where(ok, 0.0, diff)
        d_o = float(diff.max()) if ro.size else 0.0
        d_l = float(np.abs(l64[b, h][~empty] - rl[~empty]).max()) if (~empty).any() else 0.0
        worst_o, worst_l = max(worst_o, d_o), max(worst_l, d_l)
    say(f"{label}: max|dO|={worst_o:.2e} max|dLSE|={worst_l:.2e}"
        + (f" ({n_edge} element(s) representation-limited)" if n_edge else ""))
    assert worst_o <= O_TOL[dtype], f"{label}: max|dO| {worst_o:.3e} > {O_TOL[dtype]}"
    assert worst_l <= LSE_TOL, f"{label}: max|dLSE| {worst_l:.3e} > {LSE_TOL}"


def run_case(fa, B, H, n_q, n_k, d, dtype, causal, window, seed, scale=None, layout="bhnd",
             slopes=None):
    import torch
    inp = W.cross_case(B, H, n_q, n_k, d, dtype, seed)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if layout == "bhnd":
        q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    else:   # [B, N, H, d] memory seen as [B, H, N, d] views
        q, k, v = (to_dev(inp[n].transpose(1, 2).contiguous()).transpose(1, 2)
                   for n in ("q", "k", "v"))
        assert k.stride(1) == d and k.stride(2) == H * d   # rows H heads apart
    sl = None if slopes is None else torch.tensor(slopes, dtype=torch.float32, device="cuda")
    o, lse = fa.fwd_kv(q, k, v, scale, causal, window, alibi_slopes=sl)
    torch.cuda.synchronize()
    if layout != "bhnd" and n_q > 1:   # a length-1 dimension makes any view contiguous
        assert not q.is_contiguous() and o.stride() == q.stride()
    return o, lse, inp, scale


MASKS = [(False, (-1, -1)), (True, (-1, -1)), (True, (300, 0)), (False, (100, 40)),
         (False, (-1, 0))]


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("n_q", [1, 2, 3, 4])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_few_queries(fa, causal, window, n_q, d, dtype):
    for n_k, seed in ((1, 1), (77, 2), (1000, 3), (4099, 4)):
        o, lse, inp, scale = run_case(fa, 2, 3, n_q, n_k, d, dtype, causal, window, seed)
        compare(o, lse, inp, scale, causal, window, dtype,
                f"decode nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}")


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("n_q,n_k", [(5, 50), (100, 700), (300, 129), (130, 3000)])
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (128, "bf16")])
def test_many_queries(fa, causal, window, n_q, n_k, d, dtype):
    o, lse, inp, scale = run_case(fa, 2, 2, n_q, n_k, d, dtype, causal, window, seed=n_q + n_k)
    compare(o, lse, inp, scale, causal, window, dtype,
            f"mfma nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}")


@pytest.mark.parametrize("n_q,n_k", [(1, 20000), (3, 9000), (128, 8192), (200, 5000)])
@pytest.mark.parametrize("d", [64, 128])
def test_key_splits(fa, n_q, n_k, d):
    """One (batch, head): the plan splits the keys, and the merge must reproduce the whole."""
    from exact_attention_125_amd import _lib
    assert _lib.fwd_kv_workspace_size(1, 1, n_q, n_k, d) > 0
    for causal, window in ((True, (-1, -1)), (False, (-1, -1)), (True, (2500, 0))):
        o, lse, inp, scale = run_case(fa, 1, 1, n_q, n_k, d, "bf16", causal, window, seed=n_k)
        compare(o, lse, inp, scale, causal, window, "bf16",
                f"split nq={n_q} nk={n_k} d={d} causal={causal} w={window}")


@pytest.mark.parametrize("n_q,n_k", [(4, 2), (7, 3), (300, 100)])
def test_rows_without_keys(fa, n_q, n_k):
    o, lse, inp, scale = run_case(fa, 1, 2, n_q, n_k, 64, "bf16", True, (-1, -1), seed=9)
    compare(o, lse, inp, scale, True, (-1, -1), "bf16", f"empty rows nq={n_q} nk={n_k}")
    l64 = lse.cpu().numpy()
    assert np.all(np.isneginf(l64[:, :, :n_q - n_k])) and np.all(np.isfinite(l64[:, :, n_q - n_k:]))


def test_no_keys(fa):
    import torch
    q = torch.randn(2, 3, 5, 64, device="cuda").to(torch.bfloat16)
    k = torch.empty(2, 3, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = fa.fwd_kv(q, k, k, 0.125)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("n_q,n_k", [(1, 3000), (4, 500), (64, 1000), (257, 257)])
def test_strided_bnhd_layout(fa, n_q, n_k):
    for causal in (False, True):
        o, lse, inp, scale = run_case(fa, 2, 4, n_q, n_k, 128, "bf16", causal, (-1, -1),
                                      seed=11 + n_q, layout="bnhd")
        compare(o, lse, inp, scale, causal, (-1, -1), "bf16", f"bnhd nq={n_q} nk={n_k} c={causal}")


@pytest.mark.parametrize("n_q", [1, 3, 96])
def test_shared_key_value_head(fa, n_q):
    """k, v with head stride 0: every query head attends to one key/value head."""
    import torch
    B, H, n_k, d = 2, 4, 1500, 64
    inp = W.cross_case(B, 1, n_q, n_k, d, "f16", seed=21)
    qin = W.cross_case(B, H, n_q, 1, d, "f16", seed=22)
    q = to_dev(qin["q"])
    k = to_dev(inp["k"]).expand(B, H, n_k, d)
    v = to_dev(inp["v"]).expand(B, H, n_k, d)
    assert k.stride(1) == 0
    o, lse = fa.fwd_kv(q, k, v, 0.125, True)
    torch.cuda.synchronize()
    full = {"q64": qin["q64"], "k64": np.repeat(inp["k64"], H, axis=1),
            "v64": np.repeat(inp["v64"], H, axis=1)}
    compare(o, lse, full, 0.125, True, (-1, -1), "f16", f"shared kv head nq={n_q}")


def test_square_case_matches_the_oracle(fa):
    """N_q = N_k through fa_fwd_kv is plain self-attention."""
    for causal, window in ((True, (-1, -1)), (False, (64, 64))):
        o, lse, inp, scale = run_case(fa, 1, 4, 700, 700, 64, "bf16", causal, window, seed=31)
        compare(o, lse, inp, scale, causal, window, "bf16", f"square causal={causal} w={window}")


def test_negative_and_zero_scale(fa):
    for scale in (-0.2, 0.0):
        for n_q in (2, 40):
            o, lse, inp, _ = run_case(fa, 1, 2, n_q, 900, 64, "f16", True, (-1, -1), seed=41,
                                      scale=scale)
            compare(o, lse, inp, scale, True, (-1, -1), "f16", f"scale={scale} nq={n_q}")


def test_deterministic(fa):
    import torch
    inp = W.cross_case(2, 2, 1, 9000, 128, "bf16", seed=51)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    o1, l1 = fa.fwd_kv(q, k, v, None, True)
    o2, l2 = fa.fwd_kv(q, k, v, None, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("w", W.DECODES, ids=lambda w: w.name)
def test_decode_workload_sampled(fa, w):
    """The bench's decode workloads at full size, in the launch configuration the bench times;
    every row of a sample of heads is checked against the oracle."""
    import torch
    inp = W.cross_case(w.B, w.H, w.n_q, w.n_k, w.d, w.dtype, w.seed)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    o, lse = fa.fwd_kv(q, k, v, w.softmax_scale, True)
    torch.cuda.synchronize()
    heads = [(b, (5 * b + 3) % w.H) for b in range(w.B)] + [(w.B - 1, w.H - 1)]
    compare(o, lse, inp, w.softmax_scale, True, (-1, -1), w.dtype, w.name, heads=heads)


# ---------------------------------------------------------------------------- backward
def run_backward(fa, B, H, n_q, n_k, d, dtype, causal, window, seed, layout="bhnd", slopes=None):
    """fa_fwd_kv then fa_bwd_kv on seeded inputs (dO drawn after q, k, v from its own seed);
    gradients against the oracle's by relative L2 per tensor over all heads."""
    import oracle
    import torch
    inp = W.cross_case(B, H, n_q, n_k, d, dtype, seed)
    dout_in = W.cross_case(B, H, n_q, 1, d, dtype, seed + 1000)
    scale = 1.0 / math.sqrt(d)
    if layout == "bhnd":
        q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], dout_in["q"]))
    else:
        q, k, v, do = (to_dev(t.transpose(1, 2).contiguous()).transpose(1, 2)
                       for t in (inp["q"], inp["k"], inp["v"], dout_in["q"]))
    sl = None if slopes is None else torch.tensor(slopes, dtype=torch.float32, device="cuda")
    o, lse = fa.fwd_kv(q, k, v, scale, causal, window, alibi_slopes=sl)
    dq, dk, dv = fa.bwd_kv(do, q, k, v, o, lse, scale, causal, window, alibi_slopes=sl)
    torch.cuda.synchronize()
    if layout != "bhnd":
        assert dk.stride() == k.stride() and dq.stride() == q.stride()
    rq, rk, rv = oracle.cross_backward_bh(inp["q64"], inp["k64"], inp["v64"], dout_in["q64"],
                                          scale, causal, window, slopes)
    floor = 1e-3 * float(np.linalg.norm(dout_in["q64"]))
    errs = [rel_l2(to64(g), r, floor) for g, r in ((dq, rq), (dk, rk), (dv, rv))]
    say(f"bwd nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window} {layout}: "
        f"rel L2 dq={errs[0]:.2e} dk={errs[1]:.2e} dv={errs[2]:.2e}")
    for name, e in zip(("dq", "dk", "dv"), errs):
        assert e <= GRAD_REL_L2, f"{name} rel L2 {e:.3e} > {GRAD_REL_L2}"
    return dq, dk, dv


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("n_q,n_k", [(1, 300), (4, 1000), (100, 700), (300, 129), (130, 3000),
                                     (257, 257)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_backward(fa, causal, window, n_q, n_k, d, dtype):
    run_backward(fa, 2, 2, n_q, n_k, d, dtype, causal, window, seed=n_q * 7 + n_k)


@pytest.mark.parametrize("n_q,n_k", [(64, 1000), (3, 500)])
def test_backward_strided(fa, n_q, n_k):
    for causal in (False, True):
        run_backward(fa, 2, 4, n_q, n_k, 128, "bf16", causal, (-1, -1), seed=77, layout="bnhd")


def test_backward_rows_without_keys(fa):
    import torch
    dq, dk, dv = run_backward(fa, 1, 2, 300, 100, 64, "bf16", True, (-1, -1), seed=88)
    assert torch.all(dq[:, :, :200] == 0)


def test_backward_empty_sides(fa):
    import torch
    q = torch.randn(1, 2, 5, 64, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, 2, 0, 64, device="cuda").to(torch.bfloat16)
    o, lse = fa.fwd_kv(q, k, k, 0.125)
    dq, _, _ = fa.bwd_kv(torch.ones_like(q), q, k, k, o, lse, 0.125)
    q0 = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    k1 = torch.randn(1, 2, 40, 64, device="cuda").to(torch.bfloat16)
    o0, lse0 = fa.fwd_kv(q0, k1, k1, 0.125)
    _, dk, dv = fa.bwd_kv(q0, q0, k1, k1, o0, lse0, 0.125)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


def test_backward_deterministic(fa):
    import torch
    inp = W.cross_case(2, 2, 200, 900, 64, "bf16", seed=99)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    do = torch.ones_like(q)
    o, lse = fa.fwd_kv(q, k, v, None, True)
    g1 = fa.bwd_kv(do, q, k, v, o, lse, None, True)
    g2 = fa.bwd_kv(do, q, k, v, o, lse, None, True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


# ---------------------------------------------------------------------------- ALiBi
def alibi_slopes(H):
    """The geometric slopes 2^(-8 h / H), h = 1 .. H, and one steep slope first."""
    return [0.5] + [2.0 ** (-8.0 * h / H) for h in range(2, H + 1)]


ALIBI_MASKS = [(False, (-1, -1)), (True, (-1, -1)), (True, (300, 0)), (False, (100, 40))]


@pytest.mark.parametrize("causal,window", ALIBI_MASKS)
@pytest.mark.parametrize("n_q,n_k", [(1, 77), (3, 4099), (1, 20000), (100, 700), (300, 129),
                                     (128, 8192), (257, 257)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_alibi_forward(fa, causal, window, n_q, n_k, d, dtype):
    sl = alibi_slopes(4)
    o, lse, inp, scale = run_case(fa, 1, 4, n_q, n_k, d, dtype, causal, window, seed=n_q + 3 * n_k,
                                  slopes=sl)
    compare(o, lse, inp, scale, causal, window, dtype,
            f"alibi nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}", slopes=sl)


@pytest.mark.parametrize("causal,window", ALIBI_MASKS)
@pytest.mark.parametrize("n_q,n_k", [(1, 300), (100, 700), (300, 129), (257, 257)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_alibi_backward(fa, causal, window, n_q, n_k, d, dtype):
    run_backward(fa, 1, 4, n_q, n_k, d, dtype, causal, window, seed=5 * n_q + n_k,
                 slopes=alibi_slopes(4))


# Grids of at least 256 query tiles of 128 rows with one key split (B H ceil(N_q / 128) >= 512,
# or >= 256 with N_k <= 1024) and dense operands: the forward takes the ALiBi instance of the
# main kernel; the backward stays on the four-wave kernels.
ALIBI_MAIN_MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (100, 40)), (True, (300, 0)),
                    (False, (-1, 0)), (False, (0, -1))]


@pytest.mark.parametrize("causal,window", ALIBI_MAIN_MASKS)
@pytest.mark.parametrize("n_q,n_k", [(512, 512), (512, 2048), (300, 1000), (513, 700)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_alibi_forward_main_kernel(fa, causal, window, n_q, n_k, d, dtype):
    H = 64 if n_q >= 512 else 128
    sl = alibi_slopes(H)
    heads = [(b, h) for b in range(2) for h in (0, 1, H // 2, H - 1)]
    o, lse, inp, scale = run_case(fa, 2, H, n_q, n_k, d, dtype, causal, window, seed=n_q + 5 * n_k,
                                  slopes=sl)
    # the steepest slopes (0.5 and up to 2^-8 / 64 apart) put most of a row's weight on a few keys
    compare(o, lse, inp, scale, causal, window, dtype,
            f"alibi main nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}", heads=heads,
            slopes=sl, edge=True)


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (True, (300, 0)), (False, (-1, 0)),
                                           (False, (-1, -1)), (False, (100, 40))])
@pytest.mark.parametrize("n_q,n_k", [(512, 512), (512, 1500), (300, 1000)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_alibi_backward_main_kernels(fa, causal, window, n_q, n_k, d, dtype):
    """Full-grid ALiBi backward: the tuned dK/dV and dQ kernels where no visible pair lies past
    the diagonal (causal, or a right window of 0), the four-wave ones otherwise."""
    H = 64 if n_q >= 512 else 128
    run_backward(fa, 2, H, n_q, n_k, d, dtype, causal, window, seed=3 * n_q + n_k,
                 slopes=alibi_slopes(H))


def test_alibi_main_kernel_scales_and_backward(fa):
    """Zero, negative and larger scales on the main kernel's ALiBi instance, and the backward
    (four-wave kernels) from its LSE."""
    H = 64
    sl = alibi_slopes(H)
    heads = [(0, 0), (1, 5), (1, H - 1)]
    for scale in (0.0, -0.125, 0.3):
        for causal in (False, True):
            o, lse, inp, sc = run_case(fa, 2, H, 512, 1024, 64, "f16", causal, (-1, -1), seed=71,
                                       scale=scale, slopes=sl)
            compare(o, lse, inp, sc, causal, (-1, -1), "f16",
                    f"alibi main scale={scale} causal={causal}", heads=heads, slopes=sl, edge=True)
    run_backward(fa, 2, H, 512, 512, 64, "bf16", True, (-1, -1), seed=72, slopes=sl)


def test_alibi_zero_slopes_match_no_alibi(fa):
    """All-zero slopes go through the ALiBi instances and must give the plain results, up to
    rounding: those instances scale the scores before taking the row maximum, so the
    reference of the exponent (and with it the rounding of P) may differ."""
    import torch
    inp = W.cross_case(1, 2, 200, 900, 64, "bf16", seed=61)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    zero = torch.zeros(2, dtype=torch.float32, device="cuda")
    a = fa.fwd_kv(q, k, v, None, True, alibi_slopes=zero)
    b = fa.fwd_kv(q, k, v, None, True)
    torch.cuda.synchronize()
    assert float((a[0].float() - b[0].float()).abs().max()) <= O_TOL["bf16"]
    assert float((a[1] - b[1]).abs().max()) <= 1e-5


# ---------------------------------------------------------------------------- dropout
def run_dropout(fa, B, H, n_q, n_k, d, dtype, causal, window, seed, p, rng_seed, offset,
                slopes=None, backward=False):
    """fa_fwd_kv (and fa_bwd_kv) with dropout against the oracle with the same Philox masks."""
    import oracle
    import torch
    p = float(np.float32(p))   # the value the C ABI receives
    inp = W.cross_case(B, H, n_q, n_k, d, dtype, seed)
    g = W.cross_case(B, H, n_q, 1, d, dtype, seed + 1000)
    q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], g["q"]))
    scale = 1.0 / math.sqrt(d)
    sl = None if slopes is None else torch.tensor(slopes, dtype=torch.float32, device="cuda")
    kw = dict(alibi_slopes=sl, dropout_p=p, dropout_seed=rng_seed, dropout_offset=offset)
    o, lse = fa.fwd_kv(q, k, v, scale, causal, window, **kw)
    grads = fa.bwd_kv(do, q, k, v, o, lse, scale, causal, window, **kw) if backward else None
    torch.cuda.synchronize()
    ro, rl = oracle.dropout_forward_bh(inp["q64"], inp["k64"], inp["v64"], scale, causal, window,
                                       p, rng_seed, offset, slopes)
    label = f"dropout p={p:.3f} nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}"
    o64, l64 = to64(o), lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(l64), empty)
    d_o = float(np.abs(o64 - ro).max())
    d_l = float(np.abs(l64[~empty] - rl[~empty]).max()) if (~empty).any() else 0.0
    say(f"{label}: max|dO|={d_o:.2e} max|dLSE|={d_l:.2e}")
    assert d_l <= LSE_TOL, label
    diff = np.abs(o64 - ro)
    over = diff > O_TOL[dtype]
    if over.any():
        # Rows that see few keys have |O| up to about 4 / r (r ~ 1 - p the keep probability),
        # where one bf16 step exceeds the fixed tolerance.  The kernel rounds each kept weight
        # P / r once to the input type and O once at the end, so
        # |dO| <= u (sum_j P_ij M_ij / r |V_jc| + |O_ic|)
        # (u the unit roundoff); elements over the fixed tolerance must be within that bound.
        wabs, _ = oracle.dropout_forward_bh(inp["q64"], inp["k64"], np.abs(inp["v64"]), scale,
                                            causal, window, p, rng_seed, offset, slopes)
        derived = UNIT_ROUNDOFF[dtype] * (wabs + np.abs(ro)) + 1e-5
        ratio = float((diff[over] / derived[over]).max())
        say(f"{label}: {int(over.sum())} element(s) over {O_TOL[dtype]} (max |O| "
            f"{float(np.abs(ro[over]).max()):.2f}), worst |dO| / rounding bound {ratio:.2f}")
        assert ratio <= 1.0, f"{label}: max|dO| {d_o:.3e} beyond the rounding bound"
    if backward:
        rq, rk, rv = oracle.dropout_backward_bh(inp["q64"], inp["k64"], inp["v64"], g["q64"],
                                                scale, causal, window, p, rng_seed, offset, slopes)
        floor = 1e-3 * float(np.linalg.norm(g["q64"]))
        for name, got, ref in zip(("dq", "dk", "dv"), grads, (rq, rk, rv)):
            e = rel_l2(to64(got), ref, floor)
            assert e <= GRAD_REL_L2, f"{label} {name} rel L2 {e:.3e}"
    return o


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (300, 0))])
@pytest.mark.parametrize("n_q,n_k", [(1, 300), (3, 129), (100, 700), (300, 129), (128, 8192),
                                     (257, 257)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_dropout_forward(fa, causal, window, n_q, n_k, d, dtype):
    run_dropout(fa, 1, 3, n_q, n_k, d, dtype, causal, window, seed=n_q + 7 * n_k, p=0.17,
                rng_seed=0x1234_5678_9ABC, offset=3)


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (100, 40))])
@pytest.mark.parametrize("n_q,n_k", [(1, 300), (100, 700), (300, 129), (257, 257)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_dropout_backward(fa, causal, window, n_q, n_k, d, dtype):
    run_dropout(fa, 1, 2, n_q, n_k, d, dtype, causal, window, seed=3 * n_q + n_k, p=0.3,
                rng_seed=987654321, offset=0, backward=True)


@pytest.mark.parametrize("p", [0.05, 0.5, 0.9])
def test_dropout_with_alibi(fa, p):
    run_dropout(fa, 2, 4, 200, 900, 64, "bf16", True, (-1, -1), seed=12, p=p, rng_seed=42,
                offset=11, slopes=alibi_slopes(4), backward=True)


def test_dropout_reproducible_and_offset_changes_mask(fa):
    import torch
    a = run_dropout(fa, 1, 2, 64, 512, 64, "bf16", False, (-1, -1), seed=5, p=0.25, rng_seed=7,
                    offset=0)
    b = run_dropout(fa, 1, 2, 64, 512, 64, "bf16", False, (-1, -1), seed=5, p=0.25, rng_seed=7,
                    offset=0)
    c = run_dropout(fa, 1, 2, 64, 512, 64, "bf16", False, (-1, -1), seed=5, p=0.25, rng_seed=7,
                    offset=1)
    assert torch.equal(a, b) and not torch.equal(a, c)


# ---------------------------------------------------------------------------- block-sparse
def random_blocks(H, n_q, n_k, seed, density=0.5):
    rng = np.random.default_rng(seed)
    return rng.random((H, -(-n_q // 64), -(-n_k // 64))) < density


def run_blocks(fa, B, H, n_q, n_k, d, dtype, causal, window, seed, blocks, backward=False,
               slopes=None, p=0.0):
    import oracle
    import torch
    inp = W.cross_case(B, H, n_q, n_k, d, dtype, seed)
    g = W.cross_case(B, H, n_q, 1, d, dtype, seed + 1000)
    q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], g["q"]))
    scale = 1.0 / math.sqrt(d)
    bm = torch.tensor(blocks.astype(np.uint8), device="cuda")
    sl = None if slopes is None else torch.tensor(slopes, dtype=torch.float32, device="cuda")
    kw = dict(block_mask=bm, alibi_slopes=sl)
    o, lse = fa.fwd_kv(q, k, v, scale, causal, window, **kw)
    grads = fa.bwd_kv(do, q, k, v, o, lse, scale, causal, window, **kw) if backward else None
    torch.cuda.synchronize()
    compare(o, lse, inp, scale, causal, window, dtype,
            f"blocks nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}", slopes=slopes,
            block_mask=blocks)
    if backward:
        rq, rk, rv = oracle.cross_backward_bh(inp["q64"], inp["k64"], inp["v64"], g["q64"], scale,
                                              causal, window, slopes, blocks)
        floor = 1e-3 * float(np.linalg.norm(g["q64"]))
        for name, got, ref in zip(("dq", "dk", "dv"), grads, (rq, rk, rv)):
            e = rel_l2(to64(got), ref, floor)
            assert e <= GRAD_REL_L2, f"blocks {name} rel L2 {e:.3e}"


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (100, 40))])
@pytest.mark.parametrize("n_q,n_k", [(1, 3000), (4, 20000), (64, 64), (100, 700), (300, 129),
                                     (128, 8192), (257, 1000)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_block_sparse_forward(fa, causal, window, n_q, n_k, d, dtype):
    run_blocks(fa, 1, 3, n_q, n_k, d, dtype, causal, window, seed=n_q + n_k,
               blocks=random_blocks(3, n_q, n_k, seed=7 * n_q + n_k))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n_q,n_k", [(64, 64), (100, 700), (300, 129), (257, 1000), (1, 500)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_block_sparse_backward(fa, causal, n_q, n_k, d, dtype):
    run_blocks(fa, 1, 2, n_q, n_k, d, dtype, causal, (-1, -1), seed=n_q * 3 + n_k,
               blocks=random_blocks(2, n_q, n_k, seed=n_q + 5 * n_k), backward=True)


def test_block_sparse_with_alibi_and_structure(fa):
    """Block-diagonal, empty and full masks, with ALiBi slopes."""
    H, n = 3, 320
    nb = -(-n // 64)
    blocks = np.stack([np.eye(nb, dtype=bool), np.zeros((nb, nb), bool), np.ones((nb, nb), bool)])
    run_blocks(fa, 2, H, n, n, 64, "bf16", False, (-1, -1), seed=3, blocks=blocks, backward=True,
               slopes=alibi_slopes(H))


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (300, 0)),
                                           (False, (100, 40))])
@pytest.mark.parametrize("n_q,n_k", [(256, 320), (256, 1000), (512, 512), (130, 4096), (300, 2065)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_block_sparse_main_kernel(fa, causal, window, n_q, n_k, d, dtype):
    """128 heads: query tiles enough for the main forward kernel and the main dK/dV and dQ
    kernels, which visit only the steps a workgroup's blocks select.  Head 0 selects nothing
    (O = 0, LSE = -inf, zero gradients), head 1 everything, head 2 the block diagonal, head 3
    one key block per query block, the rest random at densities 0.5 and 0.2; sampled heads
    against the oracle (gradients by relative L2)."""
    import oracle
    import torch
    B, H = 8, 16
    nqb, nkb = -(-n_q // 64), -(-n_k // 64)
    blocks = np.concatenate([random_blocks(6, n_q, n_k, seed=n_q + 3 * n_k),
                             random_blocks(6, n_q, n_k, seed=n_q + 5 * n_k, density=0.2)])
    fixed = np.zeros((4, nqb, nkb), bool)
    fixed[1] = True
    fixed[2] = np.eye(nqb, nkb, dtype=bool)
    fixed[3][np.arange(nqb), (7 * np.arange(nqb)) % nkb] = True
    blocks = np.concatenate([fixed, blocks])
    inp = W.cross_case(B, H, n_q, n_k, d, dtype, seed=n_q * 7 + n_k)
    g = W.cross_case(B, H, n_q, 1, d, dtype, seed=n_q * 7 + n_k + 1000)
    q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], g["q"]))
    scale = 1.0 / math.sqrt(d)
    bm = torch.tensor(blocks.astype(np.uint8), device="cuda")
    o, lse = fa.fwd_kv(q, k, v, scale, causal, window, block_mask=bm)
    dq, dk, dv = fa.bwd_kv(do, q, k, v, o, lse, scale, causal, window, block_mask=bm)
    torch.cuda.synchronize()
    label = f"main blocks nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}"
    heads = [(b, (3 * b + 1) % H) for b in range(B)] + [(0, 0), (1, 1), (2, 2), (3, 3), (B - 1, H - 1)]
    compare(o, lse, inp, scale, causal, window, dtype, label, heads=heads, block_mask=blocks)
    assert torch.all(torch.isneginf(lse[:, 0])) and torch.all(o[:, 0] == 0)
    assert all(torch.all(t[:, 0] == 0) for t in (dq, dk, dv)), f"{label}: head 0 gradients"
    got = [to64(t) for t in (dq, dk, dv)]
    for b, h in heads:
        ref = oracle.cross_backward(inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h],
                                    g["q64"][b, h], scale, causal, window, block_mask=blocks[h])
        floor = 1e-3 * float(np.linalg.norm(g["q64"][b, h]))
        for name, gt, rf in zip(("dq", "dk", "dv"), got, ref):
            e = rel_l2(gt[b, h], rf, floor)
            assert e <= GRAD_REL_L2, f"{label} {name} b={b} h={h}: rel L2 {e:.3e}"


def test_block_sparse_main_kernel_block_workload(fa):
    """The block training workload at full size with a density-0.5 block mask (the bench's
    --block-density 0.5 step, all three main kernels); sampled heads against the oracle."""
    import oracle
    import torch
    w = W.BLOCK
    blocks = W.draw_blocks(w.H, w.n_q, w.n_k, 0.5, w.seed)
    inp = W.cross_case(w.B, w.H, w.n_q, w.n_k, w.d, w.dtype, w.seed)
    g = W.cross_case(w.B, w.H, w.n_q, 1, w.d, w.dtype, w.seed + 1000)
    q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], g["q"]))
    bm = torch.tensor(blocks.astype(np.uint8), device="cuda")
    o, lse = fa.fwd_kv(q, k, v, w.softmax_scale, True, block_mask=bm)
    dq, dk, dv = fa.bwd_kv(do, q, k, v, o, lse, w.softmax_scale, True, block_mask=bm)
    torch.cuda.synchronize()
    heads = [(0, 0), (3, 7), (w.B - 1, w.H - 1)]
    compare(o, lse, inp, w.softmax_scale, True, (-1, -1), w.dtype, w.name + " blocks 0.5",
            heads=heads, block_mask=blocks)
    got = [to64(t) for t in (dq, dk, dv)]
    for b, h in heads:
        ref = oracle.cross_backward(inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h],
                                    g["q64"][b, h], w.softmax_scale, True, block_mask=blocks[h])
        floor = 1e-3 * float(np.linalg.norm(g["q64"][b, h]))
        for name, gt, rf in zip(("dq", "dk", "dv"), got, ref):
            e = rel_l2(gt[b, h], rf, floor)
            assert e <= GRAD_REL_L2, f"{w.name} blocks {name} b={b} h={h}: rel L2 {e:.3e}"


def test_plain_self_attention_takes_the_fa_fwd_kernels(fa):
    """Equal lengths, dense operands and nothing extra: fa_fwd_kv / fa_bwd_kv give bit for bit
    what fa_fwd / fa_bwd give (they run the same kernels)."""
    import torch
    inp = W.cross_case(2, 8, 1024, 1024, 64, "bf16", seed=71)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    do = torch.ones_like(q)
    o1, l1 = fa.fwd_kv(q, k, v, None, True)
    o2, l2 = fa.fwd(q, k, v, None, True)
    g1 = fa.bwd_kv(do, q, k, v, o1, l1, None, True)
    g2 = fa.bwd(do, q, k, v, o2, l2, None, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


# ---------------------------------------------------------------------------- main kernel, N_q != N_k
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (300, 0)),
                                           (False, (100, 40)), (True, (256, 0))])
@pytest.mark.parametrize("n_q,n_k", [(256, 320), (256, 1000), (256, 2065), (512, 300), (130, 4096)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_main_kernel_queries_over_more_keys(fa, causal, window, n_q, n_k, d, dtype):
    """128 heads: enough query tiles for the main forward kernel (key offsets that are and are
    not multiples of 32; rows without keys when N_q > N_k)."""
    B, H = 8, 16
    o, lse, inp, scale = run_case(fa, B, H, n_q, n_k, d, dtype, causal, window, seed=n_q + n_k)
    heads = [(b, (3 * b + 5) % H) for b in range(B)] + [(B - 1, H - 1), (0, 0)]
    compare(o, lse, inp, scale, causal, window, dtype,
            f"main nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}", heads=heads)
    if n_q > n_k and causal:
        assert bool(torch_isneginf_rows(lse, n_q - n_k))


def torch_isneginf_rows(lse, rows):
    import torch
    return torch.all(torch.isneginf(lse[:, :, :rows])) and torch.all(torch.isfinite(lse[:, :, rows:]))



def test_autograd_kv_wrapper(fa):
    """fa.attention_kv through torch.autograd gives bit for bit what fa_fwd_kv / fa_bwd_kv give
    with the same arguments (ALiBi, dropout and a block mask together); those calls are checked
    against the oracle above."""
    import torch
    B, H, n_q, n_k, d = 1, 2, 150, 400, 64
    inp = W.cross_case(B, H, n_q, n_k, d, "bf16", seed=81)
    g = to_dev(W.cross_case(B, H, n_q, 1, d, "bf16", seed=82)["q"])
    q, k, v = (to_dev(inp[n]).requires_grad_() for n in ("q", "k", "v"))
    extra = dict(alibi_slopes=torch.tensor([0.25, 0.0625], device="cuda"), dropout_p=0.2,
                 dropout_seed=5, dropout_offset=1,
                 block_mask=torch.tensor(random_blocks(H, n_q, n_k, seed=83, density=0.7)
                                         .astype(np.uint8), device="cuda"))
    o = fa.attention_kv(q, k, v, 0.125, True, **extra)
    o.backward(g)
    o_ref, lse = fa.fwd_kv(q.detach(), k.detach(), v.detach(), 0.125, True, **extra)
    grads = fa.bwd_kv(g, q.detach(), k.detach(), v.detach(), o_ref, lse, 0.125, True, **extra)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    assert all(torch.equal(a, b) for a, b in zip((q.grad, k.grad, v.grad), grads))


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (300, 0)),
                                           (False, (100, 40))])
@pytest.mark.parametrize("n_q,n_k", [(256, 320), (256, 1000), (512, 300), (130, 2065)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_main_kernels_backward_queries_over_more_keys(fa, causal, window, n_q, n_k, d, dtype):
    """128 heads: fa_bwd_kv takes the dK/dV and dQ kernels of fa_bwd (band shifted by the key
    offset); gradients of sampled heads against the oracle by relative L2."""
    import oracle
    import torch
    B, H = 8, 16
    inp = W.cross_case(B, H, n_q, n_k, d, dtype, seed=n_q * 3 + n_k)
    g = W.cross_case(B, H, n_q, 1, d, dtype, seed=n_q * 3 + n_k + 1000)
    q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], g["q"]))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd_kv(q, k, v, scale, causal, window)
    dq, dk, dv = fa.bwd_kv(do, q, k, v, o, lse, scale, causal, window)
    torch.cuda.synchronize()
    heads = [(b, (5 * b + 2) % H) for b in range(B)] + [(0, 0), (B - 1, H - 1)]
    got = [to64(t) for t in (dq, dk, dv)]
    for b, h in heads:
        ref = oracle.cross_backward(inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h],
                                    g["q64"][b, h], scale, causal, window)
        floor = 1e-3 * float(np.linalg.norm(g["q64"][b, h]))
        for name, gt, rf in zip(("dq", "dk", "dv"), got, ref):
            e = rel_l2(gt[b, h], rf, floor)
            assert e <= GRAD_REL_L2, f"{name} b={b} h={h} nq={n_q} nk={n_k}: rel L2 {e:.3e}"
    if causal and n_q > n_k:   # rows without keys: zero dQ
        assert torch.all(dq[:, :, : n_q - n_k] == 0)


def test_block_workload_sampled(fa):
    """The bench's block training workload at full size, in the configuration the bench times
    (fa_fwd_kv, then fa_bwd_kv on the tuned kernels); sampled heads against the oracle."""
    import oracle
    import torch
    w = W.BLOCK
    inp = W.cross_case(w.B, w.H, w.n_q, w.n_k, w.d, w.dtype, w.seed)
    g = W.cross_case(w.B, w.H, w.n_q, 1, w.d, w.dtype, w.seed + 1000)
    q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], g["q"]))
    o, lse = fa.fwd_kv(q, k, v, w.softmax_scale, True)
    dq, dk, dv = fa.bwd_kv(do, q, k, v, o, lse, w.softmax_scale, True)
    torch.cuda.synchronize()
    heads = [(0, 0), (3, 7), (w.B - 1, w.H - 1)]
    compare(o, lse, inp, w.softmax_scale, True, (-1, -1), w.dtype, w.name, heads=heads)
    got = [to64(t) for t in (dq, dk, dv)]
    for b, h in heads:
        ref = oracle.cross_backward(inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h],
                                    g["q64"][b, h], w.softmax_scale, True)
        floor = 1e-3 * float(np.linalg.norm(g["q64"][b, h]))
        for name, gt, rf in zip(("dq", "dk", "dv"), got, ref):
            e = rel_l2(gt[b, h], rf, floor)
            assert e <= GRAD_REL_L2, f"{w.name} {name} b={b} h={h}: rel L2 {e:.3e}"
