"""Key padding masks on the GPU: fa_fwd_kv / fa_bwd_kv / fa_fwd_kv_fp8 with a [B, N_k] mask of
padding keys, through the C ABI, against the float64 oracle (``cross_forward`` and friends with
``key_mask``), with the fixed tolerances (max |dO| 2e-3 fp16 / 1e-2 bf16, |dLSE| 1e-3, gradients
2e-2 relative L2).

Masks hold random holes (each key padded with probability 0.3) plus whole padded ranges: whole
64-key tiles (skipped by the kernels), a padded tail, and a batch entry whose keys are all
padding (every row without a key: O = 0, LSE = -inf, dQ = 0).  The few-query kernel (with and
without key splits), the MFMA kernel (with and without splits), both backward kernels, and the
combinations with ALiBi, block masks, dropout and an FP8 cache are covered."""
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


def mask_for(B, n_k, seed):
    """Holes, two padded 64-key tiles and a padded tail in entry 0; entry B - 1 (when B > 1)
    has every key padded."""
    runs = [(0, 64, 192), (0, n_k - n_k // 5, n_k)]
    if B > 1:
        runs.append((B - 1, 0, n_k))
    return W.key_padding_case(B, n_k, seed, 0.3, runs)


def check_forward(o, lse, ro, rl, dtype, label):
    o64, l64 = to64(o), lse.detach().cpu().numpy().astype(np.float64)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(l64), empty), f"{label}: rows without keys differ"
    assert np.all(o64[empty] == 0.0), f"{label}: O of a row without keys is not 0"
    d_o = float(np.abs(o64 - ro).max()) if ro.size else 0.0
    d_l = float(np.abs(l64[~empty] - rl[~empty]).max()) if (~empty).any() else 0.0
    say(f"{label}: rows without keys {int(empty.sum())}, max|dO|={d_o:.2e} max|dLSE|={d_l:.2e}")
    assert d_o <= O_TOL[dtype], f"{label}: max|dO| {d_o:.3e} > {O_TOL[dtype]}"
    assert d_l <= LSE_TOL, f"{label}: max|dLSE| {d_l:.3e} > {LSE_TOL}"


def run(fa, B, H, n_q, n_k, d, dtype, causal, window, seed, backward=False, slopes=None,
        blocks=None, km=None):
    import oracle
    import torch
    inp = W.cross_case(B, H, n_q, n_k, d, dtype, seed)
    g = W.cross_case(B, H, n_q, 1, d, dtype, seed + 1000)
    q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], g["q"]))
    km = mask_for(B, n_k, seed + 7) if km is None else km
    scale = 1.0 / math.sqrt(d)
    kw = dict(key_padding_mask=torch.tensor(km.astype(np.uint8), device="cuda"),
              alibi_slopes=None if slopes is None else torch.tensor(slopes, dtype=torch.float32,
                                                                    device="cuda"),
              block_mask=None if blocks is None else torch.tensor(blocks.astype(np.uint8),
                                                                  device="cuda"))
    o, lse = fa.fwd_kv(q, k, v, scale, causal, window, **kw)
    grads = fa.bwd_kv(do, q, k, v, o, lse, scale, causal, window, **kw) if backward else None
    torch.cuda.synchronize()
    label = (f"kpm nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}"
             f"{' alibi' if slopes else ''}{' blocks' if blocks is not None else ''}")
    ro, rl = oracle.cross_forward_bh(inp["q64"], inp["k64"], inp["v64"], scale, causal, window,
                                     slopes, blocks, km)
    check_forward(o, lse, ro, rl, dtype, label)
    if backward:
        rq, rk, rv = oracle.cross_backward_bh(inp["q64"], inp["k64"], inp["v64"], g["q64"], scale,
                                              causal, window, slopes, blocks, km)
        floor = 1e-3 * float(np.linalg.norm(g["q64"]))
        errs = [rel_l2(to64(t), r, floor) for t, r in zip(grads, (rq, rk, rv))]
        say(f"{label}: rel L2 dq={errs[0]:.2e} dk={errs[1]:.2e} dv={errs[2]:.2e}")
        for name, e in zip(("dq", "dk", "dv"), errs):
            assert e <= GRAD_REL_L2, f"{label}: {name} rel L2 {e:.3e} > {GRAD_REL_L2}"
        dk, dv = (to64(t) for t in grads[1:])
        for b in range(B):   # padding keys get exactly zero gradients
            assert np.all(dk[b][:, km[b]] == 0.0) and np.all(dv[b][:, km[b]] == 0.0), label
        empty = np.isneginf(rl)
        assert np.all(to64(grads[0])[empty] == 0.0), f"{label}: dQ of a row without keys"
    return o, lse


MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (100, 40)), (True, (300, 0))]


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("n_q", [1, 2, 4])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_few_queries(fa, causal, window, n_q, d, dtype):
    for n_k, seed in ((77, 1), (1000, 2), (4099, 3), (20000, 4)):
        run(fa, 2, 3, n_q, n_k, d, dtype, causal, window, seed)


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("n_q,n_k", [(5, 300), (100, 700), (300, 129), (128, 8192), (257, 257)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_many_queries(fa, causal, window, n_q, n_k, d, dtype):
    run(fa, 2, 2, n_q, n_k, d, dtype, causal, window, seed=n_q + 3 * n_k)


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (100, 40))])
@pytest.mark.parametrize("n_q,n_k", [(1, 300), (100, 700), (300, 129), (257, 257), (130, 3000)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_backward(fa, causal, window, n_q, n_k, d, dtype):
    run(fa, 2, 2, n_q, n_k, d, dtype, causal, window, seed=5 * n_q + n_k, backward=True)


def test_with_alibi_and_blocks(fa):
    H, n_q, n_k = 3, 200, 900
    blocks = np.random.default_rng(5).random((H, -(-n_q // 64), -(-n_k // 64))) < 0.6
    slopes = [0.5, 2.0 ** -4, 2.0 ** -8]
    for causal in (False, True):
        run(fa, 2, H, n_q, n_k, 64, "bf16", causal, (-1, -1), seed=11, backward=True,
            slopes=slopes, blocks=blocks)
        run(fa, 2, H, 3, n_k, 128, "f16", causal, (-1, -1), seed=12, slopes=slopes,
            blocks=blocks[:, :1])


def test_no_padding_mask_is_no_mask(fa):
    """An all-zero mask gives what no mask gives on the same kernel (a decode step and a
    strided N_q != N_k call, both of which take the kernels that read the mask)."""
    import torch
    for n_q, n_k in ((1, 3000), (100, 700)):
        inp = W.cross_case(2, 2, n_q, n_k, 64, "bf16", 31)
        q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
        zero = torch.zeros(2, n_k, dtype=torch.uint8, device="cuda")
        a = fa.fwd_kv(q, k, v, None, True, key_padding_mask=zero)
        sl = torch.zeros(2, dtype=torch.float32, device="cuda")   # keeps the same kernel
        b = fa.fwd_kv(q, k, v, None, True, alibi_slopes=sl)
        torch.cuda.synchronize()
        assert float((a[0].float() - b[0].float()).abs().max()) <= O_TOL["bf16"]
        assert float((a[1] - b[1]).abs().max()) <= 1e-5


def test_bool_mask_and_autograd(fa):
    """A torch.bool mask through the autograd wrapper: the same outputs and gradients as the
    uint8 mask through fwd_kv / bwd_kv."""
    import torch
    inp = W.cross_case(2, 2, 100, 500, 64, "bf16", 41)
    km = mask_for(2, 500, 42)
    q, k, v = (to_dev(inp[n]).requires_grad_() for n in ("q", "k", "v"))
    mb = torch.tensor(km, device="cuda")
    out = fa.attention_kv(q, k, v, None, True, key_padding_mask=mb)
    do = torch.ones_like(out)
    out.backward(do)
    mu = torch.tensor(km.astype(np.uint8), device="cuda")
    o, lse = fa.fwd_kv(q.detach(), k.detach(), v.detach(), None, True, key_padding_mask=mu)
    g = fa.bwd_kv(do, q.detach(), k.detach(), v.detach(), o, lse, None, True, key_padding_mask=mu)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o)
    for a, b in zip((q.grad, k.grad, v.grad), g):
        assert torch.equal(a, b)


@pytest.mark.parametrize("n_q,n_k", [(1, 300), (100, 700)])
def test_with_dropout(fa, n_q, n_k):
    import oracle
    import torch
    B, H, d, p, seed, off = 2, 2, 64, float(np.float32(0.17)), 0x1234_5678, 5
    inp = W.cross_case(B, H, n_q, n_k, d, "bf16", 51)
    g = W.cross_case(B, H, n_q, 1, d, "bf16", 52)
    q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], g["q"]))
    km = mask_for(B, n_k, 53)
    kw = dict(key_padding_mask=torch.tensor(km.astype(np.uint8), device="cuda"), dropout_p=p,
              dropout_seed=seed, dropout_offset=off)
    scale = d ** -0.5
    o, lse = fa.fwd_kv(q, k, v, scale, False, (-1, -1), **kw)
    grads = fa.bwd_kv(do, q, k, v, o, lse, scale, False, (-1, -1), **kw)
    torch.cuda.synchronize()
    ro, rl = oracle.dropout_forward_bh(inp["q64"], inp["k64"], inp["v64"], scale, False, (-1, -1),
                                       p, seed, off, key_padding_mask=km)
    label = f"kpm + dropout nq={n_q} nk={n_k}"
    o64, l64 = to64(o), lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(l64), empty) and np.all(o64[empty] == 0.0), label
    assert float(np.abs(l64[~empty] - rl[~empty]).max()) <= LSE_TOL, label
    # each kept weight P / r is rounded once to bf16 and O once at the end
    wabs, _ = oracle.dropout_forward_bh(inp["q64"], inp["k64"], np.abs(inp["v64"]), scale, False,
                                        (-1, -1), p, seed, off, key_padding_mask=km)
    bound = np.maximum(O_TOL["bf16"], UNIT_ROUNDOFF["bf16"] * (wabs + np.abs(ro)) + 1e-5)
    ratio = float((np.abs(o64 - ro) / bound).max())
    say(f"{label}: worst |dO| / max(tolerance, rounding bound) {ratio:.2f}")
    assert ratio <= 1.0, label
    rq, rk, rv = oracle.dropout_backward_bh(inp["q64"], inp["k64"], inp["v64"], g["q64"], scale,
                                            False, (-1, -1), p, seed, off, key_padding_mask=km)
    floor = 1e-3 * float(np.linalg.norm(g["q64"]))
    for name, got, ref in zip(("dq", "dk", "dv"), grads, (rq, rk, rv)):
        e = rel_l2(to64(got), ref, floor)
        assert e <= GRAD_REL_L2, f"{label} {name} rel L2 {e:.3e}"


@pytest.mark.parametrize("n_q", [1, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_cache(fa, n_q, d):
    import oracle
    import torch
    for n_k, seed in ((300, 61), (20000, 62)):
        c = W.fp8_cache_case(2, 2, n_q, n_k, d, "bf16", seed)
        q = to_dev(c["q"])
        k, v = (torch.from_numpy(c[n]).to("cuda") for n in ("k8", "v8"))
        km = mask_for(2, n_k, seed + 1)
        o, lse = fa.fwd_kv_fp8(q, k, v, c["k_descale"], c["v_descale"], d ** -0.5, causal=True,
                               key_padding_mask=torch.tensor(km, device="cuda"))
        torch.cuda.synchronize()
        ro, rl = oracle.fp8_cache_forward_bh(c["q64"], c["k8"], c["v8"], d ** -0.5, c["k_descale"],
                                             c["v_descale"], True, key_padding_mask=km)
        check_forward(o, lse, ro, rl, "bf16", f"kpm fp8 cache nq={n_q} nk={n_k} d={d}")


def test_argument_errors(fa):
    import torch
    q = torch.zeros(2, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(2, 2, 40, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd_kv(q, k, k, key_padding_mask=torch.zeros(2, 39, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd_kv(q, k, k, key_padding_mask=torch.zeros(2, 40, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd_kv(q, k, k, key_padding_mask=torch.zeros(2, 40, dtype=torch.uint8))


def main_mask(B, n_k, seed):
    """Per batch entry: 0 holes, two padded 64-key tiles and a padded tail; 1 a padded head of
    the keys; 2 a padded tail only; 3 no padding; 4 one padding key; B - 1 every key padded;
    the rest holes of density 0.3."""
    rng = np.random.default_rng(seed)
    m = rng.random((B, n_k)) < 0.3
    m[0, 64:192] = True
    m[0, n_k - n_k // 5:] = True
    m[1] = False
    m[1, :min(n_k, 300)] = True
    m[2] = False
    m[2, n_k - n_k // 3:] = True
    m[3] = False
    m[4] = False
    m[4, n_k // 2] = True
    m[B - 1] = True
    return m


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (100, 40))])
@pytest.mark.parametrize("n_q,n_k", [(256, 320), (256, 1000), (512, 512), (130, 4096), (300, 2065)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_key_padding_main_kernels(fa, causal, window, n_q, n_k, d, dtype):
    """128 heads: query tiles enough for the main forward, dK/dV and dQ kernels; every entry of
    the batch a different padding pattern (main_mask); sampled heads of every entry against the
    oracle, forward and backward."""
    import oracle
    import torch
    B, H = 8, 16
    inp = W.cross_case(B, H, n_q, n_k, d, dtype, seed=n_q * 11 + n_k)
    g = W.cross_case(B, H, n_q, 1, d, dtype, seed=n_q * 11 + n_k + 1000)
    q, k, v, do = (to_dev(t) for t in (inp["q"], inp["k"], inp["v"], g["q"]))
    km = main_mask(B, n_k, seed=n_q + n_k)
    scale = 1.0 / math.sqrt(d)
    kpm = torch.tensor(km.astype(np.uint8), device="cuda")
    o, lse = fa.fwd_kv(q, k, v, scale, causal, window, key_padding_mask=kpm)
    dq, dk, dv = fa.bwd_kv(do, q, k, v, o, lse, scale, causal, window, key_padding_mask=kpm)
    torch.cuda.synchronize()
    label = f"kpm main nq={n_q} nk={n_k} d={d} {dtype} causal={causal} w={window}"
    got = [to64(t) for t in (dq, dk, dv)]
    for b in range(B):
        h = (5 * b + 3) % H
        ro, rl = oracle.cross_forward(inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h], scale,
                                      causal, window, key_mask=km[b])
        check_forward(o[b, h], lse[b, h], ro, rl, dtype, f"{label} b={b} h={h}")
        ref = oracle.cross_backward(inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h],
                                    g["q64"][b, h], scale, causal, window, key_mask=km[b])
        floor = 1e-3 * float(np.linalg.norm(g["q64"][b, h]))
        for name, gt, rf in zip(("dq", "dk", "dv"), got, ref):
            e = rel_l2(gt[b, h], rf, floor)
            assert e <= GRAD_REL_L2, f"{label} {name} b={b} h={h}: rel L2 {e:.3e}"
    # padding keys get zero gradients, an entry with every key padded zero dQ, O = 0, LSE = -inf
    pad = torch.tensor(km, device="cuda")
    assert torch.all(dk.permute(0, 2, 1, 3)[pad] == 0) and torch.all(dv.permute(0, 2, 1, 3)[pad] == 0)
    assert torch.all(dq[B - 1] == 0) and torch.all(o[B - 1] == 0)
    assert torch.all(torch.isneginf(lse[B - 1]))
