"""The N_q != N_k oracle against its pins (CPU only).

  * suffix property: the queries are the last N_q positions, so attention of Q's last N_q
    rows over all N_k keys is the square definition's last N_q rows (every mask mode);
  * torch CPU float64 scaled_dot_product_attention with a boolean mask that torch itself
    builds (``tril`` with diagonal N_k - N_q, i.e. aligned at the bottom-right);
  * scalar brute force (pure-Python floats, unshifted softmax) with the position rule
    written out per pair;
  * closed forms: a decode step (N_q = 1, causal) sees every key; Q = 0 gives the mean of V
    over the visible keys and LSE = ln(count); rows with no visible key give O = 0,
    LSE = -inf.
The backward: central differences of the forward, the square backward for N_q = N_k and
(for the last N_q rows, dO zero elsewhere) for N_q < N_k, torch CPU float64 autograd through
SDPA with the bottom-right mask, and the invariants sum_j dV_j = sum_i dO_i over rows that see
a key and sum_j dK_j = 0.
"""
import math

import numpy as np
import pytest
import torch

import oracle

MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 2)), (True, (4, -1)), (False, (-1, 0)),
         (False, (2, -1))]
SHAPES = [(1, 9), (3, 9), (9, 9), (5, 12), (12, 5), (1, 1), (7, 3)]


def _qkv(n_q, n_k, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n_q, d)), rng.standard_normal((n_k, d)), rng.standard_normal((n_k, d))


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("n_q", [1, 4, 11])
def test_last_rows_of_square_definition(causal, window, n_q):
    n_k = 11
    rng = np.random.default_rng(3)
    q_all = rng.standard_normal((n_k, 6))
    k = rng.standard_normal((n_k, 6))
    v = rng.standard_normal((n_k, 6))
    o, lse = oracle.cross_forward(q_all[n_k - n_q:], k, v, 0.45, causal, window)
    ro, rl = oracle.attention_forward(q_all, k, v, 0.45, causal, window)
    np.testing.assert_allclose(o, ro[n_k - n_q:], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, rl[n_k - n_q:], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("n_q,n_k", [(1, 9), (3, 9), (5, 12), (9, 9)])
def test_torch_sdpa_bottom_right_causal(n_q, n_k):
    q, k, v = _qkv(n_q, n_k, 5, seed=n_q * 31 + n_k)
    mask = torch.ones(n_q, n_k, dtype=torch.bool).tril(diagonal=n_k - n_q)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=mask[None], scale=0.6)[0].numpy()
    o, _ = oracle.cross_forward(q, k, v, 0.6, causal=True)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def _brute(q, k, v, scale, causal, window):
    n_q, n_k = len(q), len(k)
    left, right = window
    out, lse = [], []
    for i in range(n_q):
        pos = i + n_k - n_q
        js = [j for j in range(n_k)
              if not (causal and j > pos) and not (left >= 0 and j < pos - left)
              and not (right >= 0 and j > pos + right)]
        if not js:
            out.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        e = {j: math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j])))
             for j in js}
        z = math.fsum(e.values())
        out.append([math.fsum(e[j] / z * float(v[j][c]) for j in js) for c in range(len(v[0]))])
        lse.append(math.log(z))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("n_q,n_k", SHAPES)
def test_brute_force(causal, window, n_q, n_k):
    q, k, v = _qkv(n_q, n_k, 4, seed=7 * n_q + n_k)
    o, lse = oracle.cross_forward(q, k, v, 0.5, causal, window)
    bo, bl = _brute(q, k, v, 0.5, causal, window)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-12)


def test_decode_step_sees_every_key():
    q, k, v = _qkv(1, 37, 8, seed=5)
    o, lse = oracle.cross_forward(q, k, v, 0.3, causal=True)
    s = [0.3 * float(np.dot(q[0], k[j])) for j in range(37)]
    z = math.fsum(math.exp(x) for x in s)
    ref = [math.fsum(math.exp(s[j]) / z * v[j, c] for j in range(37)) for c in range(8)]
    np.testing.assert_allclose(o[0], ref, rtol=1e-12, atol=1e-12)
    assert abs(lse[0] - math.log(z)) < 1e-12


@pytest.mark.parametrize("causal,window", MASKS)
def test_zero_query_is_mean_over_visible_keys(causal, window):
    _, k, v = _qkv(1, 10, 3, seed=9)
    q = np.zeros((4, 3))
    o, lse = oracle.cross_forward(q, k, v, 1.0, causal, window)
    for i in range(4):
        pos = i + 6
        js = [j for j in range(10) if not (causal and j > pos)
              and not (window[0] >= 0 and j < pos - window[0])
              and not (window[1] >= 0 and j > pos + window[1])]
        np.testing.assert_allclose(o[i], v[js].mean(axis=0), rtol=1e-13, atol=1e-13)
        assert abs(lse[i] - math.log(len(js))) < 1e-13


def test_rows_without_keys():
    q, k, v = _qkv(7, 3, 4, seed=11)
    o, lse = oracle.cross_forward(q, k, v, 0.5, causal=True)
    # positions -4 .. 2: the first four rows see no key
    assert np.all(o[:4] == 0.0) and np.all(np.isneginf(lse[:4]))
    assert np.all(np.isfinite(lse[4:]))
    o2, lse2 = oracle.cross_forward(q, k, v, 0.5, causal=False, window=(-1, 0))
    # a right bound of 0 is the same mask as causal
    np.testing.assert_array_equal(o2, o)
    o3, lse3 = oracle.cross_forward(q, k, v, 0.5, causal=False, window=(-1, 1))
    # positions -4 .. -2 with right bound 1 see no key
    assert np.all(o3[:3] == 0.0) and np.all(np.isneginf(lse3[:3])) and np.isfinite(lse3[3])


def test_pair_count():
    assert oracle.cross_allowed_pairs(1, 4096, True) == 4096
    assert oracle.cross_allowed_pairs(4096, 4096, True) == 4096 * 4097 // 2
    assert oracle.cross_allowed_pairs(16, 100, True) == sum(85 + i for i in range(16))
    assert oracle.cross_allowed_pairs(1, 100, True, (9, 0)) == 10


def test_mutant_top_left_alignment_fails_the_suffix_pin():
    """A top-left causal alignment (query i sees keys j <= i) is a plausible mistake; the
    suffix property rejects it."""
    rng = np.random.default_rng(4)
    q_all, k, v = (rng.standard_normal((8, 4)) for _ in range(3))
    ok = np.tril(np.ones((3, 8), dtype=bool))
    s = np.where(ok, 0.5 * q_all[5:] @ k.T, -np.inf)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    wrong = (e / e.sum(axis=1, keepdims=True)) @ v
    ro, _ = oracle.attention_forward(q_all, k, v, 0.5, causal=True)
    assert not np.allclose(wrong, ro[5:], atol=1e-6)


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("n_q,n_k", [(1, 6), (3, 7), (6, 6), (7, 3), (5, 9)])
def test_backward_central_differences(causal, window, n_q, n_k):
    rng = np.random.default_rng(n_q * 13 + n_k)
    q, k, v, do = (rng.standard_normal((r, 3)) for r in (n_q, n_k, n_k, n_q))
    dq, dk, dv = oracle.cross_backward(q, k, v, do, 0.7, causal, window)
    h = 1e-6

    def loss(q_, k_, v_):
        o, _ = oracle.cross_forward(q_, k_, v_, 0.7, causal, window)
        return float((o * do).sum())

    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = plus, minus
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("causal,window", MASKS)
def test_backward_reduces_to_square_and_suffix(causal, window):
    rng = np.random.default_rng(17)
    n = 10
    q, k, v, do = (rng.standard_normal((n, 4)) for _ in range(4))
    ref = oracle.attention_backward(q, k, v, do, 0.5, causal, window)
    got = oracle.cross_backward(q, k, v, do, 0.5, causal, window)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    n_q = 4   # the last rows only: dO zero on the first n - n_q rows of the square problem
    do_sq = do.copy()
    do_sq[: n - n_q] = 0.0
    rq, rk, rv = oracle.attention_backward(q, k, v, do_sq, 0.5, causal, window)
    gq, gk, gv = oracle.cross_backward(q[n - n_q:], k, v, do[n - n_q:], 0.5, causal, window)
    np.testing.assert_allclose(gq, rq[n - n_q:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gk, rk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gv, rv, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("n_q,n_k", [(3, 8), (8, 5), (1, 6)])
def test_backward_torch_autograd(n_q, n_k):
    rng = np.random.default_rng(n_q + 5 * n_k)
    q, k, v, do = (rng.standard_normal((r, 4)) for r in (n_q, n_k, n_k, n_q))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    mask = torch.ones(n_q, n_k, dtype=torch.bool).tril(diagonal=n_k - n_q)
    live = mask.any(dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], attn_mask=mask[None], scale=0.6)[0]
    # rows without a key come out NaN from SDPA; they take no part in the loss
    (torch.where(live[:, None], o, 0.0) * torch.tensor(do)).sum().backward()
    gq, gk, gv = oracle.cross_backward(q, k, v, do, 0.6, causal=True)
    np.testing.assert_allclose(gq[live.numpy()], tq.grad.numpy()[live.numpy()], rtol=1e-10,
                               atol=1e-12)
    np.testing.assert_allclose(gk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(gv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.all(gq[~live.numpy()] == 0.0)


def test_backward_invariants():
    rng = np.random.default_rng(23)
    q, do = rng.standard_normal((9, 5)), rng.standard_normal((9, 5))
    k, v = rng.standard_normal((4, 5)), rng.standard_normal((4, 5))
    dq, dk, dv = oracle.cross_backward(q, k, v, do, 0.8, causal=True)
    live = np.isfinite(oracle.cross_forward(q, k, v, 0.8, causal=True)[1])
    np.testing.assert_allclose(dv.sum(axis=0), do[live].sum(axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    assert np.all(dq[~live] == 0.0)


# ---------------------------------------------------------------------------- ALiBi
def _brute_alibi(q, k, v, scale, slope, causal, window):
    n_q, n_k = len(q), len(k)
    left, right = window
    out, lse = [], []
    for i in range(n_q):
        pos = i + n_k - n_q
        js = [j for j in range(n_k)
              if not (causal and j > pos) and not (left >= 0 and j < pos - left)
              and not (right >= 0 and j > pos + right)]
        if not js:
            out.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        e = {j: math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j]))
                         - slope * abs(pos - j)) for j in js}
        z = math.fsum(e.values())
        out.append([math.fsum(e[j] / z * float(v[j][c]) for j in js) for c in range(len(v[0]))])
        lse.append(math.log(z))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("n_q,n_k", [(1, 9), (5, 12), (9, 9), (12, 5)])
def test_alibi_brute_force(causal, window, n_q, n_k):
    q, k, v = _qkv(n_q, n_k, 4, seed=3 * n_q + n_k)
    o, lse = oracle.cross_forward(q, k, v, 0.5, causal, window, slope=0.37)
    bo, bl = _brute_alibi(q, k, v, 0.5, 0.37, causal, window)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n_q,n_k", [(3, 8), (8, 8), (8, 5)])
def test_alibi_torch_float_mask(n_q, n_k):
    """torch CPU float64 SDPA with an additive float mask: -slope |p - j| on visible pairs,
    -inf elsewhere (torch adds a float attn_mask to the scaled scores)."""
    q, k, v = _qkv(n_q, n_k, 5, seed=n_q * 11 + n_k)
    pos = torch.arange(n_q, dtype=torch.float64)[:, None] + (n_k - n_q)
    j = torch.arange(n_k, dtype=torch.float64)[None, :]
    bias = -0.25 * (pos - j).abs()
    bias = bias.masked_fill(j > pos, float("-inf"))
    live = torch.isfinite(bias).any(dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=bias[None], scale=0.6)[0].numpy()
    o, _ = oracle.cross_forward(q, k, v, 0.6, causal=True, slope=0.25)
    np.testing.assert_allclose(o[live.numpy()], ref[live.numpy()], rtol=1e-12, atol=1e-12)


def test_alibi_closed_form_geometric():
    """Q = 0, one query at the end of n keys, causal: the weights are e^{-slope d} over the
    distances d = 0 .. n-1, so LSE = ln((1 - e^{-slope n}) / (1 - e^{-slope})) and O is the
    e^{-slope d}-weighted mean of V."""
    n, slope = 50, 0.3
    _, k, v = _qkv(1, n, 3, seed=4)
    o, lse = oracle.cross_forward(np.zeros((1, 3)), k, v, 1.0, causal=True, slope=slope)
    z = (1 - math.exp(-slope * n)) / (1 - math.exp(-slope))
    assert abs(lse[0] - math.log(z)) < 1e-13
    w = np.exp(-slope * (n - 1 - np.arange(n)))
    np.testing.assert_allclose(o[0], (w[:, None] * v).sum(axis=0) / w.sum(), rtol=1e-12)


def test_alibi_zero_slope_is_plain():
    q, k, v = _qkv(4, 9, 3, seed=6)
    a = oracle.cross_forward(q, k, v, 0.5, True, slope=0.0)
    b = oracle.cross_forward(q, k, v, 0.5, True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (-1, -1)), (False, (2, 3))])
def test_alibi_backward_central_differences(causal, window):
    rng = np.random.default_rng(31)
    q, k, v, do = (rng.standard_normal((r, 3)) for r in (4, 6, 6, 4))
    dq, dk, dv = oracle.cross_backward(q, k, v, do, 0.7, causal, window, slope=0.45)
    h = 1e-6

    def loss(q_, k_, v_):
        return float((oracle.cross_forward(q_, k_, v_, 0.7, causal, window, slope=0.45)[0]
                      * do).sum())

    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[which], args_m[which] = plus, minus
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7)


def test_mutant_alibi_sign_fails_closed_form():
    """A bias of the wrong sign (+slope |p - j|) is a plausible mistake; the geometric closed
    form rejects it."""
    n, slope = 20, 0.3
    ok = np.ones((1, n), dtype=bool)
    s = np.where(ok, +slope * np.abs((n - 1) - np.arange(n))[None, :], -np.inf)
    lse_wrong = float(np.log(np.exp(s).sum()))
    z = (1 - math.exp(-slope * n)) / (1 - math.exp(-slope))
    assert abs(lse_wrong - math.log(z)) > 1.0


# ---------------------------------------------------------------------------- block-sparse
def _random_blocks(n_qb, n_kb, seed, density=0.5):
    return np.random.default_rng(seed).random((n_qb, n_kb)) < density


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (70, 30))])
@pytest.mark.parametrize("n_q,n_k", [(130, 200), (64, 64), (200, 70)])
def test_block_sparse_torch_bool_mask(causal, window, n_q, n_k):
    """torch CPU float64 SDPA with a boolean mask expanded from the blocks by torch's own
    repeat_interleave, ANDed with the position mask written out with tril / triu."""
    q, k, v = _qkv(n_q, n_k, 4, seed=n_q + n_k)
    bm = _random_blocks(-(-n_q // 64), -(-n_k // 64), seed=n_q * n_k)
    tb = torch.from_numpy(bm).repeat_interleave(64, 0).repeat_interleave(64, 1)[:n_q, :n_k]
    off = n_k - n_q
    pos = torch.ones(n_q, n_k, dtype=torch.bool)
    if causal:
        pos &= torch.ones(n_q, n_k, dtype=torch.bool).tril(diagonal=off)
    if window[0] >= 0:
        pos &= torch.ones(n_q, n_k, dtype=torch.bool).triu(diagonal=off - window[0])
    if window[1] >= 0:
        pos &= torch.ones(n_q, n_k, dtype=torch.bool).tril(diagonal=off + window[1])
    mask = tb & pos
    live = mask.any(dim=1).numpy()
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=mask[None], scale=0.4)[0].numpy()
    o, lse = oracle.cross_forward(q, k, v, 0.4, causal, window, block_mask=bm)
    np.testing.assert_allclose(o[live], ref[live], rtol=1e-12, atol=1e-12)
    assert np.all(o[~live] == 0.0) and np.all(np.isneginf(lse[~live]))


def test_block_diagonal_is_attention_within_blocks():
    """A block-diagonal mask over equal-length queries and keys is self-attention of each
    64-row block on its own."""
    n = 200
    q, k, v = _qkv(n, n, 5, seed=8)
    nb = -(-n // 64)
    o, lse = oracle.cross_forward(q, k, v, 0.5, False, block_mask=np.eye(nb, dtype=bool))
    for b in range(nb):
        sl = slice(64 * b, min(64 * (b + 1), n))
        ro, rl = oracle.attention_forward(q[sl], k[sl], v[sl], 0.5)
        np.testing.assert_allclose(o[sl], ro, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[sl], rl, rtol=1e-13, atol=1e-13)


def test_block_sparse_all_blocks_is_plain():
    q, k, v = _qkv(100, 150, 4, seed=9)
    a = oracle.cross_forward(q, k, v, 0.5, True, block_mask=np.ones((2, 3), bool))
    b = oracle.cross_forward(q, k, v, 0.5, True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_block_sparse_backward_central_differences():
    rng = np.random.default_rng(10)
    n_q, n_k = 70, 130   # two query blocks, three key blocks; d = 2 keeps it quick
    q, k, v, do = (rng.standard_normal((r, 2)) for r in (n_q, n_k, n_k, n_q))
    bm = np.array([[1, 0, 1], [0, 1, 1]], dtype=bool)
    dq, dk, dv = oracle.cross_backward(q, k, v, do, 0.6, True, block_mask=bm)
    h = 1e-6

    def loss(q_, k_, v_):
        return float((oracle.cross_forward(q_, k_, v_, 0.6, True, block_mask=bm)[0] * do).sum())

    rows = [(0, 0, (3, 1)), (0, 1, (66, 0)), (1, 2, (5, 1)), (1, 0, (100, 1)), (2, 0, (129, 0))]
    args = [q, k, v]
    for which, grad_i, idx in [(w, w, i) for w, _, i in rows]:
        grad = (dq, dk, dv)[grad_i]
        plus, minus = args[which].copy(), args[which].copy()
        plus[idx] += h
        minus[idx] -= h
        ap, am = list(args), list(args)
        ap[which], am[which] = plus, minus
        num = (loss(*ap) - loss(*am)) / (2 * h)
        assert abs(grad[idx] - num) <= 1e-6 * max(1.0, abs(num))


# ---------------------------------------------------------------------------- key padding mask
def _random_key_mask(n_k, seed, density=0.3):
    """True = padding key; holes anywhere (not only a padded tail)."""
    return np.random.default_rng(seed).random(n_k) < density


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (6, 3)),
                                           (True, (5, -1))])
@pytest.mark.parametrize("n_q,n_k", [(1, 40), (9, 9), (12, 30), (30, 12)])
def test_key_padding_torch_bool_mask(causal, window, n_q, n_k):
    """torch CPU float64 SDPA with the boolean mask ~key_mask broadcast over the queries by
    torch, ANDed with the position mask written out with tril / triu."""
    q, k, v = _qkv(n_q, n_k, 4, seed=3 * n_q + n_k)
    km = _random_key_mask(n_k, seed=n_q * n_k + 1)
    off = n_k - n_q
    pos = torch.ones(n_q, n_k, dtype=torch.bool)
    if causal:
        pos &= torch.ones(n_q, n_k, dtype=torch.bool).tril(diagonal=off)
    if window[0] >= 0:
        pos &= torch.ones(n_q, n_k, dtype=torch.bool).triu(diagonal=off - window[0])
    if window[1] >= 0:
        pos &= torch.ones(n_q, n_k, dtype=torch.bool).tril(diagonal=off + window[1])
    mask = pos & ~torch.from_numpy(km)[None, :]
    live = mask.any(dim=1).numpy()
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=mask[None], scale=0.55)[0].numpy()
    o, lse = oracle.cross_forward(q, k, v, 0.55, causal, window, key_mask=km)
    np.testing.assert_allclose(o[live], ref[live], rtol=1e-12, atol=1e-12)
    assert np.all(o[~live] == 0.0) and np.all(np.isneginf(lse[~live]))


def test_key_padding_is_attention_over_the_other_keys():
    """Without a position mask, hiding keys is the same as deleting their rows of K and V."""
    n_q, n_k = 7, 25
    q, k, v = _qkv(n_q, n_k, 5, seed=17)
    km = _random_key_mask(n_k, seed=18, density=0.4)
    o, lse = oracle.cross_forward(q, k, v, 0.7, key_mask=km)
    ro, rl = oracle.cross_forward(q, k[~km], v[~km], 0.7)
    np.testing.assert_allclose(o, ro, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_key_padding_all_keys_hidden_and_none_hidden():
    q, k, v = _qkv(5, 8, 3, seed=19)
    o, lse = oracle.cross_forward(q, k, v, 0.5, True, key_mask=np.ones(8, bool))
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
    a = oracle.cross_forward(q, k, v, 0.5, True, key_mask=np.zeros(8, bool))
    b = oracle.cross_forward(q, k, v, 0.5, True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_key_padding_suffix_is_a_shorter_sequence():
    """Hiding the last keys of a non-causal call is the call over the first ones (the padded
    batch of a sequence of that length)."""
    q, k, v = _qkv(6, 20, 4, seed=20)
    km = np.arange(20) >= 13
    o, lse = oracle.cross_forward(q, k, v, 0.4, False, (3, 2), key_mask=km)
    # the same positions: queries still sit at the last 6 of 20 positions
    ok = oracle.cross_allowed_mask(6, 20, False, (3, 2)) & ~km[None, :]
    for i in range(6):
        js = np.nonzero(ok[i])[0]
        if len(js) == 0:
            assert o[i].sum() == 0.0 and np.isneginf(lse[i])
            continue
        s = 0.4 * (k[js] @ q[i])
        z = np.exp(s - s.max())
        np.testing.assert_allclose(o[i], (z / z.sum()) @ v[js], rtol=1e-13, atol=1e-13)


def test_key_padding_backward_torch_autograd():
    """dQ, dK, dV against torch CPU float64 autograd through SDPA with the same boolean mask
    (every row keeps a visible key, so torch's softmax has no NaN rows); the hidden keys get
    zero dK and dV."""
    n_q, n_k = 10, 16
    rng = np.random.default_rng(21)
    q, k, v, do = (rng.standard_normal((r, 4)) for r in (n_q, n_k, n_k, n_q))
    km = np.zeros(n_k, bool)
    km[[0, 3, 4, 9, 15]] = True
    mask = torch.ones(n_q, n_k, dtype=torch.bool).tril(diagonal=n_k - n_q) & ~torch.from_numpy(km)
    assert bool(mask.any(dim=1).all())
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                           attn_mask=mask[None], scale=0.65)[0]
    (out * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = oracle.cross_backward(q, k, v, do, 0.65, True, key_mask=km)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.all(dk[km] == 0.0) and np.all(dv[km] == 0.0)


def test_key_padding_batch_entries_use_their_own_row():
    """The [B, N_k] mask: entry b hides its own keys in every head."""
    rng = np.random.default_rng(22)
    q, k, v = (rng.standard_normal((2, 3, n, 4)) for n in (5, 9, 9))
    km = np.zeros((2, 9), bool)
    km[0, [1, 2]] = True
    km[1, [7, 8]] = True
    o, lse = oracle.cross_forward_bh(q, k, v, 0.5, key_padding_mask=km)
    for b in range(2):
        for h in range(3):
            ro, rl = oracle.cross_forward(q[b, h], k[b, h][~km[b]], v[b, h][~km[b]], 0.5)
            np.testing.assert_allclose(o[b, h], ro, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], rl, rtol=1e-13, atol=1e-13)


def test_mutant_query_side_mask_fails_the_deletion_pin():
    """Applying the mask to the queries instead of the keys is a plausible mistake (a
    transposed broadcast); the key-deletion pin rejects it."""
    n = 12
    q, k, v = _qkv(n, n, 4, seed=23)
    km = _random_key_mask(n, seed=24, density=0.4)
    s = 0.5 * (q @ k.T)
    s = np.where(~km[:, None], s, -np.inf)           # the mistake: rows hidden, not columns
    live = np.isfinite(s.max(axis=1))
    e = np.exp(s - np.where(live, s.max(axis=1), 0.0)[:, None])
    wrong = np.where(live[:, None], (e / np.where(live, e.sum(axis=1), 1.0)[:, None]) @ v, 0.0)
    ro, _ = oracle.cross_forward(q, k[~km], v[~km], 0.5)
    assert np.abs(wrong - ro).max() > 1e-2
