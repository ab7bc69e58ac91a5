"""The padded-batch oracle against its pins (CPU only): a key-padding-mask formulation over the
whole padded rows, independence from the padding's contents, the unpadded definition at full
length, and finite differences of its own forward."""
import math

import numpy as np
import pytest

import oracle


def _inputs(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) for _ in range(4)]


def _key_padding_reference(q, k, v, L, scale, causal, window):
    """One (batch, head) over all N rows, keys at or past L set to -inf before the softmax
    (the key padding mask of the FA3.7 page's §4.2 module), every visibility condition
    written out per pair; returns (O, LSE) of the rows below L."""
    N = q.shape[0]
    left, right = window
    s = scale * (q @ k.T)
    for i in range(N):
        for j in range(N):
            hidden = (j >= L or (causal and j > i) or (left >= 0 and j < i - left)
                      or (right >= 0 and j > i + right))
            if hidden:
                s[i, j] = -np.inf
    s = s[:L]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    o = (e / e.sum(axis=1, keepdims=True)) @ v
    return o, m[:, 0] + np.log(e.sum(axis=1))


MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 2)), (True, (4, -1))]


@pytest.mark.parametrize("causal,window", MASKS)
def test_forward_is_key_padding_mask_on_rows_below_length(causal, window):
    q, k, v, _ = _inputs(3, 2, 11, 4, seed=7)
    lens = [11, 6, 1]
    o, lse = oracle.padded_forward_bh(q, k, v, lens, 0.4, causal, window)
    for b, L in enumerate(lens):
        for h in range(2):
            ro, rl = _key_padding_reference(q[b, h], k[b, h], v[b, h], L, 0.4, causal, window)
            np.testing.assert_allclose(o[b, h, :L], ro, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, h, :L], rl, rtol=1e-12, atol=1e-12)
            assert np.all(o[b, h, L:] == 0.0)
            assert np.all(np.isneginf(lse[b, h, L:]))


def test_padding_contents_do_not_matter():
    q, k, v, do = _inputs(2, 2, 9, 4, seed=8)
    lens = [5, 9]
    ref_f = oracle.padded_forward_bh(q, k, v, lens, 0.5, True)
    ref_b = oracle.padded_backward_bh(q, k, v, do, lens, 0.5, True)
    q2, k2, v2, do2 = (t.copy() for t in (q, k, v, do))
    for t in (q2, k2, v2, do2):
        t[0, :, 5:] = 1e3 * np.random.default_rng(9).standard_normal(t[0, :, 5:].shape)
    got_f = oracle.padded_forward_bh(q2, k2, v2, lens, 0.5, True)
    got_b = oracle.padded_backward_bh(q2, k2, v2, do2, lens, 0.5, True)
    for a, b in zip(ref_f + ref_b, got_f + got_b):
        np.testing.assert_array_equal(a, b)


def test_full_lengths_are_the_unpadded_definition():
    q, k, v, do = _inputs(2, 3, 10, 4, seed=10)
    o, lse = oracle.padded_forward_bh(q, k, v, [10, 10], 0.3, False, (2, 5))
    ro, rl = oracle.attention_forward_bh(q, k, v, 0.3, False, (2, 5))
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(lse, rl)
    g = oracle.padded_backward_bh(q, k, v, do, [10, 10], 0.3, False, (2, 5))
    rg = oracle.attention_backward_bh(q, k, v, do, 0.3, False, (2, 5))
    for a, b in zip(g, rg):
        np.testing.assert_array_equal(a, b)


def test_lengths_are_clamped():
    assert oracle.clamp_lengths([-3, 0, 4, 12], 7) == [0, 0, 4, 7]
    q, k, v, _ = _inputs(2, 1, 6, 3, seed=11)
    o, lse = oracle.padded_forward_bh(q, k, v, [-1, 99], 1.0)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    ro, rl = oracle.attention_forward_bh(q[1:], k[1:], v[1:], 1.0)
    np.testing.assert_array_equal(o[1], ro[0])


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (1, 2))])
def test_backward_is_the_derivative_of_the_padded_forward(causal, window):
    """Central differences of <dO, O> over every input element, padding rows included (their
    derivative is zero: they do not reach any output)."""
    q, k, v, do = _inputs(2, 1, 5, 3, seed=12)
    lens = [3, 5]
    scale = 0.7
    grads = oracle.padded_backward_bh(q, k, v, do, lens, scale, causal, window)

    def loss(q_, k_, v_):
        o, _ = oracle.padded_forward_bh(q_, k_, v_, lens, scale, causal, window)
        return float(np.sum(do * o))

    eps = 1e-6
    for which, g in enumerate(grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            num[idx] = (up - loss(*args)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)
        assert np.all(g[0, :, 3:] == 0.0)


# --------------------------------------------------------------------------- packed batches
def _packed_case(cu, H, d, seed):
    rng = np.random.default_rng(seed)
    total = cu[-1]
    return [rng.standard_normal((H, total, d)) for _ in range(4)]


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (2, 1)),
                                           (True, (4, 0))])
def test_packed_is_block_diagonal_attention(causal, window):
    """Library cross-check: torch CPU SDPA over the whole concatenation of a head's rows, with
    a mask that lets (i, j) through only within one sequence and under the mask rules taken
    relative to that sequence's start."""
    import torch
    cu = [0, 5, 5, 12, 13, 20]          # an empty sequence and a one-row one
    H, d = 2, 4
    q, k, v, _ = _packed_case(cu, H, d, 21)
    o, lse = oracle.packed_forward(q, k, v, cu, 16, 0.7, causal, window)
    total = cu[-1]
    seg = np.zeros(total, dtype=np.int64)
    pos = np.zeros(total, dtype=np.int64)
    for b in range(len(cu) - 1):
        seg[cu[b]:cu[b + 1]] = b
        pos[cu[b]:cu[b + 1]] = np.arange(cu[b + 1] - cu[b])
    i, j = pos[:, None], pos[None, :]
    ok = seg[:, None] == seg[None, :]
    if causal:
        ok &= j <= i
    if window[0] >= 0:
        ok &= j >= i - window[0]
    if window[1] >= 0:
        ok &= j <= i + window[1]
    m = torch.from_numpy(ok)
    for h in range(H):
        t = [torch.from_numpy(x[h])[None] for x in (q, k, v)]
        ro = torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=m, scale=0.7)[0]
        np.testing.assert_allclose(o[h], ro.numpy(), rtol=1e-12, atol=1e-12)
        s = (torch.from_numpy(q[h]) @ torch.from_numpy(k[h]).T * 0.7).masked_fill(~m, -np.inf)
        np.testing.assert_allclose(lse[h], torch.logsumexp(s, 1).numpy(), rtol=1e-12, atol=1e-12)


def test_packed_matches_padded_and_leaves_gaps():
    """The same sequences laid out padded give the same outputs (forward and backward); rows no
    sequence covers stay NaN, and offsets beyond the rows are clamped as the kernels clamp them."""
    cu = [0, 7, 7, 19, 22]
    H, d, N = 3, 5, 12
    q, k, v, do = _packed_case(cu, H, d, 22)
    B = len(cu) - 1
    lens = [cu[b + 1] - cu[b] for b in range(B)]
    pad = [np.zeros((B, H, N, d)) for _ in range(4)]
    for b in range(B):
        for t, x in zip(pad, (q, k, v, do)):
            t[b, :, :lens[b]] = x[:, cu[b]:cu[b + 1]]
    po, pl = oracle.padded_forward_bh(*pad[:3], lens, 0.4, True)
    pg = oracle.padded_backward_bh(*pad, lens, 0.4, True)
    o, lse = oracle.packed_forward(q, k, v, cu, N, 0.4, True)
    g = oracle.packed_backward(q, k, v, do, cu, N, 0.4, True)
    for b in range(B):
        r = slice(cu[b], cu[b + 1])
        np.testing.assert_array_equal(o[:, r], po[b, :, :lens[b]])
        np.testing.assert_array_equal(lse[:, r], pl[b, :, :lens[b]])
        for x, y in zip(g, pg):
            np.testing.assert_array_equal(x[:, r], y[b, :, :lens[b]])
    # a gap (rows 22 .. 24 covered by no sequence) and clamping: an offset past the end counts
    # as the end, a sequence longer than max_seqlen keeps its first max_seqlen rows
    q2 = np.concatenate([q, np.ones((H, 3, d))], axis=1)
    o2, l2 = oracle.packed_forward(q2, q2, q2, [0, 7, 40], 5, 0.4, False)
    assert np.isnan(o2[:, 5:7]).all() and np.isnan(o2[:, 12:]).all()
    assert oracle.packed_ranges([0, 7, 40], 25, 5) == [(0, 5), (7, 12)]
    assert oracle.packed_ranges([3, -2, 9], 8, 100) == [(3, 3), (0, 8)]
