"""The dropout oracle against its pins (CPU only).

  * Philox4x32-10 against the known-answer vectors published with the generator
    (J. K. Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011, and the
    Random123 library that accompanies it);
  * the vectorised generator and the counter layout against a scalar pure-Python Philox with
    the layout written out per pair;
  * the fraction of kept pairs against 1 - p (binomial, 6 sigma) and independence of the
    four words of a call;
  * p = 0 is the plain definition; dropout of an all-ones mask is the plain definition
    scaled by the inverse of the keep probability, and that probability (counted over all
    2^16 draws of a pair) times the scale is exactly 1, so the drop is unbiased at every p;
  * averaging the dropout output over many seeds approaches the plain output;
  * central differences of the forward with a fixed mask pin the backward.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

KAT = [  # counter, key -> output (Philox4x32-10)
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = oracle.philox4x32_10(*ctr, *key)
    assert tuple(int(x) for x in got) == out


def _philox_scalar(c, k):
    c, k = list(c), list(k)
    for r in range(10):
        a, b = 0xD2511F53 * c[0], 0xCD9E8D57 * c[2]
        c = [(b >> 32) ^ c[1] ^ k[0], b & 0xFFFFFFFF, (a >> 32) ^ c[3] ^ k[1], a & 0xFFFFFFFF]
        if r < 9:
            k = [(k[0] + 0x9E3779B9) & 0xFFFFFFFF, (k[1] + 0xBB67AE85) & 0xFFFFFFFF]
    return c


@pytest.mark.parametrize("bh,seed,offset,p", [(0, 0, 0, 0.1), (5, 0x123456789ABCDEF, 7, 0.5),
                                              (31, 2 ** 64 - 1, 2 ** 32 - 1, 0.9)])
def test_mask_layout_per_pair(bh, seed, offset, p):
    n_q, n_k = 7, 9
    keep = oracle.dropout_keep(n_q, n_k, bh, p, seed, offset)
    thr = math.floor(p * 2 ** 16)
    for i in range(n_q):
        for j in range(n_k):
            w = _philox_scalar([j >> 2, i >> 1, bh, offset], [seed & 0xFFFFFFFF, seed >> 32])
            t = 4 * (i & 1) + (j & 3)
            u = (w[t >> 1] >> (16 * (t & 1))) & 0xFFFF
            assert keep[i, j] == (u >= thr)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.83])
def test_keep_fraction_and_word_independence(p):
    n = 512
    keeps = [oracle.dropout_keep(n, n, bh, p, seed=2024) for bh in range(4)]
    frac = np.mean([k.mean() for k in keeps])
    expect = 1.0 - math.floor(p * 2 ** 16) / 2 ** 16
    sigma = math.sqrt(expect * (1 - expect) / (4 * n * n))
    assert abs(frac - expect) < 6 * sigma
    k = keeps[0]
    # the draws of one call (2 queries x 4 keys) are independent: agreement of two members
    # of each block from different words matches independent draws
    a, b = k[0::2, 0::4].ravel(), k[1::2, 3::4].ravel()
    agree = np.mean(a == b)
    e2 = expect * expect + (1 - expect) ** 2
    assert abs(agree - e2) < 6 * math.sqrt(e2 * (1 - e2) / a.size)


def _qkv(n_q, n_k, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n_q, d)), rng.standard_normal((n_k, d)), rng.standard_normal((n_k, d))


def test_zero_probability_is_plain():
    q, k, v = _qkv(5, 9, 4, 1)
    keep = oracle.dropout_keep(5, 9, 0, 0.0, seed=3)
    assert keep.all()
    o, lse = oracle.dropout_forward(q, k, v, 0.5, True, (-1, -1), 0.0, 0.0, keep)
    ro, rl = oracle.cross_forward(q, k, v, 0.5, True)
    np.testing.assert_allclose(o, ro, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(lse, rl)
    o2, _ = oracle.dropout_forward(q, k, v, 0.5, True, (-1, -1), 0.0, 0.3, np.ones((5, 9), bool))
    np.testing.assert_allclose(o2 * float(_keep_probability(0.3)), ro, rtol=1e-13, atol=1e-13)


def _keep_probability(p):
    """The probability that a pair is kept, counted over every 16-bit draw u the rule
    ``u >= floor(p 2^16)`` can see (the draws are uniform: see the keep-fraction test)."""
    thr = math.floor(p * 2 ** 16)
    return Fraction(sum(1 for u in range(2 ** 16) if u >= thr), 2 ** 16)


@pytest.mark.parametrize("p", [0.0, 0.1, 1 / 3, 0.5, 0.9, 0.99999, 1 - 2 ** -17])
def test_drop_is_unbiased(p):
    # E[M * scale] = P(kept) * scale must be exactly 1, also where p 2^16 is far from an
    # integer (0.99999: keep probability 1/65536, where 1 / (1 - p) would be 1e5)
    # (up to the float64 rounding of the scale; a factor 1 / (1 - p) is off by 1e-5 at p = 0.1)
    assert abs(_keep_probability(p) * Fraction(oracle.keep_scale(p)) - 1) <= Fraction(1, 2 ** 52)
    # and the scale reaches the output: an all-ones mask times the keep probability is the
    # plain definition
    q, k, v = _qkv(3, 5, 4, 11)
    ro, _ = oracle.cross_forward(q, k, v, 0.5, False)
    o, _ = oracle.dropout_forward(q, k, v, 0.5, False, (-1, -1), 0.0, p, np.ones((3, 5), bool))
    np.testing.assert_allclose(o * float(_keep_probability(p)), ro, rtol=1e-13, atol=1e-13)


def test_mean_over_seeds_approaches_plain_output():
    q, k, v = _qkv(4, 16, 3, 2)
    ro, _ = oracle.cross_forward(q, k, v, 0.5, False)
    acc = np.zeros_like(ro)
    n = 4000
    for seed in range(n):
        keep = oracle.dropout_keep(4, 16, 0, 0.3, seed)
        acc += oracle.dropout_forward(q, k, v, 0.5, False, (-1, -1), 0.0, 0.3, keep)[0]
    # each output is a mean of 16 terms P_ij v_j M_ij / r (r ~ 0.7): its spread is at most
    # max |v| sqrt(0.3 / 0.7); the mean over n seeds must be within 6 sigma of that / sqrt(n)
    bound = 6 * np.abs(v).max() * math.sqrt(0.3 / 0.7) / math.sqrt(n)
    assert np.abs(acc / n - ro).max() < bound


@pytest.mark.parametrize("causal,window,slope", [(True, (-1, -1), 0.0), (False, (2, 1), 0.3)])
def test_backward_central_differences(causal, window, slope):
    rng = np.random.default_rng(9)
    q, k, v, do = (rng.standard_normal((r, 3)) for r in (4, 6, 6, 4))
    keep = oracle.dropout_keep(4, 6, 3, 0.4, seed=77)
    dq, dk, dv = oracle.dropout_backward(q, k, v, do, 0.7, causal, window, slope, 0.4, keep)
    h = 1e-6

    def loss(q_, k_, v_):
        o, _ = oracle.dropout_forward(q_, k_, v_, 0.7, causal, window, slope, 0.4, keep)
        return float((o * do).sum())

    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            ap, am = [q, k, v], [q, k, v]
            ap[which], am[which] = plus, minus
            num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7)


def test_rejects_bad_probability():
    for p in (-0.1, 1.0, 1.5):
        with pytest.raises(ValueError):
            oracle.keep_threshold(p)
