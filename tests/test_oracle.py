"""The oracle against its pins (CPU only)."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle.online import attention_forward_online

import pins


def fwd(q, k, v, scale, causal, window):
    return oracle.attention_forward(q, k, v, scale, causal, window)


def bwd(q, k, v, do, scale, causal, window):
    return oracle.attention_backward(q, k, v, do, scale, causal, window)


@pytest.mark.parametrize("check", pins.FORWARD_CHECKS, ids=lambda c: c.__name__)
def test_forward_pin(check):
    check(fwd)


def test_forward_brute_force():
    pins.check_brute_force(fwd, oracle.attention_forward_brute)


def test_brute_force_hand_cases():
    # the scalar evaluation is itself pinned by the hand-derived answers
    def brute(q, k, v, scale, causal, window):
        o, l = oracle.attention_forward_brute(q.tolist(), k.tolist(), v.tolist(), scale, causal,
                                              window)
        return np.array(o), np.array(l)
    pins.check_hand_cases(brute)
    pins.check_zero_query(brute)


@pytest.mark.parametrize("check", pins.BACKWARD_CHECKS, ids=lambda c: c.__name__)
def test_backward_pin(check):
    check(bwd)


def test_backward_finite_differences():
    pins.check_finite_differences(bwd, fwd)


def test_mask_matches_loops():
    for n in (1, 5, 13):
        for causal, window in pins.MASKS:
            assert np.array_equal(oracle.allowed_mask(n, causal, window),
                                  pins.visible(n, causal, window))


def test_allowed_pairs_closed_forms():
    # full: N^2; causal: N(N+1)/2; causal with left window w: sum_i (min(i, w) + 1)
    for n in (1, 7, 64, 300):
        assert oracle.allowed_pairs(n, False) == n * n
        assert oracle.allowed_pairs(n, True) == n * (n + 1) // 2
        for w in (0, 3, 50):
            assert oracle.allowed_pairs(n, True, (w, 0)) == sum(min(i, w) + 1 for i in range(n))


def test_rows_variant_matches_full():
    rng = np.random.default_rng(30)
    n, d = 40, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    rows = [0, 3, 17, 39]
    for causal, window in pins.MASKS:
        o, lse = fwd(q, k, v, 0.3, causal, window)
        o2, lse2 = oracle.attention_forward_rows(q, k, v, 0.3, causal, window, rows=rows)
        assert np.array_equal(o[rows], o2) and np.array_equal(lse[rows], lse2)


def test_batched_wrappers():
    rng = np.random.default_rng(31)
    q, k, v, do = (rng.standard_normal((2, 3, 9, 4)) for _ in range(4))
    o, lse = oracle.attention_forward_bh(q, k, v, 0.5, True, (2, 0))
    dq, dk, dv = oracle.attention_backward_bh(q, k, v, do, 0.5, True, (2, 0))
    for b in range(2):
        for h in range(3):
            o1, l1 = fwd(q[b, h], k[b, h], v[b, h], 0.5, True, (2, 0))
            g = bwd(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True, (2, 0))
            assert np.array_equal(o[b, h], o1) and np.array_equal(lse[b, h], l1)
            for a, c in zip((dq, dk, dv), g):
                assert np.array_equal(a[b, h], c)


@pytest.mark.parametrize("bq,bk", [(1, 1), (4, 4), (8, 3), (16, 32), (64, 64), (128, 64)])
def test_online_recurrence_equals_definition(bq, bk):
    """The tiled running-max / running-sum recurrence gives the definition's numbers."""
    rng = np.random.default_rng(32)
    for n in (1, 37, 130):
        q, k, v = (rng.standard_normal((n, 16)) for _ in range(3))
        for causal, window in pins.MASKS + [(True, (20, 0)), (False, (40, 7))]:
            o, lse = fwd(q, k, v, 0.25, causal, window)
            o2, lse2 = attention_forward_online(q, k, v, 0.25, causal, window, bq, bk)
            assert np.allclose(o, o2, rtol=0, atol=1e-12)
            assert np.allclose(lse, lse2, rtol=0, atol=1e-12)


def test_online_skips_exactly_the_hidden_tiles():
    """A key tile is visited iff at least one of its (query, key) pairs is allowed."""
    rng = np.random.default_rng(33)
    n, bq, bk = 100, 16, 8
    q, k, v = (rng.standard_normal((n, 4)) for _ in range(3))
    for causal, window in pins.MASKS + [(True, (20, 0))]:
        _, _, visits = attention_forward_online(q, k, v, 0.5, causal, window, bq, bk,
                                                return_visits=True)
        ok = pins.visible(n, causal, window)
        want = {(i0 // bq, j0 // bk) for i0 in range(0, n, bq) for j0 in range(0, n, bk)
                if ok[i0:i0 + bq, j0:j0 + bk].any()}
        assert set(visits) == want and len(visits) == len(want)


def test_online_pins():
    # the recurrence passes the same forward pins as the definition
    def online(q, k, v, scale, causal, window):
        return attention_forward_online(q, k, v, scale, causal, window, 4, 2)
    for check in pins.FORWARD_CHECKS:
        check(online)


def test_score_matrix_sizes_printed_on_pages():
    path = os.path.join(pins.GOLDEN, "pages_memory.txt")
    rows = 0
    with open(path, encoding="utf-8") as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split("|")]
            n, item, b, h, printed, tol = (int(parts[2]), int(parts[3]), int(parts[4]),
                                          int(parts[5]), float(parts[6]), float(parts[7]))
            got = oracle.score_matrix_nbytes(n, item) * b * h
            assert abs(got - printed) / printed <= tol, line
            rows += 1
    assert rows == 5
    # and the definition does materialise one N x N score block per head
    q = np.zeros((5, 2))
    s = A._scores(q, q, 1.0, np.ones((5, 5), dtype=bool))
    assert s.shape == (5, 5) and s.nbytes == oracle.score_matrix_nbytes(5, 8)


def test_fully_masked_row_convention():
    # unreachable with the supported masks; defined anyway as O = 0, LSE = -inf
    q = k = v = np.ones((1, 2))
    ok = np.zeros((1, 1), dtype=bool)
    p, m, l = A._softmax_rows(A._scores(q, k, 1.0, ok))
    assert np.all(p == 0) and m[0] == -math.inf and l[0] == 0
