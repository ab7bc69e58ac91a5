"""Checks that pin the oracle to facts that do not come from the oracle itself.

Each ``check_*`` takes an implementation (a callable with the oracle's signature)
and raises AssertionError when the implementation violates the fact.  The tests
run every check on the oracle (all must pass) and on deliberately broken copies of
it (each copy must fail at least one check), so a plausible slip in the oracle —
a dropped term, a wrong sign or index, a transposed operand — cannot go unnoticed.

Forward signature:  fwd(q, k, v, scale, causal, window) -> (O [N, d], LSE [N])
Backward signature: bwd(q, k, v, do, scale, causal, window) -> (dQ, dK, dV)
All float64 numpy, one (batch, head) slice.
"""
from __future__ import annotations

import ast
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

MASKS = [
    (False, (-1, -1)),
    (True, (-1, -1)),
    (False, (2, 0)),
    (False, (0, 2)),
    (False, (1, 3)),
    (True, (3, -1)),
    (True, (2, 5)),      # causal overrides the right bound
    (False, (0, 0)),     # diagonal only
]


# ----------------------------------------------------------------------------- helpers
def visible(n, causal, window):
    """Mask by explicit loops (independent of the oracle's vectorised mask)."""
    left, right = window
    ok = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            good = True
            if causal and j > i:
                good = False
            if left >= 0 and j < i - left:
                good = False
            if right >= 0 and j > i + right:
                good = False
            ok[i, j] = good
    return ok


def rand(rng, *shape):
    return rng.standard_normal(shape)


def eval_expr(text: str) -> float:
    """Evaluate a golden-file expression: numbers, + - * /, unary -, ln(x)."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if isinstance(node, ast.BinOp):
            a, b = ev(node.left), ev(node.right)
            if isinstance(node.op, ast.Add):
                return a + b
            if isinstance(node.op, ast.Sub):
                return a - b
            if isinstance(node.op, ast.Mult):
                return a * b
            if isinstance(node.op, ast.Div):
                return a / b
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
                and node.func.id == "ln" and len(node.args) == 1):
            return math.log(ev(node.args[0]))
        raise ValueError(f"unsupported expression: {text!r}")
    return ev(ast.parse(text, mode="eval"))


def golden_array(rows):
    return np.array([[eval_expr(x) for x in r] for r in rows], dtype=np.float64)


def load_hand_cases():
    with open(os.path.join(GOLDEN, "hand_cases.json"), encoding="utf-8") as f:
        return json.load(f)


# ----------------------------------------------------------------------------- forward pins
def check_hand_cases(fwd):
    """Hand-derived answers (tests/golden/hand_cases.json)."""
    for case in load_hand_cases()["forward"]:
        q, k, v = golden_array(case["q"]), golden_array(case["k"]), golden_array(case["v"])
        scale = eval_expr(case["scale"])
        n = k.shape[0]
        if q.shape[0] < n:                       # single query against the key set
            q = np.vstack([q, np.zeros((n - q.shape[0], q.shape[1]))])
        o, lse = fwd(q, k, v, scale, case["causal"], tuple(case["window"]))
        rows = case.get("queries", list(range(n)))
        want_o = golden_array(case["O"])
        want_l = np.array([eval_expr(x) for x in case["LSE"]])
        assert np.allclose(o[rows], want_o, rtol=0, atol=1e-13), (case["name"], o[rows], want_o)
        assert np.allclose(lse[rows], want_l, rtol=0, atol=1e-13), (case["name"], lse[rows], want_l)


def check_brute_force(fwd, brute):
    """Agreement with the scalar, unshifted-softmax evaluation on tiny shapes."""
    rng = np.random.default_rng(11)
    for n, d in [(1, 1), (2, 3), (5, 4), (9, 5), (7, 2)]:
        for causal, window in MASKS:
            q, k, v = rand(rng, n, d), rand(rng, n, d), rand(rng, n, d + 1)
            scale = 0.7
            o, lse = fwd(q, k, v, scale, causal, window)
            ob, lb = brute(q.tolist(), k.tolist(), v.tolist(), scale, causal, window)
            assert np.allclose(o, np.array(ob), rtol=0, atol=1e-12), (n, d, causal, window)
            assert np.allclose(lse, np.array(lb), rtol=0, atol=1e-12), (n, d, causal, window)


def check_torch_sdpa(fwd):
    """Agreement with torch's CPU float64 scaled_dot_product_attention (boolean mask) and
    torch.logsumexp for the LSE (the library routine of the SDPA API, [FA37] §3.2)."""
    import torch
    rng = np.random.default_rng(12)
    for n, d in [(16, 8), (33, 16)]:
        for causal, window in MASKS:
            q, k, v = rand(rng, n, d), rand(rng, n, d), rand(rng, n, d)
            scale = 1.0 / math.sqrt(d)
            o, lse = fwd(q, k, v, scale, causal, window)
            mask = torch.from_numpy(visible(n, causal, window))
            tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
            to = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=mask[None, None], scale=scale)[0, 0].numpy()
            s = torch.matmul(tq, tk.transpose(-1, -2))[0, 0] * scale
            tl = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1).numpy()
            assert np.allclose(o, to, rtol=0, atol=1e-12), (n, d, causal, window)
            assert np.allclose(lse, tl, rtol=0, atol=1e-12), (n, d, causal, window)


def check_zero_query(fwd):
    """Q = 0 (or scale = 0): every allowed key weighs the same, so O is the mean of V over
    the allowed keys and LSE = ln(#allowed keys)."""
    rng = np.random.default_rng(13)
    n, d = 11, 4
    for causal, window in MASKS:
        ok = visible(n, causal, window)
        k, v = rand(rng, n, d), rand(rng, n, d)
        for q, scale in [(np.zeros((n, d)), 0.9), (rand(rng, n, d), 0.0)]:
            o, lse = fwd(q, k, v, scale, causal, window)
            for i in range(n):
                js = np.nonzero(ok[i])[0]
                assert np.allclose(o[i], v[js].mean(axis=0), rtol=0, atol=1e-13)
                assert abs(lse[i] - math.log(len(js))) < 1e-13


def check_single_key(fwd):
    """N = 1: the only key's value row is returned and LSE = scale * q0.k0."""
    rng = np.random.default_rng(14)
    for causal, window in MASKS:
        q, k, v = rand(rng, 1, 6), rand(rng, 1, 6), rand(rng, 1, 3)
        o, lse = fwd(q, k, v, 0.4, causal, window)
        assert np.allclose(o[0], v[0], rtol=0, atol=1e-14)
        assert abs(lse[0] - 0.4 * float(q[0] @ k[0])) < 1e-14


def check_causal_first_row(fwd):
    """Causal row 0 sees only key 0: O_0 = v_0 and LSE_0 = scale * q0.k0."""
    rng = np.random.default_rng(15)
    for window in [(-1, -1), (3, -1), (0, 0)]:
        q, k, v = rand(rng, 10, 4), rand(rng, 10, 4), rand(rng, 10, 5)
        o, lse = fwd(q, k, v, 0.6, True, window)
        assert np.array_equal(o[0], v[0]) or np.allclose(o[0], v[0], rtol=0, atol=1e-15)
        assert abs(lse[0] - 0.6 * float(q[0] @ k[0])) < 1e-14


def check_constant_values(fwd):
    """All value rows equal c: the weights sum to one, so O = c in every row."""
    rng = np.random.default_rng(16)
    for causal, window in MASKS:
        q, k = rand(rng, 12, 4), rand(rng, 12, 4)
        c = rand(rng, 7)
        o, _ = fwd(q, k, np.tile(c, (12, 1)), 0.8, causal, window)
        assert np.allclose(o, np.tile(c, (12, 1)), rtol=0, atol=1e-13)


def check_identity_values(fwd):
    """V = identity (N = d_v): O is the probability matrix itself.  Its rows sum to one,
    masked entries are exactly 0, and the ratio of two allowed entries is exp of their
    score difference (the defining property of softmax)."""
    rng = np.random.default_rng(17)
    n, d = 9, 3
    for causal, window in MASKS:
        q, k = rand(rng, n, d), rand(rng, n, d)
        p, _ = fwd(q, k, np.eye(n), 0.5, causal, window)
        ok = visible(n, causal, window)
        assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert np.all(p[~ok] == 0.0)
        assert np.all(p[ok] > 0.0)
        for i in range(n):
            js = np.nonzero(ok[i])[0]
            for a in js:
                for b in js:
                    want = math.exp(0.5 * float(q[i] @ k[a]) - 0.5 * float(q[i] @ k[b]))
                    assert abs(p[i, a] / p[i, b] - want) <= 1e-12 * max(1.0, want)


def check_key_permutation(fwd):
    """Without a mask, permuting the key and value rows together changes nothing."""
    rng = np.random.default_rng(18)
    n, d = 23, 8
    q, k, v = rand(rng, n, d), rand(rng, n, d), rand(rng, n, d)
    o, lse = fwd(q, k, v, 0.35, False, (-1, -1))
    perm = rng.permutation(n)
    o2, lse2 = fwd(q, k[perm], v[perm], 0.35, False, (-1, -1))
    assert np.allclose(o, o2, rtol=0, atol=1e-13)
    assert np.allclose(lse, lse2, rtol=0, atol=1e-13)


def check_key_shift(fwd):
    """Adding c to every key adds scale*q_i.c to every score of row i: O is unchanged and
    LSE_i moves by exactly that amount."""
    rng = np.random.default_rng(19)
    n, d = 14, 5
    for causal, window in MASKS:
        q, k, v = rand(rng, n, d), rand(rng, n, d), rand(rng, n, d)
        c = rand(rng, d)
        o, lse = fwd(q, k, v, 0.45, causal, window)
        o2, lse2 = fwd(q, k + c, v, 0.45, causal, window)
        assert np.allclose(o, o2, rtol=0, atol=1e-12)
        assert np.allclose(lse2 - lse, 0.45 * (q @ c), rtol=0, atol=1e-12)


def check_large_scores(fwd):
    """Row scores shifted by a huge constant (exp would overflow without the max shift of
    [A100] §2.2): O is unchanged and LSE moves by that constant."""
    rng = np.random.default_rng(20)
    n, d, big = 10, 4, 5.0e3
    for causal, window in MASKS:
        q, k, v = rand(rng, n, d), rand(rng, n, d), rand(rng, n, d)
        o, lse = fwd(q, k, v, 1.0, causal, window)
        q2 = np.hstack([q, np.full((n, 1), big)])
        k2 = np.hstack([k, np.ones((n, 1))])
        with np.errstate(over="ignore", invalid="ignore"):
            o2, lse2 = fwd(q2, k2, v, 1.0, causal, window)
        assert np.all(np.isfinite(o2)) and np.all(np.isfinite(lse2))
        assert np.allclose(o, o2, rtol=0, atol=1e-10)
        assert np.allclose(lse2 - lse, big, rtol=0, atol=1e-9)


FORWARD_CHECKS = [check_hand_cases, check_torch_sdpa, check_zero_query, check_single_key,
                  check_causal_first_row, check_constant_values, check_identity_values,
                  check_key_permutation, check_key_shift, check_large_scores]


# ----------------------------------------------------------------------------- backward pins
def check_bwd_hand_case(bwd):
    for case in load_hand_cases()["backward"]:
        q, k, v = golden_array(case["q"]), golden_array(case["k"]), golden_array(case["v"])
        do = golden_array(case["do"])
        n = k.shape[0]
        rows = case.get("queries", list(range(n)))
        if q.shape[0] < n:
            # extra query rows get dO = 0, so they contribute nothing to any gradient
            q = np.vstack([q, np.zeros((n - q.shape[0], q.shape[1]))])
            do = np.vstack([do, np.zeros((n - do.shape[0], do.shape[1]))])
        dq, dk, dv = bwd(q, k, v, do, eval_expr(case["scale"]), case["causal"],
                         tuple(case["window"]))
        assert np.allclose(dq[rows], golden_array(case["dQ"]), rtol=0, atol=1e-13), case["name"]
        assert np.allclose(dk, golden_array(case["dK"]), rtol=0, atol=1e-13), case["name"]
        assert np.allclose(dv, golden_array(case["dV"]), rtol=0, atol=1e-13), case["name"]


def check_finite_differences(bwd, fwd):
    """Central differences of L = sum(dO * O(Q, K, V)) in float64 match the gradients."""
    rng = np.random.default_rng(21)
    n, d, h = 6, 3, 1e-6
    for causal, window in MASKS[:6]:
        q, k, v, do = (rand(rng, n, d) for _ in range(4))
        dq, dk, dv = bwd(q, k, v, do, 0.8, causal, window)

        def loss(qq, kk, vv):
            return float((fwd(qq, kk, vv, 0.8, causal, window)[0] * do).sum())

        for which, grad in ((0, dq), (1, dk), (2, dv)):
            num = np.zeros_like(grad)
            for idx in np.ndindex(grad.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                lp = loss(*args)
                args[which][idx] -= 2 * h
                lm = loss(*args)
                num[idx] = (lp - lm) / (2 * h)
            err = np.linalg.norm(num - grad) / max(np.linalg.norm(num), 1e-30)
            assert err < 1e-6, (causal, window, which, err)


def check_torch_autograd(bwd):
    """Agreement with torch CPU float64 autograd through scaled_dot_product_attention."""
    import torch
    rng = np.random.default_rng(22)
    n, d = 20, 8
    for causal, window in MASKS:
        q, k, v, do = (rand(rng, n, d) for _ in range(4))
        tq, tk, tv = (torch.from_numpy(x.copy())[None, None].requires_grad_() for x in (q, k, v))
        mask = torch.from_numpy(visible(n, causal, window))[None, None]
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                               scale=0.3)
        out.backward(torch.from_numpy(do)[None, None])
        dq, dk, dv = bwd(q, k, v, do, 0.3, causal, window)
        for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.allclose(mine, ref[0, 0].numpy(), rtol=0, atol=1e-12), (causal, window)


def check_gradient_sums(bwd):
    """Exact invariants: every probability row sums to one, so sum_j dV_j = sum_i dO_i;
    every row of dS sums to zero, so sum_j dK_j = 0."""
    rng = np.random.default_rng(23)
    n, d = 17, 6
    for causal, window in MASKS:
        q, k, v, do = (rand(rng, n, d) for _ in range(4))
        _, dk, dv = bwd(q, k, v, do, 0.5, causal, window)
        assert np.allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-12)
        assert np.allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-12)


BACKWARD_CHECKS = [check_bwd_hand_case, check_torch_autograd, check_gradient_sums]
