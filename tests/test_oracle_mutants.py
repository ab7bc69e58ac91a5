"""Broken copies of the oracle must fail at least one pin (CPU only).

Each mutant plants one plausible slip in an otherwise faithful copy of the oracle's
arithmetic; the test asserts that the pin suite rejects it.  This is what makes the
pins evidence: a pin set that passes these mutants would not notice the same slip in
the oracle itself.
"""
import numpy as np
import pytest

import pins


def _mask(n, causal, window, off_causal=0, off_left=0, off_right=0):
    left, right = window
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    ok = np.ones((n, n), dtype=bool)
    if causal:
        ok &= j <= i + off_causal
    if left >= 0:
        ok &= j >= i - left + off_left
    if right >= 0:
        ok &= j <= i + right + off_right
    return ok


def make_fwd(mutation=None):
    def fwd(q, k, v, scale, causal, window):
        n = k.shape[0]
        ok = _mask(n, causal, window,
                   off_causal=-1 if mutation == "causal_strict" else 0,
                   off_left=1 if mutation == "left_off_by_one" else 0,
                   off_right=1 if mutation == "right_off_by_one" else 0)
        if mutation == "window_swapped":
            ok = _mask(n, causal, (window[1], window[0]))
        sc = 1.0 if mutation == "scale_dropped" else scale
        kk = -k if mutation == "sign_flip" else k
        s = sc * (q @ kk.T)
        if mutation == "scale_squared":
            s = s * scale
        s = np.where(ok, s, -np.inf)
        m = s.max(axis=1)
        if mutation == "no_max_shift":
            with np.errstate(over="ignore", invalid="ignore"):
                e = np.exp(s)
                lcl = e.sum(axis=1)
                p = e / lcl[:, None]
                return p @ v, np.log(lcl)
        e = np.exp(s - m[:, None])
        lcl = e.sum(axis=1)
        p = e / lcl[:, None]
        if mutation == "unnormalised":
            p = e
        if mutation == "transposed_p":
            p = p.T
        o = p @ v
        lse = m + np.log(lcl)
        if mutation == "lse_drops_max":
            lse = np.log(lcl)
        if mutation == "lse_log2":
            lse = m + np.log2(lcl)
        if mutation == "v_is_k":
            o = p @ k[:, :v.shape[1]] if k.shape[1] >= v.shape[1] else p @ np.resize(k, v.shape)
        return o, lse
    return fwd


def make_bwd(mutation=None):
    ref = make_fwd()

    def bwd(q, k, v, do, scale, causal, window):
        n = k.shape[0]
        ok = _mask(n, causal, window)
        s = np.where(ok, scale * (q @ k.T), -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dv = p.T @ do
        if mutation == "dv_untransposed":
            dv = p @ do
        dp = do @ v.T
        d = (p * dp).sum(axis=1, keepdims=True)
        if mutation == "no_d_term":
            d = 0.0
        ds = p * (dp - d)
        if mutation == "ds_sign":
            ds = -ds
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if mutation == "dk_no_scale":
            dk = ds.T @ q
        if mutation == "dq_uses_q":
            dq = scale * (ds @ q)
        if mutation == "dk_uses_k":
            dk = scale * (ds.T @ k)
        return dq, dk, dv
    bwd.fwd = ref
    return bwd


FWD_MUTANTS = ["causal_strict", "left_off_by_one", "right_off_by_one", "window_swapped",
               "scale_dropped", "sign_flip", "scale_squared", "no_max_shift", "unnormalised",
               "transposed_p", "lse_drops_max", "lse_log2", "v_is_k"]
BWD_MUTANTS = ["dv_untransposed", "no_d_term", "ds_sign", "dk_no_scale", "dq_uses_q",
               "dk_uses_k"]


def _fails_some(checks, impl):
    for check in checks:
        try:
            check(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


def test_faithful_copy_passes():
    for check in pins.FORWARD_CHECKS:
        check(make_fwd())
    for check in pins.BACKWARD_CHECKS:
        check(make_bwd())


@pytest.mark.parametrize("mutation", FWD_MUTANTS)
def test_forward_mutant_is_caught(mutation):
    assert _fails_some(pins.FORWARD_CHECKS, make_fwd(mutation)), mutation


@pytest.mark.parametrize("mutation", BWD_MUTANTS)
def test_backward_mutant_is_caught(mutation):
    assert _fails_some(pins.BACKWARD_CHECKS, make_bwd(mutation)), mutation
