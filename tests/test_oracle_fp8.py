"""Pins of oracle/fp8.py (the FP8 E4M3 cache oracle), none of which re-types its formula:
every code against torch's float8_e4m3fn type (a library implementation of the OCP format),
the format's documented extremes, monotonic ordering, and the descale placement by invariants
of the attention definition."""
import numpy as np
import pytest
import torch

import oracle


def test_every_code_matches_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isnan(got), np.isin(codes, [0x7F, 0xFF]))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))   # -0 at 0x80


@pytest.mark.parametrize("code,value", [(0x00, 0.0), (0x38, 1.0), (0xB8, -1.0), (0x40, 2.0),
                                        (0x7E, 448.0), (0xFE, -448.0), (0x01, 2.0 ** -9),
                                        (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
                                        (0x3C, 1.5), (0x30, 0.5)])
def test_documented_values(code, value):
    # OCP 8-bit floating point, E4M3: max normal 448 = 1.75 * 2^8, min subnormal 2^-9,
    # min normal 2^-6, and the exactly representable 0.5, 1, 1.5, 2
    assert oracle.e4m3_value([code])[0] == value


def test_positive_codes_increase():
    v = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(oracle.e4m3_value(np.arange(0x80, 0xFF, dtype=np.uint8)), -v)


def _case(seed, n_q=3, n_k=50, d=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_q, d))
    k8 = rng.integers(0, 0x7F, (n_k, d), dtype=np.uint8) | (rng.integers(0, 2, (n_k, d), dtype=np.uint8) << 7)
    v8 = rng.integers(0, 0x7F, (n_k, d), dtype=np.uint8) | (rng.integers(0, 2, (n_k, d), dtype=np.uint8) << 7)
    k8 = np.where((k8 & 0x7F) > 0x50, k8 & 0xBF, k8)   # keep magnitudes moderate: |value| < 8
    return q, k8, v8


def test_key_descale_acts_like_the_softmax_scale():
    q, k8, v8 = _case(1)
    kd = 0.37
    o1, l1 = oracle.fp8_cache_forward(q, k8, v8, 0.25, kd, 1.0, causal=True)
    o2, l2 = oracle.fp8_cache_forward(q, k8, v8, 0.25 * kd, 1.0, 1.0, causal=True)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_value_descale_scales_the_output_only():
    q, k8, v8 = _case(2)
    o1, l1 = oracle.fp8_cache_forward(q, k8, v8, 0.25, 1.0, 1.0, window=(7, -1))
    o2, l2 = oracle.fp8_cache_forward(q, k8, v8, 0.25, 1.0, 3.0, window=(7, -1))
    np.testing.assert_allclose(o2, 3.0 * o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(l1, l2)


def test_one_key_returns_its_value():
    # a single visible key: softmax weight 1, O is that key's descaled value row
    q, k8, v8 = _case(3, n_q=1, n_k=1)
    o, lse = oracle.fp8_cache_forward(q, k8, v8, 0.5, 0.125, 0.25)
    np.testing.assert_allclose(o[0], 0.25 * oracle.e4m3_value(v8[0]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.5 * 0.125 * q[0] @ oracle.e4m3_value(k8[0]), rtol=1e-14)


# --------------------------------------------------------------------------- FP8 forward
def _codes(rng, shape, amax=16.0):
    """E4M3 codes of N(0, 1) * amax, rounded by torch's float8_e4m3fn conversion."""
    x = torch.from_numpy(rng.standard_normal(shape) * amax)
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_reference(q8, k8, v8, scale, qd, kd, vd, causal, window):
    """Library cross-check: torch decodes the codes (float8_e4m3fn) and torch CPU SDPA in float64
    computes the attention with a boolean mask of the visible pairs."""
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64)
    q, k, v = qd * dec(q8), kd * dec(k8), vd * dec(v8)
    n = k.shape[0]
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    ok = torch.ones(n, n, dtype=torch.bool)
    wl, wr = window
    if causal:
        ok &= j <= i
    if wl >= 0:
        ok &= j >= i - wl
    if wr >= 0:
        ok &= j <= i + wr
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=ok,
                                                         scale=scale)[0]
    s = (q @ k.T) * scale
    lse = torch.logsumexp(s.masked_fill(~ok, float("-inf")), dim=1)
    return o.numpy(), lse.numpy()


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 2)),
                                           (True, (5, 0))])
def test_fp8_forward_matches_torch(causal, window):
    rng = np.random.default_rng(11)
    q8, k8, v8 = (_codes(rng, (23, 16)) for _ in range(3))
    args = (0.25, 1 / 16, 1 / 8, 1 / 32)
    o, lse = oracle.fp8_forward(q8, k8, v8, *args, causal=causal, window=window)
    ro, rl = _torch_reference(q8, k8, v8, *args, causal, window)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)
    # the row-restricted form is the same rows of the whole
    r = [0, 7, 22]
    o2, l2 = oracle.fp8_forward(q8, k8, v8, *args, causal=causal, window=window, rows=r)
    np.testing.assert_array_equal(o2, o[r])
    np.testing.assert_array_equal(l2, lse[r])


def test_fp8_forward_descales():
    # the query and key descales multiply every score like the softmax scale; the value
    # descale multiplies O and leaves the LSE alone
    rng = np.random.default_rng(12)
    q8, k8, v8 = (_codes(rng, (30, 8)) for _ in range(3))
    o1, l1 = oracle.fp8_forward(q8, k8, v8, 0.3, 0.5, 0.25, 1.0, causal=True)
    o2, l2 = oracle.fp8_forward(q8, k8, v8, 0.3 * 0.5 * 0.25, 1.0, 1.0, 1.0, causal=True)
    o3, l3 = oracle.fp8_forward(q8, k8, v8, 0.3, 0.5, 0.25, 3.0, causal=True)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o3, 3.0 * o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(l3, l1)


def test_fp8_forward_causal_row_zero():
    # row 0 under a causal mask sees only key 0: O_0 = v_descale value(V_0),
    # LSE_0 = scale q_descale k_descale <value(Q_0), value(K_0)>
    rng = np.random.default_rng(13)
    q8, k8, v8 = (_codes(rng, (9, 16)) for _ in range(3))
    o, lse = oracle.fp8_forward(q8, k8, v8, 0.125, 0.5, 2.0, 0.25, causal=True)
    np.testing.assert_allclose(o[0], 0.25 * oracle.e4m3_value(v8[0]), rtol=0, atol=1e-15)
    qv, kv = oracle.e4m3_value(q8[0]), oracle.e4m3_value(k8[0])
    assert abs(lse[0] - 0.125 * 0.5 * 2.0 * float(qv @ kv)) <= 1e-12 * (1 + abs(lse[0]))


def test_fp8_forward_mutant_is_caught():
    # a copy of the oracle that applies the value descale to the keys instead fails the pins
    rng = np.random.default_rng(14)
    q8, k8, v8 = (_codes(rng, (12, 8)) for _ in range(3))

    def mutant(q8, k8, v8, scale, qd, kd, vd, causal=False, window=(-1, -1)):
        return oracle.attention_forward(qd * oracle.e4m3_value(q8), vd * oracle.e4m3_value(k8),
                                        kd * oracle.e4m3_value(v8), scale, causal, window)
    args = (0.25, 1 / 16, 1 / 8, 1 / 32)
    ro, _ = _torch_reference(q8, k8, v8, *args, True, (-1, -1))
    mo, _ = mutant(q8, k8, v8, *args, causal=True)
    assert np.abs(mo - ro).max() > 1e-3
