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
