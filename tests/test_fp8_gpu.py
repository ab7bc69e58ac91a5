"""Decode steps over an FP8 E4M3 key/value cache on the GPU: fa_fwd_kv_fp8 through the C ABI
against the float64 oracle (oracle/fp8.py) with the fixed tolerances (max |dO| 2e-3 fp16 /
1e-2 bf16, |dLSE| 1e-3).  Covers head dims 64 and 128, 1, 2 and 4 queries, caches shorter than
a step, ragged tails and key splits, the mask modes, rows without keys, strided caches
([B, N, H, d] memory), and sampled heads of the 16384-key decode shape."""
import numpy as np
import pytest

import workloads as W
from gpu_util import LSE_TOL, O_TOL, say, to64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_125_amd as fa
    return fa


def check(o, lse, c, scale, causal, window, dtype, label, heads=None):
    import oracle
    B, H = c["q64"].shape[:2]
    o64, l64 = to64(o), lse.detach().cpu().numpy().astype(np.float64)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    worst_o = worst_l = 0.0
    for b, h in heads:
        ro, rl = oracle.fp8_cache_forward(c["q64"][b, h], c["k8"][b, h], c["v8"][b, h], scale,
                                          c["k_descale"], c["v_descale"], causal, window)
        empty = np.isneginf(rl)
        assert np.array_equal(np.isneginf(l64[b, h]), empty), f"{label}: rows without keys differ"
        assert np.all(o64[b, h][empty] == 0), f"{label}: rows without keys must be zero"
        live = ~empty
        if live.any():
            worst_o = max(worst_o, float(np.max(np.abs(o64[b, h][live] - ro[live]))))
            worst_l = max(worst_l, float(np.max(np.abs(l64[b, h][live] - rl[live]))))
    say(f"{label}: max|dO| {worst_o:.2e}  max|dLSE| {worst_l:.2e}")
    assert worst_o <= O_TOL[dtype], f"{label}: max|dO| {worst_o:.3e}"
    assert worst_l <= LSE_TOL, f"{label}: max|dLSE| {worst_l:.3e}"


def device_case(c, dtype):
    import torch
    q = to_dev(c["q"])
    k = torch.from_numpy(c["k8"]).cuda()
    v = torch.from_numpy(c["v8"]).cuda()
    return q, k, v


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_q", [1, 2, 4])
@pytest.mark.parametrize("n_k", [1, 77, 700, 5003])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8_cache_causal(fa, d, n_q, n_k, dtype):
    c = W.fp8_cache_case(2, 3, n_q, n_k, d, dtype, seed=11 + n_k + d + n_q)
    q, k, v = device_case(c, dtype)
    scale = d ** -0.5
    o, lse = fa.fwd_kv_fp8(q, k, v, c["k_descale"], c["v_descale"], scale, causal=True)
    check(o, lse, c, scale, True, (-1, -1), dtype, f"fp8 d={d} nq={n_q} nk={n_k} {dtype}")


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (False, (100, 3)), (True, (257, -1)),
                                           (True, (0, -1))])
@pytest.mark.parametrize("n_q,n_k", [(4, 3000), (3, 2), (2, 40000)])
def test_fp8_cache_masks(fa, causal, window, n_q, n_k):
    # (3, 2) under causal: the first query row sees no key
    c = W.fp8_cache_case(1, 4, n_q, n_k, 64, "bf16", seed=5 + n_k)
    q, k, v = device_case(c, "bf16")
    o, lse = fa.fwd_kv_fp8(q, k, v, c["k_descale"], c["v_descale"], 0.125, causal=causal,
                           window_size=window)
    check(o, lse, c, 0.125, causal, window, "bf16", f"fp8 masks {causal} {window} {n_q}x{n_k}")


def test_fp8_cache_strided_and_float8_dtype(fa):
    """Keys and values as transposed views of [B, N, H, d] memory, passed as float8_e4m3fn."""
    import torch
    B, H, n_q, n_k, d = 2, 4, 1, 1500, 128
    c = W.fp8_cache_case(B, H, n_q, n_k, d, "f16", seed=31)
    q = to_dev(c["q"])
    k = torch.from_numpy(np.ascontiguousarray(c["k8"].transpose(0, 2, 1, 3))).cuda()
    v = torch.from_numpy(np.ascontiguousarray(c["v8"].transpose(0, 2, 1, 3))).cuda()
    k = k.view(torch.float8_e4m3fn).transpose(1, 2)
    v = v.view(torch.float8_e4m3fn).transpose(1, 2)
    assert not k.is_contiguous()
    o, lse = fa.fwd_kv_fp8(q, k, v, c["k_descale"], c["v_descale"], d ** -0.5, causal=True)
    check(o, lse, c, d ** -0.5, True, (-1, -1), "f16", "fp8 strided")


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_cache_decode_shape_sampled(fa, d):
    """The 16384-key decode shape (8 batches x 16 heads, one query) in the launch configuration
    the benchmark times, three sampled heads against the oracle."""
    c = W.fp8_cache_case(8, 16, 1, 16384, d, "bf16", seed=40 + d)
    q, k, v = device_case(c, "bf16")
    o, lse = fa.fwd_kv_fp8(q, k, v, c["k_descale"], c["v_descale"], d ** -0.5, causal=True)
    check(o, lse, c, d ** -0.5, True, (-1, -1), "bf16", f"fp8 decode d={d}",
          heads=[(0, 0), (3, 9), (7, 15)])


def test_fp8_cache_matches_the_16_bit_path_on_exact_values(fa):
    """FP8 codes decoded exactly on the host and passed as bf16 (every E4M3 value with a
    power-of-two descale is a bf16 value) give the same attention: both kernels read the same
    numbers, and their fp32 sums differ only in order (the two kernels split the keys and fold
    the key descale differently).  So the LSE agrees to 1e-5 and O, rounded to bf16 at the end,
    to within one bf16 step (an fp32 difference can move a value across a rounding boundary)."""
    import oracle
    import torch
    c = W.fp8_cache_case(2, 2, 2, 3000, 64, "bf16", seed=77)
    q, k, v = device_case(c, "bf16")
    o8, l8 = fa.fwd_kv_fp8(q, k, v, c["k_descale"], c["v_descale"], 0.125, causal=True)
    kb = torch.from_numpy(oracle.e4m3_value(c["k8"]) * c["k_descale"]).to(torch.bfloat16).cuda()
    vb = torch.from_numpy(oracle.e4m3_value(c["v8"]) * c["v_descale"]).to(torch.bfloat16).cuda()
    ob, lb = fa.fwd_kv(q, kb, vb, 0.125, True)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(l8 - lb)).item() <= 1e-5
    assert torch.max(torch.abs(o8.float() - ob.float())).item() <= 2 ** -7   # one bf16 ulp at 1
