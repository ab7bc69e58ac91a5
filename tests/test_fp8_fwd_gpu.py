"""fa_fwd_fp8 (FP8 E4M3 queries, keys and values) on the GPU through the C ABI against the
float64 oracle over the decoded, descaled values (oracle.fp8_forward).

The kernel rounds each probability once to E4M3 before the product with V (after an exact
power-of-two scaling, 2^4, that keeps the largest ones at most 256) and O once to the output
type; the row sums and the LSE use the unrounded probabilities.

The scores come from the FP8 matrix instruction, whose accumulation is not exact: measured on the
device over 262144 random 64-term dot products of E4M3 values, the error reaches 2^-11.9 of the
sum of the products' magnitudes (0 when all products share one binade), so a score carries
    |dS_ij| <= e_i = 2^-11 |scale| q_descale k_descale max_j sum_c |Q_ic| |K_jc|
(the maximum over the row's visible keys; 2^-11 keeps a factor of about 2 over the measurement).
It moves P_ij by a relative e_i at most, and the normalisation by as much again.

E4M3 rounds x in [0, 448] to within max(2^-4 x, 2^-10) (half a step: 2^-4 relative in the normal
range, 2^-10 absolute among subnormals), and the scaled row sum is at least 2^4 (the reference
never exceeds the row maximum), so per element
    |O_gpu - O_ref| <= (2^-4 + 2 e_i) W + 2^-14 S1 + u_out |O_ref| + 1e-4,
W = sum_j P_ij |V_jc| (the oracle with |V|), S1 = sum_j |V_jc| over the visible keys, u_out the
unit roundoff of the output type, and |LSE_gpu - LSE_ref| <= max(1e-3, e_i + 1e-5).  Those
bounds are the check, on every element.

The full-size workloads also report the relative L2 of O over the whole tensor, the typical
rather than the worst-case effect of the rounding.  With a weight's rounding error uniform over
half a step and the weights spread evenly over a binade in log scale, the RMS relative rounding
of an E4M3 weight is (2^-4 / sqrt 3) sqrt((1 / ln 2) (1/2) (1 - 1/4)) = 2.65e-2, and O, a sum
of weights times independent values, inherits about that relative error; the check allows
1.5 times it, 4e-2.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from full_parity import oracle_heads_fp8
from gpu_util import LSE_TOL, say, to64

pytestmark = pytest.mark.gpu

U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_125_amd as fa
    return fa


def _tdtype(name):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16}[name]


def _run(fa, case, scale, causal, window, out_dtype):
    import torch
    q, k, v = (torch.from_numpy(np.ascontiguousarray(case[n + "8"])).to("cuda") for n in "qkv")
    o, lse = fa.fwd_fp8(q, k, v, case["q_descale"], case["k_descale"], case["v_descale"], scale,
                        causal, window, out_dtype=_tdtype(out_dtype))
    torch.cuda.synchronize()
    return to64(o), lse.cpu().numpy().astype(np.float64)


def _bound(ro, wabs, s1, e_s, out_dtype):
    return ((2.0 ** -4 + 2.0 * e_s[:, None]) * wabs + 2.0 ** -14 * s1
            + U_OUT[out_dtype] * np.abs(ro) + 1e-4)


def score_error(q8, k8, scale, qd, kd, causal, window):
    """e_i = 2^-11 |scale| q_descale k_descale max over visible j of sum_c |Q_ic| |K_jc|."""
    aq, ak = np.abs(oracle.e4m3_value(q8)), np.abs(oracle.e4m3_value(k8))
    vis = oracle.allowed_mask(q8.shape[0], causal, window)
    m = np.where(vis, aq @ ak.T, 0.0).max(axis=1)
    return 2.0 ** -11 * abs(scale) * qd * kd * m


def _check_head(o, lse, case, b, h, scale, causal, window, out_dtype, label):
    q8, k8, v8 = case["q8"][b, h], case["k8"][b, h], case["v8"][b, h]
    args = (scale, case["q_descale"], case["k_descale"], case["v_descale"], causal, window)
    ro, rl = oracle.fp8_forward(q8, k8, v8, *args)
    wabs, _ = oracle.fp8_forward(q8, k8, v8 & 0x7F, *args)
    vis = oracle.allowed_mask(q8.shape[0], causal, window).astype(np.float64)
    s1 = vis @ (case["v_descale"] * np.abs(oracle.e4m3_value(v8)))
    e_s = score_error(q8, k8, scale, case["q_descale"], case["k_descale"], causal, window)
    d = np.abs(o[b, h] - ro)
    bound = _bound(ro, wabs, s1, e_s, out_dtype)
    if np.any(d > bound):
        i, c = np.unravel_index(np.argmax(d - bound), d.shape)
        raise AssertionError(f"{label} b={b} h={h} row={i} col={c}: gpu={o[b, h][i, c]} "
                             f"oracle={ro[i, c]} |d|={d[i, c]:.3e} > bound {bound[i, c]:.3e}")
    dl = np.abs(lse[b, h] - rl)
    lse_bound = np.maximum(LSE_TOL, e_s + 1e-5)
    assert np.all(dl <= lse_bound), (f"{label} b={b} h={h} |dLSE| {float(dl.max()):.3e} beyond "
                                     f"{float(lse_bound[np.argmax(dl - lse_bound)]):.3e}")
    return float(d.max()), float((d / bound).max())


MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (0, 0)), (True, (40, 0)), (False, (3, 5)),
         (False, (100, 0))]


@pytest.mark.parametrize("n", [1, 17, 64, 65, 127, 128, 129, 200, 513, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_fp8_forward_shapes(fa, n, d, out_dtype):
    B, H = (1, 3) if n % 2 else (2, 4)
    case = W.fp8_attention_case((B, H, n, d), seed=2000 + n + d)
    scale = 1.0 / math.sqrt(d)
    for causal, window in MASKS:
        label = f"fp8 n={n} d={d} {out_dtype} causal={causal} window={window}"
        say(f"[fp8] {label}")
        o, lse = _run(fa, case, scale, causal, window, out_dtype)
        worst = 0.0
        for b in range(B):
            for h in range(H):
                worst = max(worst, _check_head(o, lse, case, b, h, scale, causal, window,
                                               out_dtype, label)[1])
        say(f"[fp8] {label}: worst |dO| / bound {worst:.3f}")


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5, 2.0])
@pytest.mark.parametrize("descales", [(1.0, 1.0, 1.0), (0.5, 0.03125, 4.0)])
def test_fp8_forward_scales_and_descales(fa, scale, descales):
    case = W.fp8_attention_case((1, 2, 300, 128), seed=2500)
    case["q_descale"], case["k_descale"], case["v_descale"] = (d / 16 for d in descales)
    for causal, window in [(True, (-1, -1)), (False, (64, 32))]:
        label = f"fp8 scale={scale} descales={descales} causal={causal} window={window}"
        o, lse = _run(fa, case, scale, causal, window, "bf16")
        for h in range(2):
            _check_head(o, lse, case, 0, h, scale, causal, window, "bf16", label)


def test_fp8_forward_empty_and_errors(fa):
    import torch
    z = torch.empty((2, 3, 0, 64), device="cuda", dtype=torch.uint8)
    o, lse = fa.fwd_fp8(z, z, z, 1.0, 1.0, 1.0)
    assert o.shape == (2, 3, 0, 64) and lse.shape == (2, 3, 0)
    x = torch.zeros((1, 1, 8, 64), device="cuda", dtype=torch.uint8)
    with pytest.raises(fa.FaError, match="BAD_SCALE"):
        fa.fwd_fp8(x, x, x, 1.0, 0.0, 1.0)


@pytest.mark.parametrize("w", W.FP8S, ids=lambda w: w.name)
def test_fp8_workload_every_head(fa, w):
    """The full-size FP8 workloads (the benchmark's launch): every element of every head
    within the rounding bound, relative L2 of O over the workload within 4e-2."""
    say(f"[fp8 full] {w.name}")
    case = W.fp8_attention_case(w.shape, w.seed)
    o, lse = _run(fa, case, w.softmax_scale, w.causal, w.window, w.out_dtype)
    del case
    err2 = ref2 = 0.0
    worst_d = worst_ratio = worst_lse = 0.0
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h, (ro, rl, wabs, s1, e_s) in oracle_heads_fp8(w, heads, progress=say):
        d = np.abs(o[b, h] - ro)
        bound = _bound(ro, wabs, s1, e_s, w.out_dtype)
        ratio = float((d / bound).max())
        assert ratio <= 1.0, f"{w.name} b={b} h={h}: |dO| beyond the rounding bound ({ratio:.3f})"
        worst_d, worst_ratio = max(worst_d, float(d.max())), max(worst_ratio, ratio)
        dl = np.abs(lse[b, h] - rl)
        assert np.all(dl <= np.maximum(LSE_TOL, e_s + 1e-5)), f"{w.name} b={b} h={h} LSE"
        worst_lse = max(worst_lse, float(dl.max()))
        err2 += float((d * d).sum())
        ref2 += float((ro * ro).sum())
    rel = math.sqrt(err2 / ref2)
    say(f"[fp8 full] {w.name}: max|dO|={worst_d:.3e} worst |dO|/bound={worst_ratio:.3f} "
        f"max|dLSE|={worst_lse:.3e} rel L2 O={rel:.3e}")
    assert rel <= 4e-2
