"""Whole-workload parity at full size: the float64 oracle over every (batch, head) of a
workload in a pool of worker processes, compared element by element with the GPU's outputs.

The workers are started with the ``spawn`` method (fresh interpreters; the test process
itself has already used the GPU, and the workers never touch it).  Each worker draws the
workload's seeded inputs itself (``workloads.make_inputs``), so no input crosses a pipe, and
hands back the oracle's outputs for the heads it is given.  One BLAS thread per worker.

Every comparison is summarised in one JSON line appended to
``gpurun_out/parity/summary.jsonl`` (under the repository root, or ``$FA_PARITY_DIR``):
max |dO|, max |dLSE|, relative L2 of O and of each gradient, how many elements exceed the
fixed tolerance, how many of those are representation-limited (within one step of the
output type of the correctly rounded oracle value), and, over the elements with
|O_oracle| >= 1/16, how many steps of the output type separate the GPU's value from the
correctly rounded oracle value (0, 1, 2, more).
"""
from __future__ import annotations

import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_G = {}


def _init(name, with_grad):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import workloads as W
    w = W.BY_NAME[name]
    inp = W.make_inputs(w, with_grad=with_grad)
    _G.update(w=w, inp=inp, with_grad=with_grad)


def _ref_head(bh):
    import oracle
    b, h = bh
    w, inp = _G["w"], _G["inp"]
    q, k, v = inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h]
    o, lse = oracle.attention_forward(q, k, v, w.softmax_scale, w.causal, w.window)
    out = [o.astype(np.float64), lse]
    if _G["with_grad"]:
        out += list(oracle.attention_backward(q, k, v, inp["do64"][b, h], w.softmax_scale,
                                              w.causal, w.window))
    return b, h, out


def _init_fp8(name):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import workloads as W
    w = W.BY_NAME[name]
    _G.update(w=w, inp=W.fp8_attention_case(w.shape, w.seed))


def _ref_head_fp8(bh):
    """The FP8 oracle of one head, plus what the kernel's rounding bound needs: the output
    with |V| (W = sum_j P_ij |V_jc|), the plain sum of |V_jc| over the visible keys, and the
    per-row bound e_i of the score error."""
    import oracle
    b, h = bh
    w, c = _G["w"], _G["inp"]
    args = (w.softmax_scale, c["q_descale"], c["k_descale"], c["v_descale"], w.causal, w.window)
    q8, k8, v8 = c["q8"][b, h], c["k8"][b, h], c["v8"][b, h]
    o, lse = oracle.fp8_forward(q8, k8, v8, *args)
    wabs, _ = oracle.fp8_forward(q8, k8, v8 & 0x7F, *args)
    vis = oracle.allowed_mask(w.N, w.causal, w.window)
    s1 = vis.astype(np.float64) @ (c["v_descale"] * np.abs(oracle.e4m3_value(v8)))
    # bound on the score error of the FP8 product's accumulation (see tests/test_fp8_fwd_gpu.py)
    aq, ak = np.abs(oracle.e4m3_value(q8)), np.abs(oracle.e4m3_value(k8))
    e_s = 2.0 ** -11 * abs(w.softmax_scale) * c["q_descale"] * c["k_descale"] * np.where(
        vis, aq @ ak.T, 0.0).max(axis=1)
    return b, h, [o, lse, wabs, s1, e_s]


def oracle_heads_fp8(w, heads, workers=None, progress=None):
    """Yield (b, h, [O, LSE, W, S1, e]) of ``_ref_head_fp8`` for the listed heads, in any order."""
    workers = workers or workers_for(len(heads))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_init_fp8, initargs=(w.name,)) as pool:
        for i, res in enumerate(pool.imap_unordered(_ref_head_fp8, heads, chunksize=1)):
            if progress and (i + 1) % 16 == 0:
                progress(f"{w.name}: oracle {i + 1}/{len(heads)} heads")
            yield res


def workers_for(n_heads):
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(16, cores, n_heads))


def oracle_heads(w, heads, with_grad, workers=None, progress=None):
    """Yield (b, h, [O, LSE(, dQ, dK, dV)]) from the oracle for the listed heads, in any order."""
    workers = workers or workers_for(len(heads))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_init, initargs=(w.name, with_grad)) as pool:
        for i, res in enumerate(pool.imap_unordered(_ref_head, heads, chunksize=1)):
            if progress and (i + 1) % 16 == 0:
                progress(f"{w.name}: oracle {i + 1}/{len(heads)} heads")
            yield res


def ulp_steps(got64, ref64, torch_dtype):
    """Steps of the output type between ``got64`` (values of that type) and the correctly
    rounded ``ref64``."""
    import torch
    g = torch.from_numpy(np.ascontiguousarray(got64)).to(torch_dtype).view(torch.int16)
    r = torch.from_numpy(np.ascontiguousarray(ref64)).to(torch_dtype).view(torch.int16)

    def mono(t):
        t = t.to(torch.int32)
        return torch.where(t < 0, -(t & 0x7FFF), t)
    return (mono(g) - mono(r)).abs().numpy()


class Tally:
    """Running totals of one workload's comparison."""

    def __init__(self, name, o_tol, torch_dtype):
        self.name, self.o_tol, self.dt = name, o_tol, torch_dtype
        self.heads = 0
        self.max_do = self.max_dlse = 0.0
        self.over_tol = 0
        self.repr_limited = 0       # over the tolerance but within one step of the rounded oracle
        self.steps_hist = [0, 0, 0, 0]   # |O_oracle| >= 1/16: 0, 1, 2, > 2 steps from it
        self.o_err2 = self.o_ref2 = 0.0
        self.g_err2 = [0.0, 0.0, 0.0]
        self.g_ref2 = [0.0, 0.0, 0.0]
        self.t0 = time.perf_counter()

    def add_forward(self, o_gpu, lse_gpu, o_ref, lse_ref):
        self.heads += 1
        d = np.abs(o_gpu - o_ref)
        self.max_do = max(self.max_do, float(d.max()))
        self.max_dlse = max(self.max_dlse, float(np.abs(lse_gpu - lse_ref).max()))
        over = d > self.o_tol
        self.over_tol += int(over.sum())
        # steps of the output type only mean something away from zero (the type's exponent
        # range puts thousands of steps between 0 and a value of 1e-7)
        big = np.abs(o_ref) >= 1.0 / 16
        steps = ulp_steps(o_gpu, o_ref, self.dt)
        self.repr_limited += int((over & (steps <= 1)).sum())
        sb = steps[big]
        for i, n in enumerate((int((sb == 0).sum()), int((sb == 1).sum()), int((sb == 2).sum()),
                               int((sb > 2).sum()))):
            self.steps_hist[i] += n
        self.o_err2 += float((d * d).sum())
        self.o_ref2 += float((o_ref * o_ref).sum())

    def add_grads(self, got, ref):
        for t in range(3):
            e = got[t] - ref[t]
            self.g_err2[t] += float((e * e).sum())
            self.g_ref2[t] += float((ref[t] * ref[t]).sum())

    def grad_rel_l2(self):
        return [float(np.sqrt(self.g_err2[t] / max(self.g_ref2[t], 1e-300))) for t in range(3)]

    def record(self, extra=None):
        rec = {"workload": self.name, "heads": self.heads, "max_abs_dO": self.max_do,
               "max_abs_dLSE": self.max_dlse, "rel_l2_O": float(np.sqrt(self.o_err2 / self.o_ref2)),
               "o_tol": self.o_tol, "elements_over_tol": self.over_tol,
               "elements_representation_limited": self.repr_limited,
               "steps_from_rounded_oracle_0_1_2_more": self.steps_hist,
               "seconds": round(time.perf_counter() - self.t0, 1)}
        if any(self.g_ref2):
            rq, rk, rv = self.grad_rel_l2()
            rec.update(rel_l2_dQ=rq, rel_l2_dK=rk, rel_l2_dV=rv)
        if extra:
            rec.update(extra)
        out_dir = os.environ.get("FA_PARITY_DIR", os.path.join(ROOT, "gpurun_out", "parity"))
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, "summary.jsonl"), "a", encoding="utf-8") as f:
            f.write(json.dumps(rec, sort_keys=True) + "\n")
        return rec
