#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the whole path over one batch of synthetic input: the fused
forward (fa_fwd) followed by the recomputing backward (dQ with the row statistics, then dK/dV).
The default workload is B=8, H=16, N=4096, d=64, causal, bf16, with Q, K, V, dO drawn
N(0, 1) from a fixed seed.  Inputs are resident in device memory before timing starts.

Prints ONE JSON line:
  value         whole-step TFLOP/s: algorithmic FLOPs (4 d per visible (query, key) pair
                forward, 10 d backward, per (batch, head)) over the wall time of K steps
                bracketed by device synchronisation
  kernels       per kernel: mean, median and minimum duration over the K timed steps (HIP
                events on the launch stream, caches warm from the previous step), and the
                mean and median of a second pass of K steps each preceded by a write of
                --flush-mib MiB that evicts L2 and the infinity cache ("cold")
  roofline      the kernel with the largest share of the step: its algorithmic FLOPs per
                launch over its average duration (HIP events on the launch stream)
                against the published dense bf16/fp16 MFMA peak of 2516.6 TFLOP/s
  cpu_baseline  the float64 CPU oracle, timed on a bounded sample of the same workload
                (a subset of the (batch, head) slices), on this host's cores
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402

PEAK_TFLOPS = 2516.6        # MI355X dense bf16 / fp16 MFMA, published
PEAK_FP8_TFLOPS = 2 * PEAK_TFLOPS   # dense FP8 MFMA, published as twice the 16-bit rate
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ("cdna4.h", "fwd.hip", "fwd_main.hip", "fwd_split.hip", "bwd.hip", "bwd_dkdv.hip", "bwd_dq.hip",
                  "fwd_fp8.hip", "api.cpp", "launch.h")
# sources a workload's counters depend on, by workload kind (decode: the few-query kernels)
DECODE_SOURCES = ("cdna4.h", "fwd_kv.hip", "api.cpp", "launch.h")
# rocprofv3 kernel names -> the bench's kernel keys
KERNEL_KEYS = (("fwd_main_kernel", "fwd"), ("fwd_fp8_kernel", "fwd"), ("fwd_split_kernel", "fwd"),
               ("fwd_kernel", "fwd"),
               ("delta_kernel", "delta"),
               ("dkdv_main_kernel", "dkdv"), ("dq_main_kernel", "dq"),
               ("dkdv_kernel", "dkdv"), ("dq_kernel", "dq"), ("decode_kernel", "decode"),
               ("combine_kernel", "combine"))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="bytes written before each step of the cold pass (0: no cold pass)")
    ap.add_argument("--workload", default=W.TRAIN.name, choices=sorted(W.BY_NAME))
    ap.add_argument("--forward-only", action="store_true",
                    help="time the forward kernel alone (default: forward + backward)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--alibi", action="store_true",
                    help="decode and block workloads: ALiBi slopes 2^(-8 h / H), h = 1 .. H")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="decode workloads: keys and values as FP8 E4M3 codes (fa_fwd_kv_fp8)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="block workload: attention dropout probability (seed 1234)")
    ap.add_argument("--key-padding", type=float, default=0.0,
                    help="block workload: a key padding mask, each key padding with this "
                         "probability (holes anywhere)")
    ap.add_argument("--block-density", type=float, default=0.0,
                    help="block workload: a seeded block-sparse mask selecting about this "
                         "fraction of the 64 x 64 blocks (0: no mask)")
    ap.add_argument("--cpu-sample-heads", type=int, default=0,
                    help="(batch, head) slices the oracle times (default: all of them)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before warm-up, copy a buffer of this many MiB device to device three "
                         "times (a plain copy kernel of known traffic, for HBM counter scaling)")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="summarise a rocprofv3 --kernel-trace run of this bench made with the same "
                         "--workload, --steps, --warmup and --forward-only (and --flush-mib 0): "
                         "per-kernel durations of the timed dispatches, the warm-up ones apart; "
                         "updates profiles/kernel_times.json")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "bench made with --copy-calibration-mib; writes profiles/hbm_traffic.json")
    return ap.parse_args()


def allowed_pairs(n, causal, window):
    """Visible (query, key) pairs of one head: closed forms of the mask's row counts."""
    wl, wr = window
    total = 0
    # row i sees keys max(0, i - wl) .. min(n - 1, i + wr') with wr' = 0 if causal
    right = 0 if causal else wr
    for i in range(n):
        lo = max(0, i - wl) if wl >= 0 else 0
        hi = min(n - 1, i + right) if right >= 0 else n - 1
        total += max(0, hi - lo + 1)
    return total


def seqlens_of(w):
    """Per-sample lengths of a padded workload (None for a plain one)."""
    return [int(x) for x in W.draw_seqlens(w.B, w.N, w.seed)] if getattr(w, "padded", False) else None


def total_pairs(w):
    """Visible (query, key) pairs of the whole batch: every head of sample b over its own
    length in a padded batch."""
    lens = seqlens_of(w)
    if lens is None:
        return w.B * w.H * allowed_pairs(w.N, w.causal, w.window)
    return w.H * sum(allowed_pairs(L, w.causal, w.window) for L in lens)


def flops(w, pairs_total):
    fwd = 4.0 * w.d * pairs_total
    return {"fwd": fwd, "bwd": 10.0 * w.d * pairs_total,
            # algorithmic share of each backward kernel: dK/dV does 4 of the 5 products,
            # dQ does 1 (its 2 recomputed products are not counted)
            "dkdv": 8.0 * w.d * pairs_total, "dq": 2.0 * w.d * pairs_total}


def source_digest(names=KERNEL_SOURCES):
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "exact_attention_125_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        rec = json.load(f)
    ent = rec.get(f"{workload}/{kernel}")
    names = DECODE_SOURCES if workload.startswith("decode_") else KERNEL_SOURCES
    if not ent or ent.get("source_digest") != source_digest(names):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, sample_heads):
    """Time the oracle on the workload's (batch, head) slices, all of them by default
    (before any GPU use)."""
    from oracle import pool
    inp = W.make_inputs(w)
    arrays = {"q": inp["q64"], "k": inp["k64"], "v": inp["v64"]}
    if w.backward:
        arrays["do"] = inp["do64"]
    cores = pool.available_cores()
    n_heads = min(sample_heads or w.B * w.H, w.B * w.H)
    heads = [(i // w.H, i % w.H) for i in range(n_heads)]
    lens = seqlens_of(w)
    if lens is not None:   # empty samples have no work: leave them out of the sample
        heads = [(b, h) for b, h in heads if lens[b] > 0]
    _, secs, used = pool.run_heads(arrays, heads, w.softmax_scale, w.causal, w.window,
                                   backward=w.backward, workers=cores, keep=False,
                                   lengths=lens)
    per_pair = (4.0 + (10.0 if w.backward else 0.0)) * w.d
    work = sum(per_pair * allowed_pairs(lens[b] if lens else w.N, w.causal, w.window)
               for b, _ in heads)
    return {"value": round(work / secs / 1e12, 6), "unit": "TFLOP/s",
            "cores": used, "kind": "oracle",
            "sample": f"{len(heads)} of {w.B * w.H} (batch, head) slices of {w.name}, "
                      f"{'forward+backward' if w.backward else 'forward'}, float64 numpy "
                      f"materialising S and P, "
                      f"{secs:.2f} s wall, one process and one BLAS thread ({pool.blas_info()}) "
                      f"per core"}


def kernel_key(name):
    for pat, key in KERNEL_KEYS:
        if pat in name:
            return key
    return None


def pmc_summary(fetch_dir, write_dir, workload, calib_mib):
    """Mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel from two rocprofv3 --pmc
    runs, scaled by what the same counters read for the plain copy kernel of known size."""
    import csv
    import glob

    def read(d, counter):
        per = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] != counter:
                        continue
                    name = r["Kernel_Name"]
                    key = kernel_key(name) or ("copy" if "copy" in name.lower() else None)
                    if key is None:
                        continue
                    per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
                    per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        out = {}
        for k, v in per.items():
            vals = list(v.values())
            if k == "copy":   # the calibration copies only, not small copies of other buffers
                vals = [x for x in vals if x >= 0.5 * max(vals)]
            out[k] = sum(vals) / len(vals)
        return out

    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    expected_kib = calib_mib * 1024.0
    f_fac = expected_kib / fetch["copy"] if fetch.get("copy") else None
    w_fac = expected_kib / write["copy"] if write.get("copy") else None
    out = {}
    for key in sorted(set(fetch) | set(write)):
        if key == "copy":
            continue
        fk, wk = fetch.get(key), write.get(key)
        ent = {"fetch_kib_raw": fk, "write_kib_raw": wk, "fetch_scale": f_fac, "write_scale": w_fac,
               "copy_fetch_kib_raw": fetch.get("copy"), "copy_write_kib_raw": write.get("copy"),
               "copy_mib": calib_mib,
               "source_digest": source_digest(DECODE_SOURCES if workload.startswith("decode_")
                                              else KERNEL_SOURCES)}
        if fk is not None and wk is not None and f_fac and w_fac:
            ent["bytes_per_launch"] = round((fk * f_fac + wk * w_fac) * 1024.0)
        out[f"{workload}/{key}"] = ent
    return out


def pass_name(w, forward_only):
    return "fwd+bwd" if (getattr(w, "backward", False) and not forward_only) else "fwd"


def trace_summary(trace_dir, w, args):
    """Per-kernel durations from a rocprofv3 kernel trace of this bench: dispatches of each kernel
    in launch order, the first --warmup of them (the warm-up steps) reported apart, the next
    --steps averaged; later ones (a cold pass) ignored."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                key = kernel_key(r["Kernel_Name"])
                if key is None:
                    continue
                per.setdefault(key, []).append((int(r["Dispatch_Id"]),
                                                int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for key, rows in per.items():
        rows.sort()
        ns = [d for _, d in rows]
        warm, timed = ns[:args.warmup], ns[args.warmup:args.warmup + args.steps]
        if not timed:
            continue
        out[key] = {"dispatches_timed": len(timed), "avg_us": sum(timed) / len(timed) / 1e3,
                    "median_us": statistics.median(timed) / 1e3, "min_us": min(timed) / 1e3,
                    "max_us": max(timed) / 1e3,
                    "warmup_dispatches": len(warm),
                    "warmup_avg_us": (sum(warm) / len(warm) / 1e3) if warm else None,
                    "source_digest": source_digest()}
    return out


def profile_time(kernel, workload, pass_):
    """Average duration (us) of the kernel's timed dispatches from the committed rocprofv3 trace
    summary of this workload and pass, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        ent = json.load(f).get(f"{workload}/{pass_}/{kernel}")
    if not ent or ent.get("source_digest") != source_digest():
        return None
    return ent["avg_us"]


def main():
    args = parse()
    if args.trace_summary:
        w = W.BY_NAME[args.workload]
        pass_ = pass_name(w, args.forward_only)
        res = trace_summary(args.trace_summary, w, args)
        path = os.path.join(ROOT, "profiles", "kernel_times.json")
        rec = {}
        if os.path.exists(path):
            with open(path, encoding="utf-8") as f:
                rec = json.load(f)
        for key, ent in res.items():
            rec[f"{w.name}/{pass_}/{key}"] = ent
        with open(path, "w", encoding="utf-8") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
        pairs = total_pairs(w)
        fl = flops(w, pairs)
        peak = PEAK_FP8_TFLOPS if isinstance(w, W.Fp8Workload) else PEAK_TFLOPS
        print(f"| kernel | timed dispatches | average us | median us | min us | max us | "
              f"warm-up average us | TFLOP/s (average) | % of {peak} |")
        print("|---|---|---|---|---|---|---|---|---|")
        for key in sorted(res, key=lambda k: -res[k]["avg_us"]):
            e = res[key]
            kf = {"fwd": fl["fwd"], "dkdv": fl["dkdv"], "dq": fl["dq"]}.get(key)
            tf = kf / (e["avg_us"] * 1e-6) / 1e12 if kf else None
            warm = f"{e['warmup_avg_us']:.1f}" if e["warmup_avg_us"] is not None else "-"
            print(f"| {key} | {e['dispatches_timed']} | {e['avg_us']:.1f} | {e['median_us']:.1f} | "
                  f"{e['min_us']:.1f} | {e['max_us']:.1f} | {warm} | "
                  + (f"{tf:.1f} | {100 * tf / peak:.1f}% |" if tf else "- | - |"))
        return
    if args.pmc_summary:
        w = W.BY_NAME[args.workload]
        path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
        rec = {}
        if os.path.exists(path):
            with open(path, encoding="utf-8") as f:
                rec = json.load(f)
        name = variant_name(w, args)
        rec.update(pmc_summary(args.pmc_summary[0], args.pmc_summary[1], name,
                               args.copy_calibration_mib or 256))
        with open(path, "w", encoding="utf-8") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
        print(json.dumps({k: v for k, v in rec.items() if k.startswith(name + "/")}, indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the attention path needs no collectives and runs per GPU.",
              file=sys.stderr)
        sys.exit(2)
    w = W.BY_NAME[args.workload]
    if isinstance(w, W.DecodeWorkload):
        return bench_decode(args, w)
    if isinstance(w, W.BlockWorkload):
        return bench_block(args, w)
    if isinstance(w, W.Fp8Workload):
        return bench_fp8(args, w)
    backward = w.backward and not args.forward_only

    # CPU baseline first: the oracle's process pool forks before this process touches the GPU.
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w if backward else W.Workload(**{**w.__dict__, "backward": False}),
                           args.cpu_sample_heads)
        print(f"[bench] cpu baseline: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} cores",
              file=sys.stderr, flush=True)

    import torch
    import exact_attention_125_amd as fa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    inp = W.make_inputs(w, with_grad=backward)
    q, k, v = (inp[n].to("cuda") for n in "qkv")
    do = inp["do"].to("cuda") if backward else None
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, device="cuda", dtype=torch.float32)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(max(fa.bwd_workspace_size(w.B, w.H, w.N, w.d), 16), device="cuda",
                     dtype=torch.uint8)
    scale, causal, window = w.softmax_scale, w.causal, w.window
    lens = seqlens_of(w)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda") if lens is not None else None
    packed = getattr(w, "packed", False)
    if packed:   # the sequences' rows concatenated per head: [H, total, d], offsets cu
        cu = torch.tensor([0] + [int(x) for x in np.cumsum(lens)], dtype=torch.int32,
                          device="cuda")

        def pack(x):
            return torch.cat([x[b, :, :L] for b, L in enumerate(lens)], dim=1).contiguous()
        q, k, v = pack(q), pack(k), pack(v)
        do = pack(do) if do is not None else None
        o = torch.empty_like(q)
        lse = torch.empty(w.H, q.shape[1], device="cuda", dtype=torch.float32)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    # the backward as fa_bwd runs it: the statistics with dQ (one kernel on the main path), then
    # dK/dV
    stages = [("fwd", None)] + ([("dq", fa._lib.BWD_DELTA | fa._lib.BWD_DQ),
                                 ("dkdv", fa._lib.BWD_DKDV)] if backward else [])

    # events: one per stage boundary (len(stages) + 1), so that stage i spans events i .. i + 1
    def step(events=None):
        if events is not None:
            events[0].record()
        for idx, (name, st) in enumerate(stages):
            if packed and st is None:
                fa.fwd_packed(q, k, v, cu, w.N, scale, causal, window, out=o, lse=lse)
            elif packed:
                fa.bwd_packed(do, q, k, v, o, lse, cu, w.N, scale, causal, window, dq=dq, dk=dk,
                              dv=dv, workspace=ws, stages=st)
            elif st is None:
                fa.fwd(q, k, v, scale, causal, window, out=o, lse=lse, seqlens=sl)
            else:
                fa.bwd(do, q, k, v, o, lse, scale, causal, window, dq=dq, dk=dk, dv=dv,
                       workspace=ws, stages=st, seqlens=sl)
            if events is not None:
                events[idx + 1].record()

    if args.copy_calibration_mib:
        # contents do not matter: only the bytes moved are counted
        src = torch.empty(args.copy_calibration_mib << 20, device="cuda", dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_step = {name: [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]
                for i, (name, _) in enumerate(stages)}
    kernel_ms = {name: sum(t) / len(t) for name, t in per_step.items()}

    # cold pass (not part of `value`): each step after a write that evicts L2 and the
    # infinity cache, so K, V (and Q, dO) come from HBM again
    cold = None
    if args.flush_mib > 0:
        flush = torch.empty(args.flush_mib << 20, device="cuda", dtype=torch.uint8)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
               for _ in range(args.steps)]
        for s in range(args.steps):
            flush.fill_(s & 0xFF)
            step(cev[s])
        torch.cuda.synchronize()
        cold = {name: [cev[s][i].elapsed_time(cev[s][i + 1]) for s in range(args.steps)]
                for i, (name, _) in enumerate(stages)}
        del flush
    pairs = total_pairs(w)
    fl = flops(w, pairs)
    step_flops = fl["fwd"] + (fl["bwd"] if backward else 0.0)
    ms = wall / args.steps * 1e3
    value = step_flops / (ms * 1e-3) / 1e12
    nominal = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)

    kernels = {}
    for name, t in kernel_ms.items():
        kf = {"fwd": fl["fwd"], "dkdv": fl["dkdv"], "dq": fl["dq"]}.get(name)
        entry = {"ms": round(t, 4), "median_ms": round(statistics.median(per_step[name]), 4),
                 "min_ms": round(min(per_step[name]), 4)}
        if cold is not None:
            entry["cold_ms"] = round(sum(cold[name]) / len(cold[name]), 4)
            entry["cold_median_ms"] = round(statistics.median(cold[name]), 4)
        if kf is not None:
            entry["tflops"] = round(kf / (t * 1e-3) / 1e12, 2)
            entry["frac"] = round(entry["tflops"] / PEAK_TFLOPS, 4)
            if cold is not None:
                entry["cold_tflops"] = round(kf / (entry["cold_ms"] * 1e-3) / 1e12, 2)
        else:   # delta: bandwidth kernel, reads O and dO (the samples' rows), writes fp32 delta
            rows = w.H * (sum(lens) if lens is not None else w.B * w.N)
            nbytes = 2 * rows * w.d * 2 + w.B * w.H * w.N * 4
            entry["gbs"] = round(nbytes / (t * 1e-3) / 1e9, 1)
        kernels[name] = entry
    dominant = max((n for n in kernel_ms if n != "delta"), key=lambda n: kernel_ms[n])
    dom_flops = {"fwd": fl["fwd"], "dkdv": fl["dkdv"], "dq": fl["dq"]}[dominant]
    achieved = dom_flops / (kernel_ms[dominant] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 2),
                "peak": PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                "traffic": measured_traffic(dominant, w.name)}
    # the same figure from the committed rocprofv3 trace of this workload (null when that trace
    # was taken on other kernel sources)
    prof_us = profile_time(dominant, w.name, "fwd+bwd" if backward else "fwd")
    if prof_us:
        pa = dom_flops / (prof_us * 1e-6) / 1e12
        roofline.update(profile_avg_us=round(prof_us, 2), profile_achieved=round(pa, 2),
                        profile_frac=round(pa / PEAK_TFLOPS, 4))
    else:
        roofline.update(profile_avg_us=None, profile_achieved=None, profile_frac=None)

    out = {
        "metric": "attention fwd+bwd TFLOP/s on 1 MI355X (fraction of dense bf16 MFMA peak in "
                  "roofline)" if backward else "attention fwd TFLOP/s on 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) Q, K, V, dO" +
                                  (", sample lengths uniform in [N/4, N]" if lens else "") +
                                  (", packed per head)" if packed else ")"),
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len": w.N,
                   "head_dim": w.d, "causal": w.causal, "window": list(w.window),
                   "pass": "fwd+bwd" if backward else "fwd",
                   "visible_pairs_per_head": pairs // (w.B * w.H),
                   **({"seqlens": lens, "visible_pairs": pairs} if lens is not None else {}),
                   "flops_per_step": step_flops,
                   "nominal_flops_per_step": nominal * (3.5 if backward else 1.0)},
        "kernels": kernels,
        "fwd_tflops": kernels["fwd"]["tflops"], "fwd_frac_of_peak": kernels["fwd"]["frac"],
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def alibi_slopes(H):
    """The geometric ALiBi slopes 2^(-8 h / H), h = 1 .. H, as a float32 device tensor."""
    import torch
    return torch.tensor([2.0 ** (-8.0 * h / H) for h in range(1, H + 1)], dtype=torch.float32,
                        device="cuda")


def decode_bytes(w, kv_bytes=2):
    """Algorithmic HBM bytes of one decode call: Q, K, V read once, O and LSE written once
    (kv_bytes per key / value element: 2, or 1 for an FP8 cache)."""
    e = 2
    return w.B * w.H * (2 * w.n_k * w.d * kv_bytes + 2 * w.n_q * w.d * e + w.n_q * 4)


def decode_cpu_baseline(w, inp):
    """The oracle over every (batch, head) of the decode workload, one process."""
    import oracle
    from oracle import pool
    fp8 = "k8" in inp
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            if fp8:
                oracle.fp8_cache_forward(inp["q64"][b, h], inp["k8"][b, h], inp["v8"][b, h],
                                         w.softmax_scale, inp["k_descale"], inp["v_descale"],
                                         True)
            else:
                oracle.cross_forward(inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h],
                                     w.softmax_scale, True)
    secs = time.perf_counter() - t0
    return {"value": round(decode_bytes(w, 1 if fp8 else 2) / secs / 1e9, 3), "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"all {w.B * w.H} (batch, head) slices of {w.name}, float64 numpy "
                      f"materialising S and P, {secs:.2f} s wall, one process "
                      f"({pool.blas_info()})"}


def bench_decode(args, w):
    """One decode step per timed step: fa_fwd_kv with n_q new queries over the n_k-key cache,
    HBM-bound; `value` is algorithmic bytes over wall time."""
    fp8 = bool(args.kv_fp8)
    if fp8 and args.alibi:
        raise SystemExit("--kv-fp8 takes no --alibi (the FP8 cache entry point has no ALiBi)")
    inp = (W.fp8_cache_case(w.B, w.H, w.n_q, w.n_k, w.d, w.dtype, w.seed) if fp8
           else W.cross_case(w.B, w.H, w.n_q, w.n_k, w.d, w.dtype, w.seed))
    cpu = None if args.no_cpu_baseline else decode_cpu_baseline(w, inp)
    import torch
    import exact_attention_125_amd as fa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if fp8:
        q = inp["q"].to("cuda")
        k, v = (torch.from_numpy(inp[n]).to("cuda") for n in ("k8", "v8"))
    else:
        q, k, v = (inp[n].to("cuda") for n in "qkv")
    o = torch.empty_like(q)
    need = fa.fwd_kv_workspace_size(w.B, w.H, w.n_q, w.n_k, w.d)
    ws = torch.empty(max(need, 16), device="cuda", dtype=torch.uint8)
    slopes = alibi_slopes(w.H) if args.alibi else None

    def call():
        if fp8:
            fa._lib.fwd_kv_fp8(q, k, v, inp["k_descale"], inp["v_descale"], w.softmax_scale,
                               True, out=o, workspace=ws)
        else:
            fa._lib.fwd_kv(q, k, v, w.softmax_scale, True, out=o, workspace=ws,
                           alibi_slopes=slopes)

    if args.copy_calibration_mib:
        src = torch.empty(args.copy_calibration_mib << 20, device="cuda", dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = [a.elapsed_time(b) for a, b in ev]
    cold = None
    if args.flush_mib > 0:
        flush = torch.empty(args.flush_mib << 20, device="cuda", dtype=torch.uint8)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i, (a, b) in enumerate(cev):
            flush.fill_(i & 0xFF)
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        cold = [a.elapsed_time(b) for a, b in cev]
        del flush
    nbytes = decode_bytes(w, 1 if fp8 else 2)
    ms = wall / args.steps * 1e3
    t_mean = sum(times) / len(times)
    gbs = nbytes / (t_mean * 1e-3) / 1e9
    pairs = w.B * w.H * w.n_q * w.n_k
    entry = {"ms": round(t_mean, 4), "median_ms": round(statistics.median(times), 4),
             "min_ms": round(min(times), 4), "gbs": round(gbs, 1),
             "tflops": round(4.0 * w.d * pairs / (t_mean * 1e-3) / 1e12, 3)}
    if cold is not None:
        entry["cold_ms"] = round(sum(cold) / len(cold), 4)
        entry["cold_median_ms"] = round(statistics.median(cold), 4)
        entry["cold_gbs"] = round(nbytes / (entry["cold_ms"] * 1e-3) / 1e9, 1)
    # key splits of the 16-bit plan, from its workspace (one partial O and LSE per split); the
    # FP8 cache's plan, with twice the rows per step, can have fewer, which the library does
    # not report
    plan_splits = (need // (w.B * w.H * w.n_q * (w.d + 1) * 4) if need else 1) if not fp8 else None
    out = {
        "metric": "attention decode forward HBM GB/s on 1 MI355X (algorithmic bytes: Q, K, V "
                  "read once, O and LSE written once)",
        "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"fp8_e4m3 k/v, {w.dtype} q/o" if fp8 else w.dtype,
        "data": ("synthetic (seeded N(0,1) Q; K, V as E4M3 codes of N(0,1) * 16, descale 1/16)"
                 if fp8 else "synthetic (seeded N(0,1) Q, K, V)"),
        "config": {"workload": w.name + ("_kvfp8" if fp8 else ""), "kv_fp8": fp8, "batch": w.B, "heads": w.H, "n_q": w.n_q, "n_k": w.n_k,
                   "head_dim": w.d, "causal": True, "pass": "fwd", "alibi": bool(args.alibi),
                   "bytes_per_step": nbytes, "key_splits": plan_splits},
        "kernels": {"decode+combine": entry},
        # the call is the decode kernel and the split merge; timing both together
        # understates the decode kernel's own rate slightly
        "roofline": {"bound": "hbm", "kernel": "decode_kernel (+ combine_kernel)",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("decode", variant_name(w, args))},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_fp8(args, w):
    """The forward over FP8 E4M3 queries, keys and values (fa_fwd_fp8): one launch per timed
    step, TFLOP/s over the visible pairs against the dense FP8 MFMA peak."""
    import oracle
    case = W.fp8_attention_case(w.shape, w.seed)
    desc = (case["q_descale"], case["k_descale"], case["v_descale"])
    pairs = w.B * w.H * allowed_pairs(w.N, w.causal, w.window)
    fl = 4.0 * w.d * pairs
    cpu = None
    if not args.no_cpu_baseline:   # the oracle on a bounded sample: the first heads' slices
        from oracle import pool
        n = args.cpu_sample_heads or 4
        t0 = time.perf_counter()
        for i in range(n):
            b, h = divmod(i, w.H)
            oracle.fp8_forward(case["q8"][b, h], case["k8"][b, h], case["v8"][b, h],
                               w.softmax_scale, *desc, w.causal, w.window)
        secs = time.perf_counter() - t0
        cpu = {"value": round(n * fl / (w.B * w.H) / secs / 1e12, 6), "unit": "TFLOP/s",
               "cores": 1, "kind": "oracle",
               "sample": f"{n} of {w.B * w.H} (batch, head) slices of {w.name}, forward, float64 "
                         f"numpy over the decoded values materialising S and P, {secs:.2f} s "
                         f"wall, one process ({pool.blas_info()})"}
    import torch
    import exact_attention_125_amd as fa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    q, k, v = (torch.from_numpy(case[n + "8"]).to("cuda") for n in "qkv")
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[w.out_dtype]
    o = torch.empty(w.shape, device="cuda", dtype=dt)
    lse = torch.empty(w.B, w.H, w.N, device="cuda", dtype=torch.float32)

    def call():
        fa.fwd_fp8(q, k, v, *desc, w.softmax_scale, w.causal, w.window, out=o)

    if args.copy_calibration_mib:
        src = torch.empty(args.copy_calibration_mib << 20, device="cuda", dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a_, b_ in ev:
        a_.record()
        call()
        b_.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = [a_.elapsed_time(b_) for a_, b_ in ev]
    ms = wall / args.steps * 1e3
    t_mean = sum(times) / len(times)
    ach = fl / (t_mean * 1e-3) / 1e12
    entry = {"ms": round(t_mean, 4), "median_ms": round(statistics.median(times), 4),
             "min_ms": round(min(times), 4), "tflops": round(ach, 2),
             "frac_fp8_peak": round(ach / PEAK_FP8_TFLOPS, 4),
             "frac_bf16_peak": round(ach / PEAK_TFLOPS, 4)}
    roofline = {"bound": "mfma", "kernel": "fwd", "achieved": round(ach, 2),
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": measured_traffic("fwd", w.name)}
    prof_us = profile_time("fwd", w.name, "fwd")
    if prof_us:
        pa = fl / (prof_us * 1e-6) / 1e12
        roofline.update(profile_avg_us=round(prof_us, 2), profile_achieved=round(pa, 2),
                        profile_frac=round(pa / PEAK_FP8_TFLOPS, 4))
    else:
        roofline.update(profile_avg_us=None, profile_achieved=None, profile_frac=None)
    out = {
        "metric": "attention fwd TFLOP/s on 1 MI355X, FP8 E4M3 Q, K, V (fraction of the dense "
                  "FP8 MFMA peak in roofline)",
        "value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"fp8_e4m3 q/k/v, {w.out_dtype} o",
        "data": "synthetic (seeded N(0,1) * 16 as E4M3 codes, descale 1/16 per tensor)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len": w.N,
                   "head_dim": w.d, "causal": w.causal, "window": list(w.window), "pass": "fwd",
                   "visible_pairs_per_head": pairs // (w.B * w.H), "flops_per_step": fl},
        "kernels": {"fwd": entry},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def variant_name(w, args):
    """The name counter summaries file a workload's traffic under: the workload, and the extras
    that change what its kernels move (an FP8 cache, ALiBi, dropout, a block mask)."""
    name = w.name + ("_kvfp8" if getattr(args, "kv_fp8", False) else "")
    if getattr(args, "alibi", False):
        name += "_alibi"
    if getattr(args, "dropout", 0.0):
        name += f"_dropout{args.dropout:g}"
    if getattr(args, "block_density", 0.0):
        name += f"_blocks{args.block_density:g}"
    if getattr(args, "key_padding", 0.0):
        name += f"_kpm{args.key_padding:g}"
    return name


def block_traffic(workload, call):
    """HBM bytes of the kernels of one fa_fwd_kv ("fwd_kv") or fa_bwd_kv ("bwd_kv") call of the
    block workload, from the committed counter summary, or None."""
    keys = ("fwd",) if call == "fwd_kv" else ("delta", "dkdv", "dq")
    vals = [measured_traffic(k, workload) for k in keys]
    return None if any(v is None for v in vals) else sum(vals)


def block_workload_pairs(w, blocks=None, kpm=None):
    """Visible (query, key) pairs of the block workload: query i at key position i + n_k - n_q
    sees keys j <= that position (causal); a block mask [H, n_q/64, n_k/64] and a key padding
    mask [B, n_k] (True = padding) hide more."""
    import numpy as np
    off = w.n_k - w.n_q
    vis = np.arange(w.n_k)[None, :] <= (np.arange(w.n_q) + off)[:, None]          # [n_q, n_k]
    per_head = (np.ones(w.H, bool)[:, None, None] & vis[None] if blocks is None else
                vis[None] & np.asarray(blocks, bool)[:, np.arange(w.n_q)[:, None] // 64,
                                                      np.arange(w.n_k)[None, :] // 64])
    if kpm is None:
        return int(w.B * per_head.sum())
    keep = ~np.asarray(kpm, bool)                                                 # [B, n_k]
    # sum over b, h, i, j of per_head[h, i, j] * keep[b, j]
    return int((per_head.sum(axis=1) @ keep.T.astype(np.int64)).sum())


def bench_block(args, w):
    """One training step of a query block over a longer key sequence: fa_fwd_kv then fa_bwd_kv
    (the four-wave kernels), MFMA-bound; `value` is algorithmic TFLOP/s over wall time."""
    import numpy as np
    inp = W.cross_case(w.B, w.H, w.n_q, w.n_k, w.d, w.dtype, w.seed)
    g = W.cross_case(w.B, w.H, w.n_q, 1, w.d, w.dtype, w.seed + 1000)["q"]
    blocks = None
    if args.block_density > 0:
        blocks = W.draw_blocks(w.H, w.n_q, w.n_k, args.block_density, w.seed)
    kpm = None
    if args.key_padding > 0:
        kpm = W.key_padding_case(w.B, w.n_k, w.seed + 7, density=args.key_padding)
    pairs = block_workload_pairs(w, blocks, kpm)
    fwd_flops, bwd_flops = 4.0 * w.d * pairs, 10.0 * w.d * pairs
    cpu = None
    if not args.no_cpu_baseline:   # the oracle on a bounded sample: the first heads' slices
        import oracle
        n = args.cpu_sample_heads or 4
        t0 = time.perf_counter()
        for i in range(n):
            b, h = divmod(i, w.H)
            args_ = (inp["q64"][b, h], inp["k64"][b, h], inp["v64"][b, h])
            bm = None if blocks is None else blocks[h]
            km = None if kpm is None else kpm[b]
            oracle.cross_forward(*args_, w.softmax_scale, True, block_mask=bm, key_mask=km)
            oracle.cross_backward(*args_, g.double().numpy()[b, h], w.softmax_scale, True,
                                  block_mask=bm, key_mask=km)
        secs = time.perf_counter() - t0
        from oracle import pool
        cpu = {"value": round(n * (fwd_flops + bwd_flops) / (w.B * w.H) / secs / 1e12, 6),
               "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} of {w.B * w.H} (batch, head) slices of {w.name}, forward+backward, "
                         f"float64 numpy materialising S and P, {secs:.2f} s wall, one process "
                         f"({pool.blas_info()})"}
    import torch
    import exact_attention_125_amd as fa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    q, k, v, do = (t.to("cuda") for t in (inp["q"], inp["k"], inp["v"], g))
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_f = torch.empty(max(fa.fwd_kv_workspace_size(w.B, w.H, w.n_q, w.n_k, w.d), 16),
                       device="cuda", dtype=torch.uint8)
    ws_b = torch.empty(max(fa.bwd_workspace_size(w.B, w.H, w.n_q, w.d), 16), device="cuda",
                       dtype=torch.uint8)
    slopes = alibi_slopes(w.H) if args.alibi else None
    bmask = None if blocks is None else torch.tensor(blocks.astype(np.uint8), device="cuda")
    kmask = None if kpm is None else torch.tensor(kpm.astype(np.uint8), device="cuda")
    state = {}

    def step(ev=None):
        if ev:
            ev[0].record()
        drop = dict(dropout_p=args.dropout, dropout_seed=1234, block_mask=bmask,
                    key_padding_mask=kmask)
        _, state["lse"] = fa.fwd_kv(q, k, v, w.softmax_scale, True, out=o, workspace=ws_f,
                                    alibi_slopes=slopes, **drop)
        if ev:
            ev[1].record()
        fa.bwd_kv(do, q, k, v, o, state["lse"], w.softmax_scale, True, dq=dq, dk=dk, dv=dv,
                  workspace=ws_b, alibi_slopes=slopes, **drop)
        if ev:
            ev[2].record()

    if args.copy_calibration_mib:
        src = torch.empty(args.copy_calibration_mib << 20, device="cuda", dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = [e[0].elapsed_time(e[1]) for e in evs]
    b_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms = wall / args.steps * 1e3
    fm, bm = sum(f_ms) / len(f_ms), sum(b_ms) / len(b_ms)
    kernels = {"fwd_kv": {"ms": round(fm, 4), "median_ms": round(statistics.median(f_ms), 4),
                          "tflops": round(fwd_flops / (fm * 1e-3) / 1e12, 2)},
               "bwd_kv": {"ms": round(bm, 4), "median_ms": round(statistics.median(b_ms), 4),
                          "tflops": round(bwd_flops / (bm * 1e-3) / 1e12, 2)}}
    dom = "bwd_kv" if bm >= fm else "fwd_kv"
    ach = kernels[dom]["tflops"]
    out = {
        "metric": "attention fwd+bwd TFLOP/s on 1 MI355X, query block over a longer key "
                  "sequence (fa_fwd_kv + fa_bwd_kv)",
        "value": round((fwd_flops + bwd_flops) / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q, K, V, dO)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "n_q": w.n_q, "n_k": w.n_k,
                   "head_dim": w.d, "causal": True, "pass": "fwd+bwd", "alibi": bool(args.alibi),
                   "dropout_p": args.dropout, "block_density": args.block_density,
                   "key_padding": args.key_padding,
                   "visible_pairs": pairs, "flops_per_step": fwd_flops + bwd_flops},
        "kernels": kernels,
        # a call spans several kernels (fwd_kv: one, bwd_kv: delta, dK/dV, dQ), timed together;
        # traffic: the HBM bytes of all kernels of that call
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS, 4),
                     "traffic": block_traffic(variant_name(w, args), dom)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
