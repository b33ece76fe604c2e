#!/usr/bin/env python3
"""Benchmark: Muon optimizer steps/s on the GPT-2-124M hidden matrices, on one MI355X.

One step = one call of the library's muon_step over all 48 hidden matrices of
GPT-2-124M (12 layers x 768x2304, 768x768, 768x3072, 3072x768; 84.9 M fp32
parameters): Nesterov momentum, Frobenius normalisation, 5 bf16 quintic
Newton-Schulz iterations and the parameter update.  Inputs are seeded
synthetic gradients of that shape, resident in HBM before timing starts.

Prints one JSON line.  `roofline` is for the dominant kernel (the Newton-Schulz
update GEMM X <- aX + BX): algorithmic flops per launch / its mean launch time,
timed with HIP events on the launch stream in a pass of the same steps right
after the timed region (the timed region itself carries only one event per
step).
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same
workload (some layers), scaled to steps/s.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
LR, BETA, NS_STEPS = 0.02, 0.95, 5
COEFFS = (3.4445, -4.7750, 2.0315)
WORKLOAD = "c3"


def ns_flops_dense(shapes):
    """Flops of one Newton-Schulz iteration done as three dense GEMMs (no use
    of symmetry): 2 m^2 n + 2 m^3 + 2 m^2 n per matrix."""
    total = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        total += 4 * m * m * n + 2 * m * m * m
    return total


def ns_flops(shapes):
    """Algorithmic flops per launch of each Newton-Schulz GEMM, counting the
    symmetry of X X^T and of A A."""
    gram = poly = upd = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        gram += m * (m + 1) * n
        poly += m * m * (m + 1)
        upd += 2 * m * m * n
    return gram, poly, upd


def traffic_from_profiles():
    """HBM bytes per launch of the update GEMM, from committed rocprofv3 counter
    runs, if they were taken on the current kernel sources and build options."""
    path = os.path.join(ROOT, "profiles", "ns_update_c3_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from optimizer_muon_step_amd.build import update_kernel_fingerprint
    if rec.get("kernel_source_sha256") != update_kernel_fingerprint():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(budget_s):
    """Time the oracle on whole layers of the workload until the budget is used."""
    import numpy as np
    from oracle import muon_oracle as om
    from optimizer_muon_step_amd import workloads as wl
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(int(i.get("num_threads", 1)) for i in info) if info else 1
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:
        cores = os.cpu_count() or 1
    specs = wl.config_specs(WORKLOAD)
    layers = sorted({s.layer for s in specs})
    elapsed, done = 0.0, 0
    for layer in layers:
        idx = [i for i, s in enumerate(specs) if s.layer == layer]
        mats = [wl.make_matrix(WORKLOAD, i, 1) for i in idx]
        t0 = time.perf_counter()
        for m in mats:
            om.muon_step_matrix(m["W"], m["grads"][0], m["buf"], LR, BETA, NS_STEPS, COEFFS)
        elapsed += time.perf_counter() - t0
        done += 1
        if elapsed >= budget_s:
            break
    sec_per_step = elapsed / done * len(layers)
    return {"value": 1.0 / sec_per_step, "unit": "steps/s", "cores": cores, "kind": "oracle", "blas": blas,
            "sample": f"{done} of {len(layers)} layers ({4 * done} of {len(specs)} matrices), one step each, "
                      f"{elapsed:.1f} s, scaled to the full 48-matrix step"}


def bench_adamw(torch, mu, wl, calls=50):
    """The multi-tensor AdamW entry on the GPT-2-124M AdamW set (the
    parameters outside the hidden set), measured after the Muon timed region
    and reported beside it: 28 bytes per element (read p, g, u, v; write p,
    u, v), mean kernel time from HIP events on the launch stream."""
    specs = wl.adamw_specs_gpt2()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.ADAMW_SEED)
    P, G, U, V = [], [], [], []
    for s in specs:
        P.append(torch.randn(s.shape, generator=gen, device="cuda") * 0.02)
        G.append(torch.randn(s.shape, generator=gen, device="cuda") * 1e-3)
        U.append(torch.randn(s.shape, generator=gen, device="cuda") * 1e-3)
        V.append(torch.randn(s.shape, generator=gen, device="cuda").square() * 1e-6)
    wds = [1e-2 if s.decayed else 0.0 for s in specs]
    n = sum(s.numel for s in specs)
    stream = torch.cuda.current_stream()
    for k in range(5):
        mu.muon_adamw_step(P, G, U, V, 6e-4, (0.9, 0.999), 1e-8, wds, step=1000 + k, stream=stream)
    torch.cuda.synchronize()
    mu.muon_timing_enable(mu.KERNEL_ADAMW)
    t0 = time.perf_counter()
    for k in range(calls):
        mu.muon_adamw_step(P, G, U, V, 6e-4, (0.9, 0.999), 1e-8, wds, step=1005 + k, stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms, cnt = mu.muon_timing_read()
    mu.muon_timing_enable(-1)
    per = ms / max(1, cnt)
    gbs = 28.0 * n / (per * 1e-3) / 1e9
    del P, G, U, V
    return {
        "workload": "GPT-2-124M AdamW set: wte 50257x768 and wpe 1024x768 (weight decay 1e-2), 98 1-D LayerNorm "
                    "and bias tensors (no decay); 100 fp32 tensors, 39.5M params, one launch",
        "n_tensors": len(specs), "n_params": n, "lr": 6e-4, "betas": [0.9, 0.999], "eps": 1e-8,
        "bytes_per_param": 28, "ms_per_launch": round(per, 5), "calls_per_s": round(calls / wall, 1),
        "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
    }


def bench_vendor_ns(torch, wl, ns_flops_step, steps=20):
    """The same 5 Newton-Schulz iterations on the same 48 canonical bf16
    matrices done the stock way, with torch bf16 matmuls (hipBLASLt) per
    shape group, for comparison with the library's NS kernels.  Not part of
    the step; every right operand is made contiguous first (no transposed
    views in batched bf16 products)."""
    specs = wl.config_specs(WORKLOAD)
    groups = {}
    for s in specs:
        m, n = min(s.rows, s.cols), max(s.rows, s.cols)
        groups[(m, n)] = groups.get((m, n), 0) + 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    Xs = [(torch.randn((b, m, n), generator=gen, device="cuda") / (m * n) ** 0.5).to(torch.bfloat16)
          for (m, n), b in groups.items()]
    a, b, c = COEFFS

    def ns(X):
        for _ in range(NS_STEPS):
            Xt = X.transpose(1, 2).contiguous()
            A = torch.bmm(X, Xt)
            B = b * A + c * torch.bmm(A, A)
            X = a * X + torch.bmm(B, X)
        return X

    for _ in range(3):
        for X in Xs:
            ns(X)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        for X in Xs:
            ns(X)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"what": "5 NS iterations on the 48 c3 matrices with torch bf16 bmm (hipBLASLt) and torch "
                    "elementwise ops, per shape group; the transposed operand copied contiguous first",
            "ms_per_step": round(ms, 4), "TFLOP/s_algorithmic": round(ns_flops_step / (ms * 1e-3) / 1e12, 1)}


def bench_measured_peaks(torch, reps=20):
    """Measured denominators beside the spec peaks: a large square bf16
    matmul through torch (hipBLASLt) and a plain 1 GiB device-to-device
    copy (bytes read plus bytes written per second)."""
    n = 8192
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    a = torch.randn((n, n), generator=gen, device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), generator=gen, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    src = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * src.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {"bf16_gemm_TFLOP/s": round(gemm_tf, 1), "bf16_gemm_what": "torch.matmul 8192x8192x8192 bf16 (hipBLASLt)",
            "copy_GB/s": round(copy_gbs, 1), "copy_what": "1 GiB device-to-device copy, read + write bytes"}


def family_breakdown(mu, step, shapes, reps=2):
    """Per-kernel-family time of one step (HIP events around each family's
    launches, one family per pass of `reps` steps), and from it the NS
    TFLOP/s (symmetry-aware flops) and the elementwise GB/s (momentum, cast
    and apply: 12 + 10 + 10 bytes per parameter)."""
    fam = {}
    for name, k in (("momentum", mu.KERNEL_MOMENTUM), ("cast", mu.KERNEL_CAST), ("gram", mu.KERNEL_GRAM),
                    ("poly", mu.KERNEL_POLY), ("update", mu.KERNEL_UPDATE), ("apply", mu.KERNEL_APPLY)):
        mu.muon_timing_enable(k)
        for _ in range(reps):
            step()
        t, _ = mu.muon_timing_read()
        mu.muon_timing_enable(-1)
        fam[name] = t / reps
    params = sum(r * c for r, c in shapes)
    ns_ms = fam["gram"] + fam["poly"] + fam["update"]
    ew_ms = fam["momentum"] + fam["cast"] + fam["apply"]
    gram_f, poly_f, upd_f = ns_flops(shapes)
    ns_tf = NS_STEPS * (gram_f + poly_f + upd_f) / (ns_ms * 1e-3) / 1e12
    ew_gbs = 32.0 * params / (ew_ms * 1e-3) / 1e9
    return {"ns_ms_per_step": round(ns_ms, 4), "ns_TFLOP/s": round(ns_tf, 1),
            "ns_frac_bf16_peak": round(ns_tf / PEAK_BF16_TFLOPS, 4),
            "elementwise_ms_per_step": round(ew_ms, 4), "elementwise_GB/s": round(ew_gbs, 1),
            "elementwise_frac_hbm_peak": round(ew_gbs / PEAK_HBM_GBS, 4)}


def bench_small(torch, mu, wl, steps=200):
    """Small workloads, where launch overhead matters: steps/s of eager calls
    and of the same step captured once into a HIP graph and replayed."""
    out = {}
    for name in ("c1", "c2"):
        specs = wl.config_specs(name)
        W = [torch.from_numpy(wl.make_params(name, i, s)).cuda() for i, s in enumerate(specs)]
        G = [torch.from_numpy(wl.make_grad(name, i, s, 1)).cuda() for i, s in enumerate(specs)]
        M = [torch.zeros((s.rows, s.cols), device="cuda") for s in specs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(10):
                mu.muon_step(W, G, M, LR, BETA, NS_STEPS, COEFFS)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                mu.muon_step(W, G, M, LR, BETA, NS_STEPS, COEFFS)
            torch.cuda.synchronize()
            eager = steps / (time.perf_counter() - t0)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            mu.muon_step(W, G, M, LR, BETA, NS_STEPS, COEFFS)
        for _ in range(10):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        replay = steps / (time.perf_counter() - t0)
        out[name] = {"matrices": len(specs), "params": sum(s.rows * s.cols for s in specs),
                     "eager_steps_per_s": round(eager, 1), "graph_replay_steps_per_s": round(replay, 1)}
        out[name].update(family_breakdown(mu, lambda: mu.muon_step(W, G, M, LR, BETA, NS_STEPS, COEFFS),
                                          [(s.rows, s.cols) for s in specs], reps=10))
        del W, G, M, graph
    return out


def bench_large(torch, mu, wl):
    """The other two named workloads, timed like the headline one (HIP
    events around whole steps, then per-kernel events for the NS GEMMs):
    the GPT-2-XL-shaped hidden set (1.47 B params; its inputs are drawn on
    the device with the c4 distribution, since host generation of 3 B
    values would dominate the run) and the stress pair (inputs from the
    seeded generators)."""
    out = {}
    for name, warm, steps in (("c5", 5, 20), ("c4", 2, 5)):
        specs = wl.config_specs(name)
        shapes = [(s.rows, s.cols) for s in specs]
        if name == "c4":
            gen = torch.Generator(device="cuda")
            gen.manual_seed(4000)
            W, G = [], []
            for s in specs:
                W.append(torch.randn((s.rows, s.cols), device="cuda", generator=gen) * 0.02)
                G.append(torch.randn((s.rows, s.cols), device="cuda", generator=gen)
                         * (1e-3 * wl.layer_factor(name, s.layer)))
        else:
            W = [torch.from_numpy(wl.make_params(name, i, s)).cuda() for i, s in enumerate(specs)]
            G = [torch.from_numpy(wl.make_grad(name, i, s, 1)).cuda() for i, s in enumerate(specs)]
        M = [torch.zeros((s.rows, s.cols), device="cuda") for s in specs]
        stream = torch.cuda.current_stream()

        def step():
            mu.muon_step(W, G, M, LR, BETA, NS_STEPS, COEFFS, stream=stream)

        for _ in range(warm):
            step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[name] = {"matrices": len(specs), "params": sum(r * c for r, c in shapes),
                     "steps_per_s": round(1e3 / ms, 2), "ms_per_step": round(ms, 4)}
        out[name].update(family_breakdown(mu, step, shapes))
        del W, G, M
        torch.cuda.synchronize()
        mu.muon_release()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-breakdown", action="store_true",
                    help="skip the per-kernel-family timing pass after the timed region")
    ap.add_argument("--no-adamw", action="store_true", help="skip the AdamW measurement after the timed region")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the torch/hipBLASLt comparisons (Newton-Schulz iterations, measured GEMM and copy peaks)")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the small-workload (eager vs graph replay) measurement after the timed region")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the GPT-2-XL-shaped and stress workloads measured after the timed region")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the step is measured on one GPU; --gpus {args.gpus} is not supported "
              "(sharding whole matrices across ranks is not implemented)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import optimizer_muon_step_amd as mu
    from optimizer_muon_step_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mu._lib.load()
    torch.cuda.set_device(0)
    specs = wl.config_specs(WORKLOAD)
    shapes = [(s.rows, s.cols) for s in specs]
    n_params = sum(r * c for r, c in shapes)
    W, G, M = [], [], []
    for i, s in enumerate(specs):
        W.append(torch.from_numpy(wl.make_params(WORKLOAD, i, s)).cuda())
        G.append(torch.from_numpy(wl.make_grad(WORKLOAD, i, s, 1)).cuda())
        M.append(torch.zeros((s.rows, s.cols), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        mu.muon_step(W, G, M, LR, BETA, NS_STEPS, COEFFS, stream=stream)

    for _ in range(args.warmup):
        step()
    # Per-step HIP events on the launch stream.  torch creates an event's HIP
    # handle on its first record; recording each one here, before the timed
    # region, keeps that creation out of it (a first-time creation inside the
    # region has blocked the host for tens of milliseconds and left the GPU
    # idle for a step).  The region holds nothing but the steps and these
    # events: no library instrumentation, no garbage collection.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for e in evs:
        e.record(stream)
    torch.cuda.synchronize()
    host_t = []
    gc.disable()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for k in range(args.steps):
        step()
        evs[k + 1].record(stream)
        host_t.append(time.perf_counter())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    wall_s = t1 - t0
    ms_per_step = wall_s * 1e3 / args.steps
    ev_ms_per_step = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps)])
    enq_ms = np.diff(np.array([t0] + host_t)) * 1e3

    # The roofline kernel's launch time, in a pass of its own after the
    # timed region: the library brackets every update-GEMM launch with HIP
    # events on the launch stream.  A first pass creates the library's
    # events; the second is read.
    roof_steps = max(args.steps, 20)
    for rep in range(2):
        mu.muon_timing_enable(mu.KERNEL_UPDATE)
        for _ in range(roof_steps):
            step()
        upd_ms_total, upd_launches = mu.muon_timing_read()
        mu.muon_timing_enable(-1)
    torch.cuda.synchronize()

    gram_f, poly_f, upd_f = ns_flops(shapes)
    ns_flops_step = NS_STEPS * (gram_f + poly_f + upd_f)
    upd_ms = upd_ms_total / max(1, upd_launches)
    upd_tflops = upd_f / (upd_ms * 1e-3) / 1e12

    breakdown = None
    if not args.no_kernel_breakdown:
        names = ["momentum", "cast", "gram", "poly", "update", "apply"]
        per_launch_work = [12 * n_params, 10 * n_params, gram_f, poly_f, upd_f, 10 * n_params]
        breakdown = {}
        for k, name in enumerate(names):
            mu.muon_timing_enable(k)
            for _ in range(20):
                step()
            ms, cnt = mu.muon_timing_read()
            mu.muon_timing_enable(-1)
            per = ms / max(1, cnt)
            if k in (2, 3, 4):
                ach = per_launch_work[k] / (per * 1e-3) / 1e12
                breakdown[name] = {"ms_per_launch": round(per, 5), "launches_per_step": cnt // 20,
                                   "TFLOP/s": round(ach, 1), "frac_bf16_peak": round(ach / PEAK_BF16_TFLOPS, 4)}
            else:
                ach = per_launch_work[k] / (per * 1e-3) / 1e9
                breakdown[name] = {"ms_per_launch": round(per, 5), "launches_per_step": cnt // 20,
                                   "GB/s": round(ach, 1), "frac_hbm_peak": round(ach / PEAK_HBM_GBS, 4)}
        torch.cuda.synchronize()
        ns_ms = sum(breakdown[k]["ms_per_launch"] * breakdown[k]["launches_per_step"] for k in ("gram", "poly", "update"))
        ns_tf = ns_flops_step / (ns_ms * 1e-3) / 1e12
        dense_tf = NS_STEPS * ns_flops_dense(shapes) / (ns_ms * 1e-3) / 1e12
        breakdown["ns_all"] = {"ms_per_step": round(ns_ms, 5), "TFLOP/s": round(ns_tf, 1),
                               "frac_bf16_peak": round(ns_tf / PEAK_BF16_TFLOPS, 4),
                               "dense_equivalent_TFLOP/s": round(dense_tf, 1)}

    adamw = None if args.no_adamw else bench_adamw(torch, mu, wl)
    small = None if args.no_small else bench_small(torch, mu, wl)
    large = None if args.no_large else bench_large(torch, mu, wl)
    vendor = None if args.no_vendor else bench_vendor_ns(torch, wl, ns_flops_step)
    peaks = None if args.no_vendor else bench_measured_peaks(torch)
    if peaks is not None and breakdown is not None:
        for name, v in breakdown.items():
            if "TFLOP/s" in v:
                v["frac_measured_gemm_peak"] = round(v["TFLOP/s"] / peaks["bf16_gemm_TFLOP/s"], 4)
            elif "GB/s" in v:
                v["frac_measured_copy"] = round(v["GB/s"] / peaks["copy_GB/s"], 4)

    # A plain copy of known size, outside the timed region: it calibrates
    # rocprofv3's FETCH_SIZE / WRITE_SIZE counters when this script is profiled.
    calib = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
    calib2 = torch.empty_like(calib)
    calib2.copy_(calib)
    torch.cuda.synchronize()
    del calib, calib2

    out = {
        "metric": "Muon steps/s on GPT-2-124M hidden matrices; NS TFLOP/s as % bf16 MFMA peak",
        "value": round(args.steps / wall_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_hip_events": round(ev_ms_per_step, 5),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 5) for q in (10, 50, 90)],
        "step_ms_max": round(float(step_ms.max()), 5),
        "host_enqueue_ms_per_step": [round(float(enq_ms.mean()), 4), round(float(enq_ms.max()), 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "GPT-2-124M hidden set: 12 layers x (768x2304, 768x768, 768x3072, 3072x768), "
                        "48 fp32 matrices, 84.9M params; grads N(0,1e-3^2) x 10^U(-1,1) per layer",
            "n_matrices": len(shapes), "n_params": n_params, "ns_steps": NS_STEPS, "lr": LR, "beta": BETA,
            "coeffs": list(COEFFS),
        },
        "ns_tflops_per_step": round(ns_flops_step / 1e12, 4),
        "ns_tflops_per_s_whole_step": round(ns_flops_step / (ms_per_step * 1e-3) / 1e12, 1),
        "roofline": {
            "kernel": "ns_update (X <- aX + BX, bf16 MFMA)",
            "bound": "mfma",
            "achieved": round(upd_tflops, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(upd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_from_profiles(),
            "flops_per_launch": upd_f,
            "ms_per_launch": round(upd_ms, 5),
            "launches": upd_launches,
            "timing": f"HIP events around each update launch on the launch stream, {roof_steps} steps "
                      "measured after the timed region",
        },
    }
    if breakdown is not None:
        out["kernels"] = breakdown
    if adamw is not None:
        out["adamw"] = adamw
    if small is not None:
        out["small_workloads"] = small
    if large is not None:
        out["large_workloads"] = large
    if vendor is not None:
        if breakdown is not None:
            vendor["library_ns_ms_per_step"] = breakdown["ns_all"]["ms_per_step"]
            vendor["speedup_of_library"] = round(vendor["ms_per_step"] / breakdown["ns_all"]["ms_per_step"], 2)
        out["vendor_ns_baseline"] = vendor
    if peaks is not None:
        out["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
