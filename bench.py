#!/usr/bin/env python3
"""Batch-1 gated subspace linear maps on one MI355X: tokens/s and HBM roofline.

Workload (default): a GPT-J-6B-shaped stack of 28 layers x 4 linear maps
(QKV 4096->12288, out 4096->4096, fc_in 4096->16384 with k=256, fc_out
16384->4096 with k=512), bf16 weights, per-layer bases that follow a depth
cascade, eps=0.05 and exactly 5% slow tokens per map over 512 synthetic
decode steps.  One step = one token through all 112 maps: one gsi_stack
call, i.e. one launch of stack_kernel (projection, gate and the chosen
path's output of every map).  Inputs are synthetic and resident in HBM
before timing starts.

Prints one JSON line (rank 0, N=1):
  value        decode steps (= tokens at batch 1) per second, wall clock
  roofline     stack_kernel: algorithmic bytes per launch (averaged over the
               timed steps) / its mean launch time from HIP events recorded
               on the launch stream around the timed region, against 8 TB/s;
               traffic: HBM bytes per launch from the rocprofv3 counter
               record in profiles/ (null unless that record was taken on the
               same kernel sources, by sha256)
  status       the stack's device status word after the timed region and
               after the per-launch pass (0: every wait finished; the run
               exits with status 3 otherwise)
  cpu_baseline the fp64 oracle on a bounded sample of the same workload, on
               all host threads and on one thread
Other workloads (--workload): the chained stack, the 13B-shaped stack, the
batched T=256 map, single GPT-J-shaped maps at T=1, the operating-point
sweep and the basis calibration.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "GSI linear tokens/s at d=4096 batch-1 + achieved HBM GB/s vs peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=512)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--workload", default="gptj6b-28L",
                   choices=["gptj6b-28L", "gptj6b-28L-chained", "llama13b-40L", "batched-t256", "sweep",
                            "calibrate-gptj6b-28L", "gptj-maps-t1"])
    p.add_argument("--layers", type=int, default=None, help="override the layer count")
    p.add_argument("--exact-rho", action="store_true",
                   help="every map caches E = V^T V - I and gates on the exact residual ratio")
    p.add_argument("--shared-bases", action="store_true",
                   help="maps that read one input (GPT-J qkv and fc_in, LLaMA gate and up) share "
                        "its tokens and basis, hence one projection")
    p.add_argument("--dense-steps", type=int, default=16)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--cells", default=None,
                   help="batched-t256 only: run just these cells, 'k:slow_share,...' (for profiling)")
    p.add_argument("--trace", action="store_true",
                   help="stack workloads: per-job trace of three steps through the instrumented library "
                        "(rank_gated_memory_amd/libgsi_trace.so, build.build_traced()); prints the "
                        "summary instead of the bench line")
    return p.parse_args()


def build_workload(name, layers_override, dev, shared=False, exact=False):
    import torch

    from rank_gated_memory_amd import gsi, synth

    cfg, layers, roles, steps, rate, cascade = synth.STACKS[name]
    if layers_override:
        layers = layers_override
    t0 = time.perf_counter()
    data = synth.stack_config(cfg, layers, roles, steps, rate, device=dev, cascade=cascade,
                              share=synth.SHARED_INPUTS[name] if shared else None)
    torch.cuda.synchronize()
    log(f"inputs drawn in {time.perf_counter() - t0:.1f}s")
    t0 = time.perf_counter()
    maps = [[gsi.Map(mi.W, mi.V, exact_rho=exact) for mi in row] for row in data]
    for row in maps:
        for m in row:
            gsi.gsi_prepare(m)
    torch.cuda.synchronize()
    log(f"images M prepared in {time.perf_counter() - t0:.2f}s")
    outs = []
    for row in data:
        orow = []
        for mi in row:
            orow.append((torch.empty((steps, mi.d_out), dtype=torch.bfloat16, device=dev),
                         torch.empty(steps, dtype=torch.float32, device=dev),
                         torch.zeros(steps, dtype=torch.uint8, device=dev)))
        outs.append(orow)
    t0 = time.perf_counter()
    plans = []
    for s in range(steps):
        calls = []
        for row, mrow, orow in zip(data, maps, outs):
            for mi, m, (Y, R, S) in zip(row, mrow, orow):
                calls.append((m, mi.X[s], Y[s], 0.05, R[s:s + 1], S[s:s + 1]))
        plans.append(gsi.Stack(calls, device=dev))
    torch.cuda.synchronize()
    log(f"{steps} stack plans of {len(plans[0]._keep)} calls built in {time.perf_counter() - t0:.2f}s")
    return dict(cfg=cfg, layers=layers, roles=roles, steps=steps, rate=rate, data=data, maps=maps,
                outs=outs, plans=plans, exact=exact)


class _Shape:
    """d, d_out, k of one call, for byte accounting; shared: the call reads
    the projection of an earlier call with the same input and basis."""

    def __init__(self, d, d_out, k, shared=False):
        self.d, self.d_out, self.k, self.shared = d, d_out, k, shared


def call_bytes(mi, slow):
    """Algorithmic bytes of one call: V_k and x are not read again by a call
    that shares an earlier call's projection."""
    from rank_gated_memory_amd import accounting as acc

    b = acc.token_bytes(mi.d, mi.d_out, mi.k, 2, slow)
    if getattr(mi, "shared", False):
        b -= acc.project_bytes(mi.d, mi.k, 2)
    return b


def build_chained_workload(layers_override, dev):
    """GPT-J-shaped layers whose maps feed each other: one decode step is one
    token through 28 parallel blocks as 56 waves (qkv and fc_in on the layer
    input; out on the value third of qkv's output, fc_out on fc_in's output,
    which is the next layer's input), one gsi_stack launch with device-side
    barriers between the waves.  Weights carry each layer's input subspace to
    the next (synth.subspace_map), so the slow share set at the first layer
    (5% of the steps) carries down the stack."""
    import torch

    from rank_gated_memory_amd import gsi, synth

    layers = layers_override or 28
    steps, rate = 512, 0.05
    d, k, f, kf = 4096, 256, 16384, 512
    t0 = time.perf_counter()
    cfg, (vh0, uh0) = synth.chain_config(d, k, f, kf, layers, (6, 0), device=dev, dtype=torch.bfloat16)
    mask = synth.pick_slow(steps, int(round(rate * steps)), (6, 0, 0, synth.P_PICK), dev)
    X0, _ = synth.tokens(vh0, uh0, mask, (6, 0, 0))
    X0 = X0.to(torch.bfloat16)
    torch.cuda.synchronize()
    log(f"chained inputs drawn in {time.perf_counter() - t0:.1f}s")
    roles = (("qkv", d, 3 * d, k), ("out", d, d, k), ("fc_in", d, f, k), ("fc_out", f, d, kf))
    maps = [{r: gsi.Map(*layer.maps[r]) for r, *_ in roles} for layer in cfg]
    for row in maps:
        for m in row.values():
            gsi.gsi_prepare(m)
    outs = [{r: (torch.empty((steps, m.d_out), dtype=torch.bfloat16, device=dev),
                 torch.empty(steps, dtype=torch.float32, device=dev),
                 torch.zeros(steps, dtype=torch.uint8, device=dev)) for r, m in row.items()} for row in maps]
    plans = []
    t0 = time.perf_counter()
    for s_ in range(steps):
        calls, h = [], X0[s_]
        for l in range(layers):
            mp, o = maps[l], outs[l]
            for r in ("qkv", "fc_in"):
                Y, R, S = o[r]
                calls.append((mp[r], h, Y[s_], 0.05, R[s_:s_ + 1], S[s_:s_ + 1], 2 * l))
            Y, R, S = o["out"]
            calls.append((mp["out"], o["qkv"][0][s_, 2 * d:3 * d], Y[s_], 0.05, R[s_:s_ + 1], S[s_:s_ + 1], 2 * l + 1))
            Y, R, S = o["fc_out"]
            calls.append((mp["fc_out"], o["fc_in"][0][s_], Y[s_], 0.05, R[s_:s_ + 1], S[s_:s_ + 1], 2 * l + 1))
            h = Y[s_]
        plans.append(gsi.Stack(calls, device=dev))
    torch.cuda.synchronize()
    log(f"{steps} chained plans of {len(plans[0]._keep)} calls built in {time.perf_counter() - t0:.2f}s")
    order = ("qkv", "fc_in", "out", "fc_out")  # the call order inside a layer of a plan
    dims = {r: (dd, do, kk) for r, dd, do, kk in roles}
    # fc_in reads the same input with the same basis as qkv: one projection
    data = [[_Shape(*dims[r], shared=(r == "fc_in")) for r in order] for _ in range(layers)]
    flat_outs = [[outs[l][r] for r in order] for l in range(layers)]
    return dict(cfg=6, layers=layers, roles=[(r, *dims[r]) for r in order], steps=steps, rate=rate,
                data=data, maps=maps, outs=flat_outs, plans=plans, chained=True, host_cfg=cfg, X0=X0)


def step_bytes(wl, step_slow):
    """Algorithmic bytes of one step split by phase, given its gate per map."""
    from rank_gated_memory_amd import accounting as acc

    proj = apply = 0
    i = 0
    for row in wl["data"]:
        for mi in row:
            slow = bool(step_slow[i])
            if not getattr(mi, "shared", False):
                proj += acc.project_bytes(mi.d, mi.k, 2)
                if wl.get("exact"):
                    proj += acc.gram_bytes(mi.k, 2)
            apply += acc.apply_bytes(mi.d, mi.d_out, mi.k, 2, slow)
            i += 1
    return proj, apply


def cpu_baseline_chained(wl, seconds):
    """The fp64 oracle chain on a bounded sample: the first two layers (8
    chained calls) of each step, steps in order, time scaled to all layers."""
    import numpy as np
    import torch

    from oracle import gsi_oracle as orc

    cores = blas_threads()
    d = 4096
    host = []
    for l in range(2):
        mp = {}
        for r, (W, V) in wl["host_cfg"][l].maps.items():
            Wf = W.to("cpu", torch.float64).numpy()
            Vf = V.to("cpu", torch.float64).numpy()
            mp[r] = (Wf, Vf, orc.prepare(Wf, Vf))
        host.append(mp)
    X0 = wl["X0"].to("cpu", torch.float64).numpy()

    def calls_for(s_):
        cs = []
        h_src = None  # index of the call whose output is the layer input
        for l in range(2):
            idx = {}
            for r in ("qkv", "fc_in"):
                W, V, M = host[l][r]
                c = {"W": W, "V": V, "M": M, "eps": 0.05}
                if h_src is None:
                    c["x"] = X0[s_]
                else:
                    c["src"] = (h_src, 0)
                idx[r] = len(cs)
                cs.append(c)
            W, V, M = host[l]["out"]
            cs.append({"W": W, "V": V, "M": M, "eps": 0.05, "src": (idx["qkv"], 2 * d)})
            W, V, M = host[l]["fc_out"]
            h_src = len(cs)
            cs.append({"W": W, "V": V, "M": M, "eps": 0.05, "src": (idx["fc_in"], 0)})
        return cs

    t0 = time.perf_counter()
    done = 0
    while True:
        orc.chain(calls_for(done % wl["steps"]), "bf16")
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    maps_total = sum(len(r) for r in wl["data"])
    per_step = el / done * (maps_total / 8)
    return {"value": 1.0 / per_step, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} decode steps (in order) through the first 2 of {wl['layers']} chained layers "
                      f"(8 of {maps_total} maps), fp64 numpy, {el:.1f}s; step time scaled by {maps_total}/8 maps"}


def host_cpu():
    """The host's CPU model and logical CPU count (context of the CPU baseline)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # noqa: BLE001
        return os.cpu_count()


def with_single_thread(fn, wl, seconds):
    """fn's CPU baseline on every BLAS thread, then again limited to one thread."""
    full = fn(wl, seconds)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = fn(wl, seconds / 2)
        full["single_thread"] = {"value": one["value"], "cores": 1, "sample": one["sample"]}
    except ImportError:
        full["single_thread"] = None
    full.update(host_cpu())
    return full


def cpu_baseline(wl, seconds):
    """The fp64 oracle on a bounded sample: two layers' maps, tokens in step order."""
    import numpy as np
    import torch

    from oracle import gsi_oracle as orc

    cores = blas_threads()
    layers = wl["layers"]
    pick = [0, layers // 2] if layers > 1 else [0]
    host = []
    for l in pick:
        for mi in wl["data"][l]:
            W = mi.W.to("cpu", torch.float64).numpy()
            V = mi.V.to("cpu", torch.float64).numpy()
            host.append((W, V, orc.prepare(W, V), mi.X.to("cpu", torch.float64).numpy()))
    # time whole steps of the sampled maps, in step order (wrapping round the
    # workload's steps), until the time budget is spent
    t0 = time.perf_counter()
    done = 0
    while True:
        for W, V, M, X in host:
            orc.linear_token(W, V, M, X[done % wl["steps"]], 0.05)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    maps_total = sum(len(r) for r in wl["data"])
    per_step = el / done * (maps_total / len(host))
    return {"value": 1.0 / per_step, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} decode steps (of the workload's {wl['steps']}, in order, wrapping) "
                      f"through {len(host)} of {maps_total} maps (layers {pick}), fp64 numpy, "
                      f"{el:.1f}s; step time scaled by {maps_total}/{len(host)} maps"}


STACK_SOURCES = ("gsi_kernels.hip", "gsi_internal.h", "gsi_gram.h")
BATCHED_SOURCES = ("gsi_batched.hip", "gsi_batched.h", "gsi_gram.h")


def kernel_source_sha(files=STACK_SOURCES) -> str:
    """sha256 of the kernel sources; counter figures are only reported for the code they measured."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "rank_gated_memory_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str, files=STACK_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches this code."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_sha(files):
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else float(k["hbm_bytes_per_launch"])


PEAK_BF16_TFLOPS = 2500.0


def bench_batched(args):
    """T=256 tokens through one bf16 map d=4096 -> 16384, k x slow-share sweep.

    Prints one JSON line: tokens/s per cell (whole gsi_linear call: projection
    GEMM, gate, compacted fast and slow GEMMs), algorithmic GB/s, and the
    matrix-core fraction of the whole call at each cell.  Each cell is timed
    twice: cache-hot (the same map and tokens every call: the ~155 MB
    working set of a call fits in the 256 MB MALL) and rotated (call i reads
    replica i mod R of V_k, M and X and replica i mod R_w of W, >= 1 GB of
    each, so every call reads its bytes from HBM); the rotated figure is the
    HBM one.
    """
    import numpy as np
    import torch

    from rank_gated_memory_amd import gsi, synth

    dev = torch.device("cuda:0")
    cells = []
    grid = [(k, frac) for k in (64, 256, 512) for frac in (0.0, 0.1, 0.5, 1.0)]
    if args.cells:
        grid = [(int(c.split(":")[0]), float(c.split(":")[1])) for c in args.cells.split(",")]
    prep = []
    GB = 1.0e9
    for k, frac in grid:
        mi = synth.config5(k, frac, device=dev, w_device=dev)
        m = gsi.Map(mi.W, mi.V)
        gsi.gsi_prepare(m)
        if not any(p["k"] == k for p in prep):
            # the image M = W V_k (once per map, off the per-token path)
            reps = 5
            torch.cuda.synchronize()
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p0.record()
            for _ in range(reps):
                gsi.gsi_prepare(m)
            p1.record()
            torch.cuda.synchronize()
            pus = p0.elapsed_time(p1) / reps * 1e3
            pfl = 2.0 * mi.d * mi.d_out * k
            prep.append({"k": k, "us_per_map": pus, "tflops": pfl / pus / 1e6,
                         "mfma_frac": pfl / pus / 1e6 / PEAK_BF16_TFLOPS})
            log(f"prepare M (d={mi.d}, d_out={mi.d_out}, k={k}): {pus:.1f} us, {pfl / pus / 1e6:.0f} TFLOP/s")
        T = mi.X.shape[0]
        y = torch.empty(T, mi.d_out, dtype=torch.bfloat16, device=dev)
        rho = torch.empty(T, device=dev)
        sl = torch.empty(T, dtype=torch.uint8, device=dev)
        ws = gsi.workspace(gsi.gsi_linear_workspace(m, T), dev)
        gsi.gsi_linear(m, mi.X, 0.05, y=y, rho=rho, slow=sl, ws=ws)
        torch.cuda.synchronize()
        ns = int(sl.sum())
        nf = T - ns
        d, do = mi.d, mi.d_out
        byts = 2 * (d * k + T * d + T * do) + (2 * do * k if nf else 0) + (2 * d * do if ns else 0)
        flops = 2 * T * d * k + 2 * 2 * nf * do * k + 2 * ns * d * do
        # replicas for the rotated timing
        vmx = mi.V.numel() * 2 + m.M.numel() + mi.X.numel() * 2
        R = int(min(256, max(2, np.ceil(1.0 * GB / vmx))))
        Rw = int(max(2, np.ceil(1.0 * GB / (mi.W.numel() * 2)))) if ns else 1
        Ws = [mi.W] + replicas(mi.W, Rw - 1)
        Vs = [mi.V] + replicas(mi.V, R - 1)
        Ms = [m.M] + replicas(m.M, R - 1)
        Xs = [mi.X] + replicas(mi.X, R - 1)
        rot = [gsi.Map(Ws[j % Rw], Vs[j], M=Ms[j]) for j in range(R)]
        timing = {}
        for place in ("hot", "rotated"):
            def call(i):
                if place == "hot":
                    gsi.gsi_linear(m, mi.X, 0.05, y=y, rho=rho, slow=sl, ws=ws)
                else:
                    gsi.gsi_linear(rot[i % R], Xs[i % R], 0.05, y=y, rho=rho, slow=sl, ws=ws)
            for i in range(args.warmup):
                call(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(args.steps):
                call(i)
            e1.record()
            torch.cuda.synchronize()
            timing[place] = e0.elapsed_time(e1) / args.steps * 1e3
            assert int(sl.sum()) == ns, "gates changed between replicas"
        us = timing["rotated"]
        cells.append({"k": k, "slow_share": frac, "slow_tokens": ns, "us_per_call": us,
                      "tokens_per_s": T / (us * 1e-6), "gbps": byts / us / 1e3,
                      "tflops": flops / us / 1e6, "mfma_frac": flops / us / 1e6 / PEAK_BF16_TFLOPS,
                      "bytes_per_call": byts, "replicas": [R, Rw],
                      "hot_us_per_call": timing["hot"], "hot_gbps": byts / timing["hot"] / 1e3})
        log(f"k={k} slow={frac}: rotated {us:.1f} us ({byts / us / 1e3:.0f} GB/s), "
            f"cache-hot {timing['hot']:.1f} us, {T / us * 1e6:.0f} tokens/s")
        del m, mi, ws, y, rot, Ws, Vs, Ms, Xs
        torch.cuda.empty_cache()
    heads = [c for c in cells if c["k"] == 256 and c["slow_share"] == 0.1]
    head = heads[0] if heads else cells[0]
    cpu = None if args.no_cpu else with_single_thread(cpu_baseline_batched, head, args.cpu_seconds)
    print(json.dumps({
        "metric": "GSI batched gated linear tokens/s (T=256, d=4096 -> 16384)",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["us_per_call"] / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "batched-t256: T=256, d=4096, d_out=16384, value at k=256, 10% slow, "
                               "calls rotated over >= 1 GB of map and token replicas",
                   "cells": cells, "prepare": prep},
        # the whole gsi_linear call of the head cell (projection GEMM, gate,
        # output kernels) against the HBM roof: its algorithmic bytes (V_k,
        # X, Y, M once if any token is fast, W once if any is slow) over the
        # rotated call time
        "roofline": {"bound": "hbm", "kernel": "gsi_linear (bproj, bgate, bout)",
                     "achieved": head["gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": head["gbps"] / PEAK_HBM_GBPS,
                     # bytes out of the L2s per call of the head cell (bproj + bgate + bout
                     # counters), when the committed record matches these sources
                     "traffic": measured_traffic("batched-t256", "gsi_linear (bproj, bgate, bout)",
                                                 BATCHED_SOURCES)},
        "cpu_baseline": cpu,
    }), flush=True)


def cpu_baseline_batched(head, seconds):
    """The fp64 oracle on the head cell's map (k=256, 10 % slow): its tokens
    one by one through orc.linear_token until the time budget is spent."""
    import torch

    from oracle import gsi_oracle as orc
    from rank_gated_memory_amd import synth

    mi = synth.config5(head["k"], head["slow_share"], device="cpu", w_device="cpu")
    W = mi.W.double().numpy()
    V = mi.V.double().numpy()
    M = orc.prepare(W, V)
    X = mi.X.double().numpy()
    cores = blas_threads()
    t0 = time.perf_counter()
    done = 0
    while True:
        orc.linear_token(W, V, M, X[done % X.shape[0]], 0.05)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} tokens of the k={head['k']}, {head['slow_share'] * 100:.0f}%-slow cell "
                      f"(the same recipe drawn on the host; tokens in order, wrapping), one token at "
                      f"a time, fp64 numpy, {el:.1f}s"}


def replicas(t, n):
    """n independent copies of tensor t (same values, distinct memory)."""
    return [t.clone() for _ in range(n)]


def bench_single_maps(args):
    """Each GPT-J-shaped map alone at batch 1: 1000 sequential single-token
    gsi_linear calls (50 slow at seeded positions, eps = 0.05), per map.

    Two placements of the map's bytes:
      * cache-hot: every call reads the same V_k, M (and W for the slow
        tokens); M + V_k of a map (4-21 MB) stay in the 256 MB MALL, so this
        is not an HBM figure;
      * rotated: token t reads replica t mod R of (V_k, M) and replica
        t mod R mod R_w of W, the replicas together >= 1 GB for each of the
        two kinds, so successive calls miss the caches: the HBM figure.
    Each placement runs its 1000 calls issued from the host one by one, and
    as one captured HIP graph (the graph's replays are checked bitwise
    against the eager outputs).  Two entry points: gsi_linear at T = 1 (a
    projection launch and an output launch per token) and, rotated, a
    one-call gsi_stack plan per token (one launch per token).  Bytes per token: 2k(d + d_out) + 2d + 2d_out
    fast, + 2 d d_out slow.  The dense line is the same calls forced slow.
    """
    import numpy as np
    import torch

    from rank_gated_memory_amd import accounting as acc
    from rank_gated_memory_amd import gsi, synth

    dev = torch.device("cuda:0")
    T, eps = 1000, 0.05
    GB = 1.0e9
    results = []
    stream = torch.cuda.Stream()
    for role in synth.GPTJ_MAPS:
        mi = synth.config2(T=T, device=dev, w_device=dev, maps=[role])[0]
        base = gsi.Map(mi.W, mi.V)
        gsi.gsi_prepare(base)
        vm_bytes = base.V.numel() * 2 + base.M.numel()
        R = max(1, int(np.ceil(1.0 * GB / vm_bytes)))
        Rw = max(1, int(np.ceil(1.0 * GB / (mi.W.numel() * 2))))
        Ws = [mi.W] + replicas(mi.W, Rw - 1)
        Vs = [mi.V] + replicas(mi.V, R - 1)
        Ms = [base.M] + replicas(base.M, R - 1)
        rot = [gsi.Map(Ws[j % Rw], Vs[j], M=Ms[j]) for j in range(R)]
        y = torch.empty((T, mi.d_out), dtype=torch.bfloat16, device=dev)
        rho = torch.empty(T, dtype=torch.float32, device=dev)
        sl = torch.empty(T, dtype=torch.uint8, device=dev)
        ws = gsi.workspace(gsi.gsi_linear_workspace(base, 1), dev)

        plans = {}
        for place, maps_of in (("hot", lambda t: base), ("rotated", lambda t: rot[t % R])):
            plans[place] = [gsi.Stack([(maps_of(t), mi.X[t], y[t], eps, rho[t:t + 1], sl[t:t + 1])], device=dev)
                            for t in range(T)]
        ws1 = gsi.workspace(max(p.ws_bytes for pl in plans.values() for p in pl), dev)

        def issue(maps_of, mode=gsi.GATED, kind="gsi_linear", place="hot"):
            if kind == "gsi_stack":
                for t in range(T):
                    gsi.gsi_stack(plans[place][t], mode, ws1, stream=stream)
                return
            for t in range(T):
                gsi.gsi_linear(maps_of(t), mi.X[t:t + 1], eps, mode=mode, y=y[t:t + 1], rho=rho[t:t + 1],
                               slow=sl[t:t + 1], ws=ws, stream=stream)

        cell = {"map": role[0], "d": mi.d, "d_out": mi.d_out, "k": mi.k, "tokens": T,
                "replicas_vk_m": R, "replicas_w": Rw}
        for place, maps_of, kind in (("hot", lambda t: base, "gsi_linear"),
                                     ("rotated", lambda t: rot[t % R], "gsi_linear"),
                                     ("rotated", lambda t: rot[t % R], "gsi_stack")):
            for mode, tag in ((gsi.GATED, "gated"), (gsi.FORCE_SLOW, "dense")):
                with torch.cuda.stream(stream):
                    issue(maps_of, mode, kind, place)
                    stream.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    issue(maps_of, mode, kind, place)
                    e1.record(stream)
                    stream.synchronize()
                eager_us = e0.elapsed_time(e1) * 1e3 / T
                ref = (y.clone(), rho.clone(), sl.clone())
                slow = ref[2].cpu().numpy().astype(bool)
                byts = sum(acc.token_bytes(mi.d, mi.d_out, mi.k, 2, bool(s_)) for s_ in slow)
                # the same calls captured once as a graph, replayed
                g = torch.cuda.CUDAGraph()
                y.zero_()
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=stream):
                    issue(maps_of, mode, kind, place)
                reps = 3
                ok = True
                times = []
                for _ in range(reps):
                    y.zero_()
                    sl.fill_(7)
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    with torch.cuda.stream(stream):
                        # the graph's kernels run on the stream it is replayed on
                        e0.record(stream)
                        g.replay()
                        e1.record(stream)
                    torch.cuda.synchronize()
                    times.append(e0.elapsed_time(e1) * 1e3 / T)
                    ok = ok and torch.equal(y.view(torch.int16), ref[0].view(torch.int16)) and torch.equal(sl, ref[2])
                del g
                graph_us = float(np.median(times))
                key = f"{place}_{tag}" + ("_single_launch" if kind == "gsi_stack" else "")
                cell[key] = {"us_per_token_eager": eager_us, "us_per_token_graph": graph_us,
                             "slow_tokens": int(slow.sum()), "bytes_per_token": byts / T,
                             "gbps_graph": byts / T / graph_us / 1e3,
                             "hbm_frac_graph": byts / T / graph_us / 1e3 / PEAK_HBM_GBPS,
                             "graph_replays_match_eager": bool(ok)}
                log(f"{role[0]} {key}: eager {eager_us:.2f} us/token, graph {graph_us:.2f} us/token, "
                    f"{byts / T / graph_us / 1e3:.0f} GB/s, replays match {ok}")
                if not ok:
                    raise SystemExit(f"graph replay of {role[0]} {key} differs from the eager outputs")
        cell["speedup_vs_dense_rotated_graph"] = (cell["rotated_dense"]["us_per_token_graph"]
                                                 / cell["rotated_gated"]["us_per_token_graph"])
        results.append(cell)
        del rot, Ws, Vs, Ms, base, mi, y, ws, plans, ws1
        torch.cuda.empty_cache()
    qkv = results[0]
    print(json.dumps({
        "metric": "GSI single-map batch-1 latency: us per token per GPT-J-shaped map (rotated, HBM)",
        "value": qkv["rotated_gated"]["us_per_token_graph"], "unit": "us/token", "n_gpus": 1, "steps": T,
        "warmup": T, "ms_per_step": qkv["rotated_gated"]["us_per_token_graph"] / 1e3,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gptj-maps-t1: QKV 4096->12288, out 4096->4096, fc_in 4096->16384 (k=256), "
                               "fc_out 16384->4096 (k=512); 1000 sequential single-token calls per map, "
                               "50 slow, eps=0.05; value: QKV, rotated over >= 1 GB of replicas, graph replay",
                   "maps": results},
        "roofline": {"bound": "hbm", "kernel": "gsi_linear T=1 (proj_kernel + apply_kernel)",
                     "achieved": qkv["rotated_gated"]["gbps_graph"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": qkv["rotated_gated"]["hbm_frac_graph"], "traffic": None},
    }), flush=True)


def bench_sweep(args):
    """Operating points: basis size k, threshold eps and the forced modes on spectral tokens.

    GPT-J-shaped maps (28 layers by default) whose tokens have a power-law
    spectrum, so that the fast share follows from k and eps.  For each k
    (fc_out takes 2k, as in the GPT-J shapes) and each of gated eps = 0.05,
    gated eps = 0.10, static projection (every token fast) and dense (every
    token slow), one batch-1 decode pass over the workload's steps through
    gsi_stack: fast share, algorithmic bytes and GB/s, tokens/s, parameters
    read per token, and the output error against the dense outputs.
    """
    import numpy as np
    import torch

    from rank_gated_memory_amd import accounting as acc
    from rank_gated_memory_amd import gsi, synth

    dev = torch.device("cuda:0")
    layers = args.layers or 28
    steps = 128
    t0 = time.perf_counter()
    data = synth.sweep_config(layers, steps, device=dev)
    torch.cuda.synchronize()
    log(f"sweep inputs drawn in {time.perf_counter() - t0:.1f}s")
    params = sum(e["d"] * e["d_out"] for row in data for e in row)
    cells = []
    for kk in (128, 256):
        ks = [[2 * kk if e["name"] == "fc_out" else kk for e in row] for row in data]
        maps = [[gsi.Map(e["W"], e["V64"][:, :k].to(torch.bfloat16).contiguous()) for e, k in zip(row, krow)]
                for row, krow in zip(data, ks)]
        for row in maps:
            for m in row:
                gsi.gsi_prepare(m)
        outs = [[(torch.empty((steps, e["d_out"]), dtype=torch.bfloat16, device=dev),
                  torch.empty(steps, dtype=torch.float32, device=dev),
                  torch.zeros(steps, dtype=torch.uint8, device=dev)) for e in row] for row in data]
        flat = [(e, m, o, k) for row, mrow, orow, krow in zip(data, maps, outs, ks)
                for e, m, o, k in zip(row, mrow, orow, krow)]

        def plans_for(eps):
            return [gsi.Stack([(m, e["X"][s], Y[s], eps, R[s:s + 1], S[s:s + 1])
                               for e, m, (Y, R, S), _ in flat], device=dev) for s in range(steps)]

        plans = {0.05: plans_for(0.05), 0.10: plans_for(0.10)}
        ws = gsi.workspace(max(p.ws_bytes for p in plans[0.05]), dev)

        def run(mode, eps):
            for i in range(4):
                gsi.gsi_stack(plans[eps][i], mode, ws)
            torch.cuda.synchronize()
            t = time.perf_counter()
            for i in range(steps):
                gsi.gsi_stack(plans[eps][i], mode, ws)
            torch.cuda.synchronize()
            return time.perf_counter() - t

        run(gsi.FORCE_SLOW, 0.05)
        dense_y = [Y.clone() for _, _, (Y, _, _), _ in flat]
        for label, mode, eps in (("gated", gsi.GATED, 0.05), ("gated", gsi.GATED, 0.10),
                                 ("static projection", gsi.FORCE_FAST, 0.05),
                                 ("dense", gsi.FORCE_SLOW, 0.05)):
            wall = run(mode, eps)
            slow = torch.stack([S for _, _, (_, _, S), _ in flat], dim=1).cpu().numpy().astype(bool)
            byts = sum(acc.token_bytes(e["d"], e["d_out"], k, 2, bool(slow[s, j]))
                       for s in range(steps) for j, (e, _, _, k) in enumerate(flat))
            read = sum((e["d"] * k + (e["d_out"] * e["d"] if slow[s, j] else e["d_out"] * k))
                       for s in range(steps) for j, (e, _, _, k) in enumerate(flat)) / steps
            errs = []
            for (_, _, (Y, _, _), _), Yd in zip(flat, dense_y):
                yd = Yd.float()
                errs.append(((Y.float() - yd).norm(dim=1) / yd.norm(dim=1)).cpu())
            err = torch.cat(errs).numpy()
            cell = {"k": kk, "k_fc_out": 2 * kk, "mode": label, "eps": eps if mode == gsi.GATED else None,
                    "fast_share": float(1.0 - slow.mean()), "tokens_per_s": steps / wall,
                    "us_per_step": wall / steps * 1e6, "gbytes_per_step": byts / steps / 1e9,
                    "gbps": byts / wall / 1e9, "params_read_per_token_M": read / 1e6,
                    "params_k_over_d_M": params * kk / 4096 / 1e6,
                    "rel_err_vs_dense_mean": float(err.mean()), "rel_err_vs_dense_p99": float(np.quantile(err, 0.99)),
                    "rel_err_vs_dense_max": float(err.max())}
            cells.append(cell)
            log(f"k={kk} {label} eps={cell['eps']}: fast {cell['fast_share']:.3f}, {cell['tokens_per_s']:.0f} tok/s, "
                f"{cell['gbps']:.0f} GB/s, err mean {cell['rel_err_vs_dense_mean']:.2e} max {cell['rel_err_vs_dense_max']:.2e}")
        del maps, outs, flat, plans, ws, dense_y
        torch.cuda.empty_cache()
    head = [c for c in cells if c["k"] == 256 and c["mode"] == "gated" and c["eps"] == 0.05][0]
    print(json.dumps({
        "metric": "GSI operating points: tokens/s at batch 1 vs fast share, bytes and error",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": 4,
        "ms_per_step": head["us_per_step"] / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"sweep: {layers} layers x 4 GPT-J-shaped maps, power-law (alpha 1.1) "
                               f"spectral tokens with 5% outliers, {steps} decode steps; value at k=256, eps=0.05",
                   "params": params, "cells": cells},
    }), flush=True)


def bench_calibrate(args):
    """Basis calibration of a GPT-J-shaped 28-layer stack on the GPU.

    Per layer three inputs are calibrated (the block input read by qkv and
    fc_in, k=256; the attention output read by out, k=256; fc_in's output
    read by fc_out, d=16384, k=512) from n=2048 synthetic activation samples
    each, whose dominant subspace follows a depth cascade (rotated from
    layer to layer, mean principal cosine > 0.9) over a weaker tail.  Cold:
    every input from a Gaussian start, `cold` sweeps.  Cascade (GSI-TS
    §2.3): layer 0 cold, every later layer warm-started from the same
    input's basis one layer below, `warm` sweeps.  Reports seconds for the
    whole stack and the worst principal-angle gap to the samples' own top-k
    subspace (fp64 SVD on the host, outside the timed region) for a sample
    of inputs.
    """
    import numpy as np
    import torch

    from rank_gated_memory_amd import gsi, synth

    dev = torch.device("cuda:0")
    layers, n, cold, warm = args.layers or 28, 2048, 8, 2
    inputs = (("block_in", 4096, 256), ("attn_out", 4096, 256), ("mlp_hidden", 16384, 512))
    t0 = time.perf_counter()
    data = []
    for r, (name, d, k) in enumerate(inputs):
        frames = synth.cascade_frames(d, k, 256, layers, (7, 0, r, synth.P_CASCADE), dev)
        spec = torch.cat([torch.linspace(8.0, 4.0, k, dtype=torch.float64),
                          torch.linspace(1.0, 0.2, 256, dtype=torch.float64)])
        row = []
        for l in range(layers):
            A = synth.frame_samples(torch.cat(frames[l], 1), spec, n, (7, l, r, 1), dev).to(torch.bfloat16)
            frames[l] = None
            row.append(A)
        R0 = synth.gaussian_block(d, k, (7, 0, r, 2), dev).to(torch.bfloat16)
        data.append((name, d, k, row, R0))
    torch.cuda.synchronize()
    log(f"calibration samples drawn in {time.perf_counter() - t0:.1f}s")
    wss = {(d, k): gsi.workspace(int(gsi.lib().gsi_calibrate_workspace(ctypes_calib(n, d, k))), dev)
           for _, d, k, _, _ in data}

    def run(mode):
        out = []
        torch.cuda.synchronize()
        t = time.perf_counter()
        for name, d, k, row, R0 in data:
            prev = None
            bases = []
            for l, A in enumerate(row):
                if mode == "cascade" and prev is not None:
                    V, _ = gsi.gsi_calibrate(A, prev, warm, ws=wss[(d, k)])
                else:
                    V, _ = gsi.gsi_calibrate(A, R0, cold, ws=wss[(d, k)])
                bases.append(V)
                prev = V
            out.append(bases)
        torch.cuda.synchronize()
        return time.perf_counter() - t, out

    run("cascade")  # warm-up (module load, first launches)
    t_cold, cold_b = run("cold")
    t_casc, casc_b = run("cascade")
    status = max(int(ws[:4].view(torch.int32).item()) for ws in wss.values())
    log(f"cold ({cold} sweeps): {t_cold:.3f}s; cascade ({cold} then {warm} sweeps): {t_casc:.3f}s; status {status}")

    from oracle import gsi_oracle as orc
    gaps = {"cold": 0.0, "cascade": 0.0}
    for (name, d, k, row, _), cb, wb in zip(data, cold_b, casc_b):
        for l in (1, layers // 2, layers - 1):
            A = row[l].to("cpu", torch.float64).numpy()
            top = orc.dominant_subspace(A, k)
            for key, b in (("cold", cb), ("cascade", wb)):
                V = orc.dgks_orth(b[l].to("cpu", torch.float64).numpy())
                gaps[key] = max(gaps[key], float(1.0 - orc.principal_cosines(V, top).min()))
    log(f"worst principal-angle gap to the samples' top-k subspace: cold {gaps['cold']:.2e}, "
        f"cascade {gaps['cascade']:.2e}")
    print(json.dumps({
        "metric": "GSI basis calibration time, 28-layer GPT-J-shaped stack (84 inputs)",
        "value": t_casc, "unit": "s", "n_gpus": 1, "steps": 1, "warmup": 1, "ms_per_step": t_casc * 1e3,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"calibrate-gptj6b-28L: {layers} layers x 3 inputs (4096/k256, 4096/k256, "
                               f"16384/k512), {n} samples each; cascade {cold} cold sweeps at layer 0 then "
                               f"{warm} warm sweeps per layer; cold {cold} sweeps everywhere",
                   "cold_s": t_cold, "cascade_s": t_casc, "saving": 1.0 - t_casc / t_cold,
                   "worst_gap_cold": gaps["cold"], "worst_gap_cascade": gaps["cascade"], "status": status},
    }), flush=True)


def ctypes_calib(n, d, k):
    import ctypes

    from rank_gated_memory_amd import gsi
    return ctypes.byref(gsi.GsiCalibStruct(n, d, k, 1, 16, 16, 16, 1, 0))


TRACE_KINDS = {1: "projection unit", 2: "output unit", 8: "choosing the next job (incl. waits)"}


def trace_summary(rec, us_event, calls, slow):
    """Summary of one traced step.  rec: records (n, 4) uint64 from
    gsi_trace_read; calls: per call (d, d_out, k, wave, shares_projection);
    slow: per call gate of the step."""
    import numpy as np

    t0, t1 = rec[:, 0].astype(np.int64), rec[:, 1].astype(np.int64)
    meta, cu = rec[:, 2].astype(np.int64), rec[:, 3].astype(np.int64)
    blk, kind = meta >> 32, (meta >> 8) & 0xff
    call = cu >> 32
    T0 = t0.min()
    us = lambda x: (x - T0) * 10.0 / 1000.0  # 100 MHz constant clock
    span = float(us(t1.max()))
    out = {"workgroups": int(blk.max() + 1), "span_us": span, "event_us": float(us_event), "jobs": {}}
    for k, name in TRACE_KINDS.items():
        m = kind == k
        d = (t1[m] - t0[m]) * 10.0 / 1000.0
        if m.any():
            out["jobs"][name] = {"count": int(m.sum()), "mean_us": float(d.mean()), "p50_us": float(np.median(d)),
                                 "max_us": float(d.max()), "workgroup_us": float(d.sum())}
    sl = (meta & 1).astype(bool)
    for name, m in (("output unit, fast path", (kind == 2) & ~sl), ("output unit, slow path", (kind == 2) & sl)):
        if m.any():
            d = (t1[m] - t0[m]) * 10.0 / 1000.0
            out["jobs"][name] = {"count": int(m.sum()), "mean_us": float(d.mean()), "p50_us": float(np.median(d)),
                                 "max_us": float(d.max()), "workgroup_us": float(d.sum())}
    # the first job of every workgroup: from the workgroup's start to its end
    first = {}
    for i in np.argsort(t0):
        b = int(blk[i])
        if kind[i] in (1, 2) and b not in first:
            first[b] = i
    fs = np.array([us(t0[i]) for i in first.values()])
    if fs.size:
        out["first_unit_start_us"] = {"min": float(fs.min()), "mean": float(fs.mean()), "max": float(fs.max())}
    starts, exits = us(t0[kind == 9]), us(t0[kind == 7])
    out["start_spread_us"] = float(starts.max() - starts.min())
    out["exits_us"] = [float(exits.min()), float(exits.max())]
    # algorithmic bytes of each unit: the call's V_k (projection) or chosen
    # matrix (output) over the number of its units in the trace
    C = len(calls)
    d_, do_, k_ = (np.array([c[i] for c in calls], dtype=np.float64) for i in range(3))
    npj = np.bincount(call[kind == 1], minlength=C)
    nout = np.bincount(call[kind == 2], minlength=C)
    vb = d_ * k_ * 2.0
    ob = np.where(slow.astype(bool), d_ * do_ * 2.0, do_ * k_ * 2.0)
    byt = np.zeros(len(rec))
    m1, m2 = kind == 1, kind == 2
    byt[m1] = (vb / np.maximum(npj, 1))[call[m1]]
    byt[m2] = (ob / np.maximum(nout, 1))[call[m2]]
    out["unit_bytes"] = float(byt.sum())
    out["tb_per_s_over_span"] = float(byt.sum() / (span * 1e-6) / 1e12)
    nb = int(span) + 2
    bw, busy = np.zeros(nb), np.zeros(nb)
    for i in np.nonzero(m1 | m2)[0]:
        a, b = us(t0[i]), us(t1[i])
        if b <= a:
            continue
        rate = byt[i] / (b - a)
        for j in range(int(a), int(b) + 1):
            ov = min(b, j + 1) - max(a, j)
            if ov > 0:
                bw[j] += rate * ov
                busy[j] += ov
    out["tb_per_s_by_10us"] = [round(float(bw[j:j + 10].mean() / 1e6), 2) for j in range(0, nb, 10)]
    out["busy_workgroups_by_10us"] = [round(float(busy[j:j + 10].mean()), 0) for j in range(0, nb, 10)]
    waves = np.array([c[3] for c in calls])
    if waves.max() > 0:
        # per wave: entry (first job of the wave starts) -> last projection
        # unit ends -> last output unit ends
        jw = np.where(m1 | m2, waves[np.minimum(call, C - 1)], -1)
        ph, oph, tot, gap, fo, span_o = [], [], [], [], [], []
        prev_end = None
        for w in range(int(waves.max()) + 1):
            mw = jw == w
            if not mw.any():
                continue
            a = us(t0[mw].min())
            pe = us(t1[mw & m1].max()) if (mw & m1).any() else a
            e = us(t1[mw].max())
            ph.append(pe - a)
            oph.append(e - pe)
            tot.append(e - a)
            if (mw & m2).any():
                o0 = us(t0[mw & m2].min())
                fo.append(o0 - pe)
                span_o.append(e - o0)
            if prev_end is not None:
                gap.append(a - prev_end)
            prev_end = e
        out["waves"] = {"count": len(tot), "mean_us": float(np.mean(tot)),
                        "projection_phase_mean_us": float(np.mean(ph)),
                        "after_last_projection_mean_us": float(np.mean(oph)),
                        "last_projection_to_first_output_mean_us": float(np.mean(fo)) if fo else None,
                        "first_output_to_last_output_mean_us": float(np.mean(span_o)) if span_o else None,
                        "previous_wave_end_to_first_job_mean_us": float(np.mean(gap)) if gap else None}
    return out


def bench_trace(args):
    """Per-job trace of three decode steps of a stack workload (instrumented
    library; see gsi_kernels.hip)."""
    import ctypes

    import numpy as np
    import torch

    from rank_gated_memory_amd import gsi

    dev = torch.device("cuda:0")
    L = gsi.lib()
    if not hasattr(L, "gsi_trace_read"):
        print(f"{gsi.LIB_PATH} is not the instrumented build: set GSI_LIBRARY to "
              "rank_gated_memory_amd/libgsi_trace.so (build.build_traced())", file=sys.stderr)
        sys.exit(2)
    L.gsi_trace_read.restype = ctypes.c_int
    L.gsi_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_int]
    L.gsi_trace_reset.restype = ctypes.c_int
    chained = args.workload == "gptj6b-28L-chained"
    if chained:
        wl = build_chained_workload(args.layers, dev)
    else:
        wl = build_workload(args.workload, args.layers, dev, shared=args.shared_bases, exact=args.exact_rho)
    plans = wl["plans"]
    ws = gsi.workspace(max(p.ws_bytes for p in plans), dev)
    calls = []
    for li, row in enumerate(wl["data"]):
        for ri, mi in enumerate(row):
            wave = (2 * li + (1 if ri >= 2 else 0)) if chained else 0
            calls.append((mi.d, mi.d_out, mi.k, wave, bool(getattr(mi, "shared", False))))
    for i in range(8):
        gsi.gsi_stack(plans[i], gsi.GATED, ws)
    torch.cuda.synchronize()
    buf = np.zeros((1024 * 512, 4), dtype=np.uint64)
    steps = {}
    for s_ in (3, 10, 17):
        if L.gsi_trace_reset() != 0:
            raise RuntimeError("gsi_trace_reset failed")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gsi.gsi_stack(plans[s_], gsi.GATED, ws)
        e1.record()
        torch.cuda.synchronize()
        word = plans[s_].status(ws)
        if word != 0:
            raise gsi.StackIncomplete(word)
        n = L.gsi_trace_read(buf.ctypes.data, buf.shape[0])
        if n <= 0:
            raise RuntimeError(f"gsi_trace_read returned {n}")
        rec = buf[:n][buf[:n, 0] != 0].copy()  # unused slots are zero
        # the gates of this step, written by the traced run itself
        slow_s = torch.stack([S_[s_] for row in wl["outs"] for (_, _, S_) in row]).cpu().numpy()
        steps[f"step{s_}"] = trace_summary(rec, e0.elapsed_time(e1) * 1e3, calls, slow_s)
        log(f"step {s_}: {len(rec)} records, {steps[f'step{s_}']['event_us']:.1f} us")
    print(json.dumps({"workload": args.workload, "trace": "per-job, instrumented build", "steps": steps}))


def main():
    args = parse()
    if args.gpus != 1:
        print("the library runs on one GPU only: --gpus must be 1 (the path would shard by output "
              "rows or tokens across GPUs; only the one-GPU share is built and measured)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "batched-t256":
        bench_batched(args)
        return
    if args.workload == "sweep":
        bench_sweep(args)
        return
    if args.workload == "gptj-maps-t1":
        bench_single_maps(args)
        return
    if args.workload == "calibrate-gptj6b-28L":
        bench_calibrate(args)
        return
    if args.trace:
        bench_trace(args)
        return
    import numpy as np
    import torch

    from rank_gated_memory_amd import accounting as acc
    from rank_gated_memory_amd import gsi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    gsi.lib()
    if args.workload == "gptj6b-28L-chained":
        wl = build_chained_workload(args.layers, dev)
    else:
        wl = build_workload(args.workload, args.layers, dev, shared=args.shared_bases, exact=args.exact_rho)
    chained = bool(wl.get("chained"))
    plans = wl["plans"]
    S = wl["steps"]
    ws = gsi.workspace(max(p.ws_bytes for p in plans), dev)
    stream = torch.cuda.current_stream()

    # copy bandwidth of torch's copy kernel (context for the roofline)
    a = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * a.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    log(f"torch copy: {copy_gbps:.0f} GB/s (read+write)")

    offsets = sorted({p.status_offset for p in plans})

    def status_word():
        torch.cuda.synchronize()
        w = 0
        for o in offsets:
            w |= int(ws[o:o + 4].cpu().view(torch.int32)[0])
        return w

    # ---- timed region: K decode steps, gated; HIP events on the launch stream ----
    for i in range(args.warmup):
        gsi.gsi_stack(plans[i % S], gsi.GATED, ws)
    torch.cuda.synchronize()
    K = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        gsi.gsi_stack(plans[i % S], gsi.GATED, ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_launch = ev0.elapsed_time(ev1) * 1e-3 / K
    tok_s = K / wall
    status_timed = status_word()
    log(f"gated: {K} steps in {wall * 1e3:.1f} ms -> {tok_s:.1f} tokens/s; status word {status_timed:#x}")

    # gates of every (step, map): deterministic, written by every run
    slow = torch.stack([S_ for row in wl["outs"] for (_, _, S_) in row], dim=1).cpu().numpy()
    bytes_steps = [step_bytes(wl, slow[s]) for s in range(S)]
    proj_b = np.array([b[0] for b in bytes_steps], dtype=np.float64)
    apply_b = np.array([b[1] for b in bytes_steps], dtype=np.float64)
    idx = np.arange(K) % S
    total_bytes = float((proj_b[idx] + apply_b[idx]).sum())
    step_gbps = total_bytes / wall / 1e9
    step_b = proj_b[idx] + apply_b[idx]
    stack_gbps = float(step_b.mean() / t_launch / 1e9)
    log(f"stack_kernel mean over the timed region {t_launch * 1e6:.1f} us, {stack_gbps:.0f} GB/s")

    # ---- per-launch pass: HIP events around each gsi_stack on the launch stream ----
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        evs[i][0].record(stream)
        gsi.gsi_stack(plans[i % S], gsi.GATED, ws)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    t_stack = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    status_pass = status_word()
    log(f"per-launch events: stack_kernel mean {t_stack.mean() * 1e6:.1f} us, "
        f"{float(step_b.sum() / t_stack.sum() / 1e9):.0f} GB/s; status word {status_pass:#x}")
    two_launch = None
    if not chained:
        # the same steps as two launches (projection, then outputs): context
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for i in range(K):
            p = plans[i % S]
            evs[i][0].record(stream)
            gsi.gsi_stack_phase(p, gsi.GATED, gsi.PHASE_PROJECT, ws)
            evs[i][1].record(stream)
            gsi.gsi_stack_phase(p, gsi.GATED, gsi.PHASE_APPLY, ws)
            evs[i][2].record(stream)
        torch.cuda.synchronize()
        t_proj = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
        t_apply = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
        two_launch = {
            "us_per_step": float((t_proj + t_apply).mean() * 1e6),
            "proj_kernel": {"gbps": float(proj_b[idx].sum() / t_proj.sum() / 1e9),
                            "mean_us": float(t_proj.mean() * 1e6), "bytes_per_launch": float(proj_b[idx].mean())},
            "apply_kernel": {"gbps": float(apply_b[idx].sum() / t_apply.sum() / 1e9),
                             "mean_us": float(t_apply.mean() * 1e6), "bytes_per_launch": float(apply_b[idx].mean())},
        }
        log(f"two launches: {two_launch['us_per_step']:.1f} us per step (proj {t_proj.mean() * 1e6:.1f}, "
            f"apply {t_apply.mean() * 1e6:.1f})")

    # ---- dense baseline (same kernels, every token slow) and static projection ----
    D = max(1, args.dense_steps)
    for i in range(2):
        gsi.gsi_stack(plans[i % S], gsi.FORCE_SLOW, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(D):
        gsi.gsi_stack(plans[i % S], gsi.FORCE_SLOW, ws)
    torch.cuda.synchronize()
    dense_wall = time.perf_counter() - t0
    dense_tok_s = D / dense_wall
    dense_bytes = sum(call_bytes(mi, True) for row in wl["data"] for mi in row)
    t0 = time.perf_counter()
    for i in range(K):
        gsi.gsi_stack(plans[i % S], gsi.FORCE_FAST, ws)
    torch.cuda.synchronize()
    fast_wall = time.perf_counter() - t0
    fast_bytes = sum(call_bytes(mi, False) for row in wl["data"] for mi in row)
    # restore the gated outputs of the last steps (the forced runs overwrote them)
    for i in range(min(K, S)):
        gsi.gsi_stack(plans[i], gsi.GATED, ws)
    torch.cuda.synchronize()
    log(f"dense (forced slow): {dense_tok_s:.1f} tokens/s, {D * dense_bytes / dense_wall / 1e9:.0f} GB/s; "
        f"all-fast: {K / fast_wall:.1f} tokens/s, {K * fast_bytes / fast_wall / 1e9:.0f} GB/s")

    cpu = None
    if not args.no_cpu:
        cpu = with_single_thread(cpu_baseline_chained if chained else cpu_baseline, wl, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.3f} tokens/s on {cpu['cores']} threads, "
            f"{(cpu['single_thread'] or {}).get('value', float('nan')):.3f} on one ({cpu['model']})")

    maps_per_step = sum(len(r) for r in wl["data"])
    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}{' (shared bases)' if args.shared_bases else ''}"
                        f"{' (exact rho)' if args.exact_rho else ''}: "
                        f"{wl['layers']} layers x {len(wl['roles'])} maps "
                        f"({maps_per_step} gated batch-1 calls per step"
                        + (f" in {2 * wl['layers']} dependent waves" if chained else "") + "), "
                        f"{wl['rate'] * 100:.0f}% slow tokens" + (" at the first layer" if chained else " per map")
                        + ", eps=0.05",
            "layers": wl["layers"],
            "maps": [[n, d, o, k] for n, d, o, k in wl["roles"]],
            "distinct_steps": S,
            "timed_steps": K,
            # share of slow calls over the steps the timed region ran
            "slow_share": float(slow[idx].mean()),
        },
        "status": {"timed": status_timed, "per_launch_pass": status_pass},
        "hbm_gbps": step_gbps,
        "hbm_frac": step_gbps / PEAK_HBM_GBPS,
        "bytes_per_step": total_bytes / K,
        "roofline": {
            "bound": "hbm",
            "kernel": "stack_kernel",
            "achieved": stack_gbps,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": stack_gbps / PEAK_HBM_GBPS,
            "traffic": measured_traffic(args.workload + ("-shared" if args.shared_bases else "")
                                        + ("-exact" if args.exact_rho else ""),
                                        "stack_kernel"),
            "bytes_per_launch": float(step_b.mean()),
            "mean_launch_us": float(t_launch * 1e6),
            "per_launch_events_mean_us": float(t_stack.mean() * 1e6),
        },
        "two_launch": two_launch,
        "dense_tokens_per_s": dense_tok_s,
        "speedup_vs_dense": tok_s / dense_tok_s,
        "all_fast_tokens_per_s": K / fast_wall,
        "copy_gbps": copy_gbps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    if status_timed or status_pass:
        log("a device-side wait ran out during the run: the outputs were incomplete, the figures invalid")
        sys.exit(3)


if __name__ == "__main__":
    main()
