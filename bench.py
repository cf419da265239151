"""Benchmark of the owner-side Muon step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--precision P]

A step is one full muon_step over every batch of the workload (momentum,
normalisation, transpose-first, K Newton-Schulz steps, decay and update), with
all inputs resident in device memory; several batches are spread over
--streams streams (muon_step_batches).  Prints ONE JSON line with:

* value: Newton-Schulz TFLOP/s, counting 4 m^2 n + 2 m^3 flops per
  Newton-Schulz step per matrix (m <= n), divided by the full step time;
* ms_per_step: batched step latency;
* roofline: the dominant kernel (largest share of traced time), its
  algorithmic bytes (or flops) per launch over its average launch time,
  measured with HIP events recorded by the library on the launch stream
  (with batches on several streams a launch's time includes what it shares
  with the other lanes' kernels);
* cpu_baseline: the float64 CPU oracle timed on a bounded sample of the same
  workload on this host.
"""
from __future__ import annotations

import argparse
import dataclasses
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 (vector / MFMA)
SKINNY_MAX_ROWS = 32


def dsize(dtype: str) -> int:
    return 2 if dtype == "bf16" else 4


def kernel_model(name, count, M, N, prec, pdt, gdt, with_ns_out=False, ns_steps=5):
    """(bound, algorithmic quantity per launch, unit) of one kernel launch, or
    None if the kernel does not run on this batch's path.

    Bytes are what the kernel's function needs to move once (inputs read once,
    outputs written once); flops are the products the algorithm needs (the
    symmetric products counted on one triangle, diagonal included)."""
    m, n = min(M, N), max(M, N)
    E = count * m * n
    xs = 2 if prec == "bf16" else 4
    gs, ps = dsize(gdt), dsize(pdt)
    if m <= SKINNY_MAX_ROWS:
        L = 512 if prec == "bf16" else 256      # chunk widths of the split-K skinny kernels
        S = math.ceil(n / L)
        T = m * (m + 1) // 2
        part = count * S * T * 4
        if name == "sk_momentum_norm_gram":
            return "hbm", E * (gs + 4 + 4 + xs) + part + count * S * 4, "B"
        if name == "sk_ns_step":
            return "hbm", E * 2 * xs + 2 * part, "B"
        if name == "sk_bprime":
            return "hbm", part + count * 4096, "B"
        if name == "sk_gram_ns":
            return "hbm", part + count * S * 4 + count * 4096, "B"
        if name == "sk_apply_update":
            return "hbm", E * (xs + 2 * ps + (4 if with_ns_out else 0)), "B"
        if name == "sk_ns_apply_update":   # the partials once per matrix, then as sk_apply_update
            return "hbm", part + count * S * 4 + E * (xs + 2 * ps + (4 if with_ns_out else 0)), "B"
    else:
        if name == "tl_momentum_layout":
            # G read, M read and written, X written (bf16 operands unless f32),
            # X^T too unless the products use 256 x 256 tiles, the fp32 master
            ops = 4 if prec == "f32" else 2
            mp, np_ = -(-m // 128) * 128, -(-n // 128) * 128
            big = prec != "f32" and mp % 256 == 0 and np_ % 256 == 0
            return "hbm", E * (gs + 8) + E * (ops * (1 if big else 2) + (4 if prec == "bf16_x32" else 0)), "B"
        if name == "tl_gram":
            return "mfma", count * m * (m + 1) * n, "flop"
        if name == "tl_poly":
            return "mfma", count * m * m * (m + 1), "flop"
        if name in ("tl_apply", "tl_apply_update"):
            return "mfma", count * 2 * m * m * n, "flop"
        if name == "tl_norm_finalize":
            return "hbm", count * 4 * 1024, "B"
    return None


def kernel_form(b, skinny_kernel: int, prec: str) -> str:
    """Which kernels a batch runs: tiled products, Gram space in two launches
    (the iteration and the apply in one, for bf16 precision where W's stored
    rows are its long side, unless plan option 1 asks for three), Gram space
    in three launches, or step by step."""
    if b.path == 0:
        return "tiled"
    if b.path == 2:
        return "skinny_stepwise"
    two = skinny_kernel in (0, 3) and prec == "bf16" and b.M <= b.N
    return "skinny_gram_2launch" if two else "skinny_gram_3launch"


def executed_flops(plan, K: int) -> float:
    """Flops the kernels as built perform in one step (padding excluded):
    tiled products m(m+1)n (one triangle of the Gram), m^2(m+1) (one triangle of
    A^2) and 2m^2 n (apply) per step; the Gram-space skinny path one Gram m^2 n,
    four m x m products per step and one apply 2m^2 n; the step-by-step skinny
    path a Gram and an apply per step."""
    tot = 0.0
    for b in plan.batches:
        m, n = min(b.M, b.N), max(b.M, b.N)
        if b.path == 0:
            tot += b.count * K * (m * (m + 1) * n + m * m * (m + 1) + 2.0 * m * m * n)
        elif b.path == 1:
            tot += b.count * (m * m * n + K * 4 * 2.0 * m ** 3 + 2.0 * m * m * n)
        else:
            tot += b.count * K * (m * m * n + 2.0 * m ** 3 + 2.0 * m * m * n)
    return tot


def device_info() -> dict:
    import torch
    p = torch.cuda.get_device_properties(0)
    info = {"name": torch.cuda.get_device_name(0), "compute_units": getattr(p, "multi_processor_count", None),
            "arch": getattr(p, "gcnArchName", None), "l2_bytes": getattr(p, "L2_cache_size", None),
            "total_memory": getattr(p, "total_memory", None)}
    clk = getattr(p, "clock_rate", None)
    if clk:
        info["clock_khz"] = clk
    return info


def kernel_sources_sha256(files=None):
    """Hash of the code in the HIP/C++ sources the kernels are built from:
    comments are removed and whitespace runs collapsed first, so an edit that
    touches only comments or layout keeps counter summaries valid.  With
    `files`, a dict {file: hash} over just those files; else one hash over
    all of them."""
    import hashlib
    import re
    d = os.path.join(ROOT, "matrix_optimizer_amd", "csrc")

    def code(f):
        with open(os.path.join(d, f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        return " ".join(src.split()).encode()

    if files is not None:
        return {f: hashlib.sha256(code(f)).hexdigest() for f in files}
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            h.update(code(f))
    return h.hexdigest()


# source files whose code decides each traced kernel's memory traffic
KERNEL_SOURCES = {"sk_": ["common.h", "internal.h", "skinny.hip"], "tl_": ["common.h", "internal.h", "tiled.hip"]}


def kernel_source_files(kernel: str):
    for prefix, files in KERNEL_SOURCES.items():
        if kernel.startswith(prefix):
            return files
    return None


def measured_traffic(workload: str, kernel: str, prec: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current code of the kernel's sources
    (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{prec}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    recorded = rec.get("sources_sha256")
    if not isinstance(recorded, dict) or not recorded:
        return None
    files = kernel_source_files(kernel)
    if files is None or any(f not in recorded for f in files):
        return None
    if kernel_sources_sha256(files) != {f: recorded[f] for f in files}:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["bytes_per_launch"]


def make_device_batches(wl, plan, dtype, reuse_shapes: bool):
    """Per-batch device buffers from the seeded generator.  With reuse_shapes,
    batches of identical [count, M, N] get copies of the first one's data."""
    import torch
    from tests import harness as H
    cache = {}
    out = []
    for b in plan.batches:
        key = (b.count, b.M, b.N)
        if reuse_shapes and key in cache:
            src = cache[key]
            out.append({k: v.clone() for k, v in src.items()})
            continue
        arrays = H.batch_arrays(wl, b)
        dev = {"param": H.to_device(arrays["param"], dtype), "grad": H.to_device(arrays["grad"], dtype),
               "momentum": H.to_device(arrays["momentum"], "f32")}
        del arrays
        if reuse_shapes:
            cache[key] = dev
        out.append(dev)
    return out


def make_device_batches_gpu(wl, plan, dtype, seed=0):
    """Per-batch device buffers drawn on the GPU with seeded torch generators,
    following the workload's recipes (for large workloads, where drawing on
    the host would take minutes).  Not the generator the parity tests use."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = []
    for b in plan.batches:
        g = torch.Generator(device="cuda").manual_seed(seed * 100003 + b.index)
        shp = (b.count, b.M, b.N)
        p = (torch.randn(shp, generator=g, device="cuda") * 0.02).to(tdt)
        if wl.grad_recipe == "normal":
            gr = torch.randn(shp, generator=g, device="cuda") * wl.grad_scale
        elif wl.grad_recipe == "row_scaled":
            r = torch.exp(torch.empty((b.count, b.M, 1), device="cuda").uniform_(
                math.log(0.1), math.log(10.0), generator=g))
            gr = torch.randn(shp, generator=g, device="cuda") * wl.grad_scale * r
        else:
            U = torch.randn((b.count, b.M, 64), generator=g, device="cuda")
            V = torch.randn((b.count, b.N, 64), generator=g, device="cuda")
            gr = torch.bmm(U, V.transpose(1, 2).contiguous()) + 0.1 * torch.randn(shp, generator=g, device="cuda")
            del U, V
        gr = gr.to(tdt)
        if wl.momentum_recipe == "zeros":
            mom = torch.zeros(shp, dtype=torch.float32, device="cuda")
        else:
            mom = torch.randn(shp, generator=g, device="cuda")
        out.append({"param": p, "grad": gr, "momentum": mom})
        torch.cuda.synchronize()
    return out


def cpu_baseline(wl, plan, dtype, hp, budget_s=12.0, max_matrices=None):
    """Time the float64 oracle on this host on a bounded sample of the workload."""
    from oracle import muon_oracle as ORC
    from tests import harness as H
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    kw = None
    flops = 0.0
    t0 = time.perf_counter()
    done = 0
    reps = 0
    samples = []
    for b in plan.batches:
        ids = H.matrix_ids(b)
        take = ids if max_matrices is None else ids[:max_matrices]
        for (pi, mi) in take:
            samples.append((b, pi, mi))
    # decode the sample once, then run the oracle until the budget is used
    data = []
    for (b, pi, mi) in samples:
        W = H.decode(wl.matrix(pi, mi, "param"))
        G = H.decode(wl.matrix(pi, mi, "grad"))
        Mo = wl.matrix(pi, mi, "momentum").astype(np.float64)
        data.append((b, W, G, Mo))
        if max_matrices is not None and len(data) >= max_matrices:
            break
    # a full step on one very large matrix can take minutes here: then time the
    # oracle's momentum + one Newton-Schulz step of it instead (same arithmetic)
    b0 = data[0][0]
    m0, n0 = min(b0.M, b0.N), max(b0.M, b0.N)
    est = hp.ns_steps * (4.0 * m0 * m0 * n0 + 2.0 * m0 ** 3) / 0.3e12
    steps = hp.ns_steps if est <= 2.5 * budget_s else 1
    t0 = time.perf_counter()
    while True:
        for (b, W, G, Mo) in data:
            kw = H.oracle_kwargs(hp, b.M, b.N)
            kw["ns_steps"] = steps
            if steps != hp.ns_steps:
                kw["coeffs"] = kw["coeffs"][:3]
            ORC.muon_step_matrix(W, G, Mo, **kw)
            m, n = min(b.M, b.N), max(b.M, b.N)
            flops += steps * (4.0 * m * m * n + 2.0 * m ** 3)
            done += 1
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(data)} matrices of the workload x {reps} repetitions ({done} oracle steps of "
                      f"{steps} Newton-Schulz iterations, {el:.1f} s, float64 NumPy)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="fused_74x24x10240")
    ap.add_argument("--precision", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="accepted for older profile commands; the 512 MiB reference copy always runs")
    ap.add_argument("--launch", choices=["graph", "eager"], default="eager",
                    help="timed steps as eager muon_step calls (default) or replays of one captured HIP graph")
    ap.add_argument("--skinny-kernel", type=int, default=0,
                    help="short sides <= 32: 0 or 1 Newton-Schulz in Gram space, 2 step by step")
    ap.add_argument("--device-inputs", action="store_true",
                    help="draw the inputs on the GPU with seeded torch generators (large workloads)")
    ap.add_argument("--streams", type=int, default=2,
                    help="spread the batches of a step over this many streams (muon_step_batches; at most the "
                         "number of batches; 1 = the batches in plan order on one stream)")
    ap.add_argument("--reuse-shapes", action="store_true",
                    help="batches of identical shape share generated input values (copied per batch)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the step would shard by whole matrices, one owner GPU per matrix).", file=sys.stderr)
        sys.exit(2)

    import torch
    from matrix_optimizer_amd import binding as B
    from matrix_optimizer_amd import workloads as WL
    from tests import harness as H

    wl = WL.WORKLOADS[args.workload]
    prec = args.precision or wl.hp.precision
    dtype = wl.params[0].dtype
    hp = H.c_hparams(wl.hp, precision=prec)
    torch.cuda.set_device(0)
    plan = B.Plan([p.shape for p in wl.params], skinny_kernel=args.skinny_kernel)
    if args.device_inputs:
        bufs = make_device_batches_gpu(wl, plan, dtype)
    else:
        bufs = make_device_batches(wl, plan, dtype, args.reuse_shapes)
    stream = torch.cuda.current_stream()
    # lr and decay from device scalars, so a captured step needs no recapture
    lr_wd = torch.tensor([hp.lr, hp.weight_decay], dtype=torch.float32, device="cuda")
    hp_run = dataclasses.replace(hp, lr_wd=lr_wd)
    nstreams = max(1, min(args.streams, len(plan.batches)))
    bidx = [b.index for b in plan.batches]
    lane_of, lane_ws = B.plan_lanes(plan, bidx, hp_run, nstreams)
    wss = [torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None for n in lane_ws]
    side = [torch.cuda.Stream() for _ in range(nstreams - 1)]
    step_bufs = [(bufs[i]["param"], bufs[i]["grad"], bufs[i]["momentum"]) for i in bidx]

    def step():
        # the caller's part on the current stream (the capture stream while a
        # graph is recorded), the other lanes on side streams
        if nstreams == 1:
            for b in plan.batches:
                d = bufs[b.index]
                B.muon_step(plan, b.index, d["param"], d["grad"], d["momentum"], hp_run, wss[0])
        else:
            B.muon_step_batches(plan, bidx, step_bufs, hp_run, wss, [None] + [s.cuda_stream for s in side])

    # eager timing: the same calls with their arguments marshalled once, so the
    # host enqueues a step well inside the GPU's time for it
    if nstreams == 1:
        prepared = [B.PreparedStep(plan, b.index, step_bufs[i], hp_run, wss[0], stream.cuda_stream)
                    for i, b in enumerate(plan.batches)]
    else:
        prepared = [B.PreparedStep(plan, bidx, step_bufs, hp_run, wss,
                                   [stream.cuda_stream] + [s.cuda_stream for s in side])]

    def step_prepared():
        for call in prepared:
            call()

    for _ in range(args.warmup):
        step_prepared()
    torch.cuda.synchronize()
    run = step_prepared
    if args.launch == "graph":
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                step()
        stream.wait_stream(side)
        run = graph.replay
        run()   # one untimed replay
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gc.disable()   # no collector pause inside the timed region
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    gc.enable()
    ms = e0.elapsed_time(e1) / args.steps

    # per-kernel times: a second pass of the same K steps with library launch tracing
    launches = 0
    for b in plan.batches:
        launches += 64
    B.muon_trace_start(args.steps * launches + 16)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step_prepared()
    t1.record(stream)
    torch.cuda.synchronize()
    traced_ms = t0.elapsed_time(t1) / args.steps
    recs = B.muon_trace_stop()
    per = {}
    for name, t in recs:
        per.setdefault(name, []).append(t)
    kernels = {k: {"launches_per_step": len(v) / args.steps, "avg_ms": float(np.mean(v)),
                   "total_ms_per_step": float(np.sum(v)) / args.steps} for k, v in per.items()}
    dom = max(kernels, key=lambda k: kernels[k]["total_ms_per_step"])
    # algorithmic quantity of one launch of the dominant kernel, averaged over the
    # batches it runs on (its launches per batch per step follow from the path)
    qty = 0.0
    nlaunch = 0
    bound, unit = "hbm", "B"
    for b in plan.batches:
        res = kernel_model(dom, b.count, b.M, b.N, prec, dtype, dtype, ns_steps=hp.ns_steps)
        if res is None:
            continue
        bd, q, u = res
        per_batch = {"sk_ns_step": hp.ns_steps - 1, "sk_bprime": hp.ns_steps, "tl_gram": hp.ns_steps,
                     "tl_poly": hp.ns_steps, "tl_apply": hp.ns_steps - 1}.get(dom, 1)
        qty += q * per_batch
        nlaunch += per_batch
        bound, unit = bd, u
    qty_per_launch = qty / max(nlaunch, 1)
    avg_s = kernels[dom]["avg_ms"] / 1e3
    if bound == "hbm":
        achieved = qty_per_launch / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": None}
    else:
        achieved = qty_per_launch / avg_s / 1e12
        peak = FP32_PEAK_TFLOPS if prec == "f32" else BF16_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None}
    roof["traffic"] = measured_traffic(wl.name, dom, prec)
    roof["kernel"] = dom
    roof["avg_launch_ms"] = kernels[dom]["avg_ms"]
    roof["algorithmic_per_launch"] = qty_per_launch
    roof["algorithmic_unit"] = "bytes" if unit == "B" else "flops"

    flops = wl.nominal_ns_flops()
    if hp.ns_steps != wl.hp.ns_steps:
        flops = flops / wl.hp.ns_steps * hp.ns_steps
    value = flops / (ms / 1e3) / 1e12
    cfg = {"workload": wl.name, "matrices": int(sum(b.count for b in plan.batches)), "launch": args.launch,
           "streams": nstreams, "lanes": lane_of,
           "batches": [[b.count, b.M, b.N] for b in plan.batches],
           "kernels": [kernel_form(b, args.skinny_kernel, prec) for b in plan.batches],
           "param_dtype": dtype,
           "precision": prec, "ns_steps": hp.ns_steps, "coeffs": list(hp.coeffs),
           "inputs": ("seeded synthetic, drawn on the GPU (torch generators)" if args.device_inputs else
                      "seeded synthetic" + (", same-shape batches share values" if args.reuse_shapes else ""))}
    out = {"metric": "Muon-step NS TFLOP/s (bf16 MFMA)", "value": value, "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if prec != "f32" else "f32",
           "data": "synthetic", "config": cfg, "roofline": roof,
           "detail": {"ns_frac_of_bf16_peak": value / BF16_PEAK_TFLOPS, "traced_ms_per_step": traced_ms,
                      "executed_tflop_per_step": executed_flops(plan, hp.ns_steps) / 1e12,
                      "nominal_tflop_per_step": flops / 1e12,
                      "kernels": kernels, "device": device_info()}}

    # plain device copy of known size (512 MiB read + 512 MiB written): the
    # measured bandwidth the HBM roofline is also quoted against, and the
    # reference for the HBM byte counters
    src = torch.empty(1 << 29, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        dst.copy_(src)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    ms_copy = c0.elapsed_time(c1) / 5
    copy_gbps = 2 * (1 << 29) / (ms_copy / 1e3) / 1e9
    out["detail"]["copy"] = {"bytes_read": 1 << 29, "bytes_written": 1 << 29, "avg_ms": ms_copy, "GBps": copy_gbps}
    if roof["bound"] == "hbm":
        roof["frac_of_measured_copy"] = roof["achieved"] / copy_gbps

    if ms < 20.0:
        # cold steps: reading 1 GiB between steps evicts the 256 MB Infinity
        # Cache with clean lines, so each timed step starts from HBM (the warm
        # value above may be served partly from that cache) and pays for no
        # write-back of someone else's data
        cold = []
        flush = torch.cat([src.view(torch.int32), dst.view(torch.int32)])
        for _ in range(min(args.steps, 10)):
            flush.sum()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            step_prepared()
            a1.record(stream)
            torch.cuda.synchronize()
            cold.append(a0.elapsed_time(a1))
        out["detail"]["cold_ms_per_step"] = float(np.median(cold))
        out["detail"]["cold_tflops"] = flops / (np.median(cold) / 1e3) / 1e12
    del src, dst
    flush = None
    if not args.no_cpu_baseline:
        maxm = None if min(wl.params[0].matrix_shape) <= SKINNY_MAX_ROWS else 1
        out["cpu_baseline"] = cpu_baseline(wl, plan, dtype, hp, args.cpu_budget, maxm)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
