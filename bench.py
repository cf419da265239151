"""Benchmark of the owner-side Muon step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--precision P]

A step is one full Muon step over every batch of the workload (momentum,
normalisation, transpose-first, K Newton-Schulz steps, decay and update), with
all inputs resident in device memory; the batches are spread over --streams
streams (muon_step_batches).  The default workload is the largest one that
fits one GPU: 16 bf16 matrices of 8192 x 28672 plus 16 of 28672 x 8192, in 16
batches of two, with a master copy of X (bf16_x32: bf16 plus a bf16 residue).

Protocol (the DMuon-2 paper's timing, App. D.3): W untimed repetitions, then
K timed ones; before each, W and M are restored from device copies (outside
the timed events), so every repetition runs the same step on the same
values; each repetition is timed between HIP events on the caller's stream
and ms_per_step is their median.  The first timed repetition's W' and M' are
checked against the float64 oracle: at the sampled positions the oracle's
values were stored for (tests/golden/), or against the oracle run of the
cpu_baseline leg on the same matrices.  Prints ONE JSON line with:

* value: Newton-Schulz TFLOP/s, counting 4 m^2 n + 2 m^3 flops per
  Newton-Schulz step per matrix (m <= n), divided by the full step time;
  detail.executed_tflops counts the flops the kernels perform (symmetric
  products on one triangle);
* ms_per_step: batched step latency (median over the timed repetitions);
* roofline: the dominant kernel (largest share of traced time) of a pass on
  one stream, its algorithmic bytes (or flops) per launch over its average
  launch time, from HIP events the library records at the kernel's start and
  end;
* cpu_baseline: the float64 CPU oracle timed on a bounded sample of the same
  workload on this host (for the 8192 x 28672 matrices one Newton-Schulz
  iteration of one matrix, extrapolated).
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
            # X^T too unless the products use 256 x 256 tiles, the master's bf16 residue
            ops = 4 if prec == "f32" else 2
            mp, np_ = -(-m // 128) * 128, -(-n // 128) * 128
            big = prec != "f32" and mp % 256 == 0 and np_ % 256 == 0
            return "hbm", E * (gs + 8) + E * (ops * (1 if big else 2) + (2 if prec in ("bf16_x32", "bf16_x32c") else 0)), "B"
        if name == "tl_gram":
            return "mfma", count * m * (m + 1) * n, "flop"
        if name == "tl_poly":
            return "mfma", count * m * m * (m + 1), "flop"
        if name in ("tl_apply", "tl_apply_update"):   # compensated: B X~ and B R in one launch
            return "mfma", count * 2 * m * m * n * (2 if prec == "bf16_x32c" and m >= 128 else 1), "flop"
        if name == "tl_norm_finalize":
            return "hbm", count * 4 * 1024, "B"
    return None


def kernel_form(b, skinny_kernel: int, prec: str) -> str:
    """Which kernels a batch runs: tiled products, Gram space in two launches
    (the iteration and the apply in one, unless plan option 1 asks for
    three), Gram space in three launches, or step by step."""
    if b.path == 0:
        return "tiled"
    if b.path == 2:
        return "skinny_stepwise"
    return "skinny_gram_2launch" if skinny_kernel in (0, 3) else "skinny_gram_3launch"


def executed_flops(plan, K: int, prec: str = "bf16") -> float:
    """Flops the kernels as built perform in one step (padding excluded):
    tiled products m(m+1)n (one triangle of the Gram), m^2(m+1) (one triangle of
    A^2) and 2m^2 n (apply, twice in the compensated mode) per step; the
    Gram-space skinny path one Gram m^2 n, four m x m products per step and one
    apply 2m^2 n; the step-by-step skinny path a Gram and an apply per step."""
    tot = 0.0
    for b in plan.batches:
        m, n = min(b.M, b.N), max(b.M, b.N)
        if b.path == 0:
            napply = 2 if prec == "bf16_x32c" and m >= 128 else 1
            tot += b.count * K * (m * (m + 1) * n + m * m * (m + 1) + napply * 2.0 * m * m * n)
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
    the host would take minutes).  Not the generator the parity tests use:
    the matrices the bench checks are redrawn with it afterwards
    (put_host_matrices)."""
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


def locate(plan, pi: int, mi: int):
    """(batch, position in the batch) of matrix mi of parameter pi."""
    for b in plan.batches:
        for (p, first, num, off) in b.segments:
            if p == pi and first <= mi < first + num:
                return b, off // (b.M * b.N) + mi - first
    raise KeyError((pi, mi))


def put_host_matrices(wl, plan, bufs, ids, dtype):
    """Overwrite matrices `ids` [(param, matrix)] of device-drawn buffers with
    the seeded host generator's values (the parity tests' inputs), drawn in
    threads.  Returns {(param, matrix): stored host arrays}."""
    from concurrent.futures import ThreadPoolExecutor
    from tests import harness as H
    jobs = [(pi, mi, kind) for (pi, mi) in ids for kind in ("param", "grad", "momentum")]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        mats = list(ex.map(lambda j: wl.matrix(*j), jobs))
    host = {}
    for (pi, mi, kind), arr in zip(jobs, mats):
        host.setdefault((pi, mi), {})[kind] = arr
        b, q = locate(plan, pi, mi)
        bufs[b.index][kind][q].copy_(H.to_device(arr, "f32" if kind == "momentum" else dtype))
    return host


def blas_info():
    """(threads, description) of the BLAS library NumPy calls."""
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:
        info = []
    if not info:
        return os.cpu_count() or 1, "unknown"
    i = info[0]
    return int(i.get("num_threads", 1)), f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')})"


def cpu_baseline(wl, plan, hp, samples, budget_s=12.0):
    """Time the float64 oracle on this host on a bounded sample of the workload.

    samples: [(param, matrix)].  Each sampled matrix runs the oracle's full
    step, or, where a full step would take minutes (the 8192 x 28672
    matrices), its momentum and one Newton-Schulz iteration, whose rate then
    stands for the whole step's (labelled extrapolated).  Repeats until the
    budget is spent.  Returns (record, refs): refs maps each matrix that ran
    the full step to the oracle's W', M' and O (first repetition), for checking
    the GPU's timed result."""
    from oracle import muon_oracle as ORC
    from tests import harness as H
    threads, blas = blas_info()
    data = []
    for (pi, mi) in samples:
        W = H.decode(wl.matrix(pi, mi, "param"))
        G = H.decode(wl.matrix(pi, mi, "grad"))
        Mo = wl.matrix(pi, mi, "momentum").astype(np.float64)
        data.append(((pi, mi), wl.params[pi].matrix_shape, W, G, Mo))
    (M0, N0) = data[0][1]
    m0, n0 = min(M0, N0), max(M0, N0)
    est = hp.ns_steps * (4.0 * m0 * m0 * n0 + 2.0 * m0 ** 3) / 0.3e12
    steps = hp.ns_steps if est <= 2.5 * budget_s else 1
    refs = {}
    flops = 0.0
    done = reps = 0
    t0 = time.perf_counter()
    while True:
        for (key, (M, N), W, G, Mo) in data:
            kw = H.oracle_kwargs(hp, M, N)
            kw["ns_steps"] = steps
            if steps != hp.ns_steps:
                kw["coeffs"] = kw["coeffs"][:3]
            r = ORC.muon_step_matrix(W, G, Mo, **kw)
            if reps == 0 and steps == hp.ns_steps:
                refs[key] = {"W": r["W"], "M": r["M"], "O": r["O"]}
            m, n = min(M, N), max(M, N)
            flops += steps * (4.0 * m * m * n + 2.0 * m ** 3)
            done += 1
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    what = (f"{len(data)} matrices of the workload x {reps} repetitions ({done} oracle steps of {steps} "
            f"Newton-Schulz iterations, {el:.1f} s, float64 NumPy)")
    rec = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": what, "blas": blas, "host_cpus": os.cpu_count(),
           "extrapolated": steps != hp.ns_steps}
    if steps != hp.ns_steps:
        rec["sample"] = ("extrapolated: " + what + f"; the rate of momentum plus one of the {hp.ns_steps} "
                         "iterations on that matrix stands for the whole step")
        rec["full_step_s_extrapolated"] = wl.nominal_ns_flops() / (flops / el) if flops else None
    return rec, refs


GOLDEN = {"large_8192x28672": os.path.join(ROOT, "tests", "golden", "large_8192x28672_samples.npz")}


def check_plan(wl, plan):
    """Matrices whose timed results are checked, and their reference:
    ("golden", npz) -- oracle values stored at sampled positions -- or
    ("oracle", None) -- the cpu_baseline leg's oracle results on the same
    matrices (all matrices of skinny batches, the first matrix of each
    distinct tiled batch shape)."""
    if wl.name in GOLDEN and os.path.exists(GOLDEN[wl.name]):
        gold = np.load(GOLDEN[wl.name])
        meta = json.loads(str(gold["meta"]))
        return [(pi, meta["matrix"]) for pi in meta["params"]], ("golden", gold)
    ids, seen = [], set()
    for b in plan.batches:
        mats = [(pi, first + q) for (pi, first, num, off) in b.segments for q in range(num)]
        if min(b.M, b.N) <= SKINNY_MAX_ROWS:
            ids += mats
        elif (b.M, b.N) not in seen:
            ids.append(mats[0])
        seen.add((b.M, b.N))
    return ids, ("oracle", None)


def snapshot(plan, bufs, ids, ref, o_bufs=None):
    """Device copies of W' and M' (and O, from o_bufs {batch: [count, M, N]})
    of the checked matrices, at the golden positions or whole, taken on the
    current stream right after a step."""
    import torch
    snap = {}
    for (pi, mi) in ids:
        b, q = locate(plan, pi, mi)
        ts = [bufs[b.index]["param"][q], bufs[b.index]["momentum"][q]]
        if o_bufs is not None:
            ts.append(o_bufs[b.index][q])
        if ref[0] == "golden":
            gold = ref[1]
            idx = torch.from_numpy(gold[f"p{pi}_rows"] * b.N + gold[f"p{pi}_cols"]).to("cuda")
            snap[(pi, mi)] = tuple(t.reshape(-1).index_select(0, idx) for t in ts)
        else:
            snap[(pi, mi)] = tuple(t.clone() for t in ts)
    return snap


def check_result(wl, plan, hp, snap, snap_o, host, ref, refs):
    """The timed step's result against the oracle.

    snap: W' and M' of the first timed repetition; snap_o: W', M' and O of
    the same batches stepped once more (untimed, from the same restored
    inputs) with O written out.  Checks: that repetition's W' and M' are
    bitwise those of the timed one (the step is deterministic, so O is the
    timed step's O); O within the relative Frobenius bound (3e-2 bf16 modes,
    1e-5 fp32); M' elementwise within 1e-6 (|mu M| + |G|); W' - W within the
    O bound plus the bf16 rounding of the stored W' (dW_allowed: that bound plus
    the half-ulp rounding of W' relative to the size of dW, per matrix)."""
    from tests import harness as H
    out = {"reference": ref[0], "matrices": 0, "max_O_error": 0.0, "max_dW_error": 0.0,
           "bound": H.o_tolerance(hp.precision), "per_matrix": [], "bitwise_as_timed": True,
           "momentum_ok": True, "ok": True}
    for (pi, mi), (Wd, Md) in snap.items():
        Wo, Mo_, Od = snap_o[(pi, mi)]
        arr = host[(pi, mi)]
        if ref[0] == "golden":
            gold = ref[1]
            rows, cols = gold[f"p{pi}_rows"], gold[f"p{pi}_cols"]
            W0 = H.decode(arr["param"][rows, cols])
            G = H.decode(arr["grad"][rows, cols])
            M0 = arr["momentum"][rows, cols].astype(np.float64)
            Wref, Oref = gold[f"p{pi}_W"], gold[f"p{pi}_O"]
        else:
            if (pi, mi) not in refs:
                continue
            W0, G = H.decode(arr["param"]), H.decode(arr["grad"])
            M0 = arr["momentum"].astype(np.float64)
            Wref, Oref = refs[(pi, mi)]["W"], refs[(pi, mi)]["O"]
        Wg, Mg, Og = H.to_host(Wd), H.to_host(Md), H.to_host(Od)
        if not (np.array_equal(Wg, H.to_host(Wo)) and np.array_equal(Mg, H.to_host(Mo_))):
            out["bitwise_as_timed"] = False
        try:
            H.check_momentum(Mg, M0, G, H.f32(hp.momentum))
        except AssertionError:
            out["momentum_ok"] = False
        eo = H.rel_fro(Og.astype(np.float64), Oref)
        dW_ref = Wref - W0
        half_ulp = 0.0
        if Wg.dtype == np.uint16:
            half_ulp = np.linalg.norm(2.0 ** (np.floor(np.log2(np.maximum(np.abs(Wref), 1e-38))) - 8))
        nref = np.linalg.norm(dW_ref)
        e = H.rel_fro(H.decode(Wg) - W0, dW_ref)
        slack = half_ulp / nref if nref > 0 else 0.0
        out["max_O_error"] = max(out["max_O_error"], eo)
        out["max_dW_error"] = max(out["max_dW_error"], e)
        out["matrices"] += 1
        out["per_matrix"].append({"matrix": [int(pi), int(mi)], "O_error": float(eo), "dW_error": float(e),
                                  "dW_allowed": float(out["bound"] + slack + 1e-6)})
        if not (np.all(np.isfinite(Og)) and eo <= out["bound"] and e <= out["bound"] + slack + 1e-6):
            out["ok"] = False
    out["ok"] = bool(out["ok"] and out["momentum_ok"] and out["bitwise_as_timed"] and out["matrices"] > 0)
    if ref[0] == "golden":
        out["positions_per_matrix"] = int(len(ref[1][f"p{next(iter(snap))[0]}_rows"]))
    return out


def progress(msg: str) -> None:
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30, help="timed repetitions of the step")
    ap.add_argument("--warmup", type=int, default=20, help="untimed repetitions before them")
    ap.add_argument("--workload", default="large_8192x28672")
    ap.add_argument("--precision", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="accepted for older profile commands; the 512 MiB reference copy always runs")
    ap.add_argument("--launch", choices=["graph", "eager"], default="eager",
                    help="timed steps as eager muon_step calls (default) or replays of one captured HIP graph")
    ap.add_argument("--skinny-kernel", type=int, default=0,
                    help="short sides <= 32: 0 or 1 Newton-Schulz in Gram space, 2 step by step")
    ap.add_argument("--inputs", choices=["auto", "host", "device"], default="auto",
                    help="host: every matrix from the seeded host generator; device: drawn on the GPU with "
                         "seeded torch generators, the checked matrices from the host generator; auto: device "
                         "above 2^28 elements")
    ap.add_argument("--device-inputs", action="store_true", help="same as --inputs device")
    ap.add_argument("--max-batch-elems", type=int, default=0,
                    help="plan cap on elements per batch (0: the library default, 2^29)")
    ap.add_argument("--streams", type=int, default=2,
                    help="spread the batches of a step over this many streams (muon_step_batches; at most the "
                         "number of batches; 1 = the batches in plan order on one stream)")
    ap.add_argument("--trace-steps", type=int, default=0,
                    help="steps of the one-stream traced pass (0: enough for about 2 s, at most --steps)")
    ap.add_argument("--reuse-shapes", action="store_true",
                    help="host inputs: batches of identical shape share generated values (copied per batch)")
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
    plan = B.Plan([p.shape for p in wl.params], max_batch_elems=args.max_batch_elems,
                  skinny_kernel=args.skinny_kernel)
    inputs = "device" if args.device_inputs else args.inputs
    if inputs == "auto":
        inputs = "device" if wl.num_elements() > (1 << 28) else "host"
    check_ids, ref = check_plan(wl, plan)
    if inputs == "device":
        bufs = make_device_batches_gpu(wl, plan, dtype)
        host = put_host_matrices(wl, plan, bufs, check_ids, dtype)
    else:
        bufs = make_device_batches(wl, plan, dtype, args.reuse_shapes)
        host = {(pi, mi): {k: wl.matrix(pi, mi, k) for k in ("param", "grad", "momentum")} for (pi, mi) in check_ids}
    torch.cuda.synchronize()
    progress(f"inputs ready ({inputs}; {len(plan.batches)} batches, {len(check_ids)} checked matrices)")
    # pristine copies: every repetition starts from the same W and M
    pristine = [{"param": d["param"].clone(), "momentum": d["momentum"].clone()} for d in bufs]
    stream = torch.cuda.current_stream()

    def restore():
        for d, p in zip(bufs, pristine):
            d["param"].copy_(p["param"])
            d["momentum"].copy_(p["momentum"])

    # lr and decay from device scalars, so a captured step needs no recapture
    lr_wd = torch.tensor([hp.lr, hp.weight_decay], dtype=torch.float32, device="cuda")
    hp_run = dataclasses.replace(hp, lr_wd=lr_wd)
    nstreams = max(1, min(args.streams, len(plan.batches)))
    bidx = [b.index for b in plan.batches]
    lane_of, lane_ws = B.plan_lanes(plan, bidx, hp_run, nstreams)
    wss = [torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None for n in lane_ws]
    side = [torch.cuda.Stream() for _ in range(nstreams - 1)]
    step_bufs = [(bufs[i]["param"], bufs[i]["grad"], bufs[i]["momentum"]) for i in bidx]

    # the step as deployed: every batch, its arguments marshalled once
    # (muon_step per batch on one stream, or muon_step_batches over lanes)
    if nstreams == 1:
        prepared = [B.PreparedStep(plan, b.index, step_bufs[i], hp_run, wss[0], stream.cuda_stream)
                    for i, b in enumerate(plan.batches)]
    else:
        prepared = [B.PreparedStep(plan, bidx, step_bufs, hp_run, wss,
                                   [stream.cuda_stream] + [s.cuda_stream for s in side])]

    def step_prepared():
        for call in prepared:
            call()

    run = step_prepared
    if args.launch == "graph":
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                if nstreams == 1:
                    for b in plan.batches:
                        d = bufs[b.index]
                        B.muon_step(plan, b.index, d["param"], d["grad"], d["momentum"], hp_run, wss[0])
                else:
                    B.muon_step_batches(plan, bidx, step_bufs, hp_run, wss, [None] + [s.cuda_stream for s in side])
        stream.wait_stream(cap)
        run = graph.replay

    for _ in range(args.warmup):
        restore()
        run()
    torch.cuda.synchronize()
    progress(f"{args.warmup} warm-up repetitions done")

    # timed repetitions: W and M restored before each (outside the events),
    # the step between two events on the caller's stream (which the other
    # lanes join); the first repetition's W' and M' are kept for the check
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    snap = None
    torch.cuda.synchronize()
    gc.disable()   # no collector pause inside the timed region
    w0 = time.perf_counter()
    for r in range(args.steps):
        restore()
        ev[r][0].record(stream)
        run()
        ev[r][1].record(stream)
        if r == 0:
            snap = snapshot(plan, bufs, check_ids, ref)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gc.enable()
    per_rep = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.median(per_rep))
    del ev
    progress(f"{args.steps} timed repetitions: median {ms:.4f} ms")

    # the checked batches once more, untimed, from the same restored inputs,
    # with O written out (the deployed step writes none)
    restore()
    o_bufs = {}
    for (pi, mi) in check_ids:
        b, q = locate(plan, pi, mi)
        if b.index in o_bufs:
            continue
        o_bufs[b.index] = torch.empty((b.count, b.M, b.N), dtype=torch.float32, device="cuda")
        d = bufs[b.index]
        ws = wss[lane_of[bidx.index(b.index)]] if nstreams > 1 else wss[0]
        B.muon_step(plan, b.index, d["param"], d["grad"], d["momentum"], hp_run, ws, ns_out=o_bufs[b.index])
    snap_o = snapshot(plan, bufs, check_ids, ref, o_bufs)
    torch.cuda.synchronize()
    del o_bufs

    # per-kernel times: a pass on one stream (plan order) with library launch
    # tracing, so each launch's time is its own and not shared with a lane;
    # the steps run back to back on the evolving values (no restore: its
    # copies would leave dirty lines whose write-back competes with the
    # kernels, and the kernels' time does not depend on the values)
    one = [B.PreparedStep(plan, b.index, step_bufs[i], hp_run, wss[lane_of[i]] if nstreams > 1 else wss[0],
                          stream.cuda_stream) for i, b in enumerate(plan.batches)]
    tsteps = args.trace_steps or max(1, min(args.steps, int(math.ceil(2000.0 / max(ms, 1e-3)))))
    B.muon_trace_start(tsteps * 64 * len(plan.batches) + 16)
    tr = []
    for _ in range(tsteps):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for call in one:
            call()
        t1.record(stream)
        tr.append((t0, t1))
    torch.cuda.synchronize()
    traced_ms = float(np.median([a.elapsed_time(b) for a, b in tr]))
    recs = B.muon_trace_stop()
    progress(f"one-stream traced pass: {tsteps} steps, {traced_ms:.4f} ms per step")
    per = {}
    for name, t in recs:
        per.setdefault(name, []).append(t)
    kernels = {k: {"launches_per_step": len(v) / tsteps, "avg_ms": float(np.mean(v)),
                   "total_ms_per_step": float(np.sum(v)) / tsteps} for k, v in per.items()}
    dom = max(kernels, key=lambda k: kernels[k]["total_ms_per_step"])

    def per_launch(kname):
        """(bound, algorithmic quantity of one launch, unit) of a traced kernel,
        averaged over the batches it runs on (its launches per batch per step
        follow from the path), or None without a model."""
        qty, nl, bd, u = 0.0, 0, None, None
        for b in plan.batches:
            res = kernel_model(kname, b.count, b.M, b.N, prec, dtype, dtype, ns_steps=hp.ns_steps)
            if res is None:
                continue
            bd, q, u = res
            per_batch = {"sk_ns_step": hp.ns_steps - 1, "sk_bprime": hp.ns_steps, "tl_gram": hp.ns_steps,
                         "tl_poly": hp.ns_steps, "tl_apply": hp.ns_steps - 1}.get(kname, 1)
            qty += q * per_batch
            nl += per_batch
        return None if bd is None else (bd, qty / max(nl, 1), u)

    # every traced kernel against its own roofline (the dominant one is `roofline`)
    for k, rec in kernels.items():
        r = per_launch(k)
        if r is None:
            continue
        bd, q, u = r
        s_ = rec["avg_ms"] / 1e3
        if bd == "hbm":
            rec.update({"bound": "hbm", "achieved": q / s_ / 1e9, "unit": "GB/s", "frac": q / s_ / 1e9 / HBM_PEAK_GBPS})
        else:
            pk = FP32_PEAK_TFLOPS if prec == "f32" else BF16_PEAK_TFLOPS
            rec.update({"bound": "mfma", "achieved": q / s_ / 1e12, "unit": "TFLOP/s", "frac": q / s_ / 1e12 / pk})
    bound, qty_per_launch, unit = per_launch(dom) or ("hbm", 0.0, "B")
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
    roof["timing"] = "library HIP events at the kernel's start and end, one-stream traced pass"

    flops = wl.nominal_ns_flops()
    if hp.ns_steps != wl.hp.ns_steps:
        flops = flops / wl.hp.ns_steps * hp.ns_steps
    exe = executed_flops(plan, hp.ns_steps, prec)
    value = flops / (ms / 1e3) / 1e12
    cfg = {"workload": wl.name, "matrices": int(sum(b.count for b in plan.batches)), "launch": args.launch,
           "streams": nstreams, "lanes": lane_of, "max_batch_elems": args.max_batch_elems or (1 << 29),
           "batches": [[b.count, b.M, b.N] for b in plan.batches],
           "kernels": [kernel_form(b, args.skinny_kernel, prec) for b in plan.batches],
           "param_dtype": dtype,
           "precision": prec, "ns_steps": hp.ns_steps, "coeffs": list(hp.coeffs),
           "inputs": ("seeded synthetic: drawn on the GPU with seeded torch generators, the checked matrices "
                      "from the seeded host generator" if inputs == "device" else
                      "seeded synthetic (host generator)" + (", same-shape batches share values"
                                                             if args.reuse_shapes else ""))}
    out = {"metric": "Muon-step NS TFLOP/s (bf16 MFMA)", "value": value, "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if prec != "f32" else "f32",
           "data": "synthetic", "config": cfg, "roofline": roof,
           "detail": {"timing": "median of the timed repetitions, each between HIP events on the caller's "
                                "stream, W and M restored from device copies before each",
                      "ms_per_rep": {"median": ms, "mean": float(np.mean(per_rep)), "min": float(np.min(per_rep)),
                                     "max": float(np.max(per_rep))},
                      "wall_s_timed_region": wall,
                      "ns_frac_of_bf16_peak": value / BF16_PEAK_TFLOPS,
                      "executed_tflop_per_step": exe / 1e12, "executed_tflops": exe / (ms / 1e3) / 1e12,
                      "executed_frac_of_bf16_peak": exe / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
                      "nominal_tflop_per_step": flops / 1e12,
                      "traced_ms_per_step_one_stream": traced_ms, "traced_steps": tsteps,
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
        # back to back: the same step repeated without restores (the
        # accumulated state does not change the work)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_bb = max(args.steps, 50)
        a0.record(stream)
        for _ in range(n_bb):
            run()
        a1.record(stream)
        torch.cuda.synchronize()
        out["detail"]["back_to_back_ms_per_step"] = a0.elapsed_time(a1) / n_bb
        # cold steps: reading 1 GiB between steps evicts the 256 MB Infinity
        # Cache with clean lines, so each timed step starts from HBM (the warm
        # value above may be served partly from that cache) and pays for no
        # write-back of someone else's data
        flush = torch.cat([src.view(torch.int32), dst.view(torch.int32)])
        ncold = min(args.steps, 10)

        def cold_steps():
            times = []
            for _ in range(ncold):
                restore()
                flush.sum()
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record(stream)
                step_prepared()
                a1.record(stream)
                torch.cuda.synchronize()
                times.append(a0.elapsed_time(a1))
            return times

        cold = cold_steps()
        # the same again with launch tracing (its events lengthen the step,
        # so the step time above is taken without): per-kernel times from HBM
        B.muon_trace_start(ncold * 64 * len(plan.batches) + 16)
        cold_steps()
        cper = {}
        for name, t in B.muon_trace_stop():
            cper.setdefault(name, []).append(t)
        out["detail"]["cold_ms_per_step"] = float(np.median(cold))
        out["detail"]["cold_tflops"] = flops / (np.median(cold) / 1e3) / 1e12
        out["detail"]["cold_kernels"] = {k: {"launches_per_step": len(v) / ncold, "median_ms": float(np.median(v))}
                                         for k, v in cper.items()}
        if roof["bound"] == "hbm" and dom in cper:
            roof["cold_achieved"] = qty_per_launch / (float(np.median(cper[dom])) / 1e3) / 1e9
            roof["cold_frac"] = roof["cold_achieved"] / HBM_PEAK_GBPS
        del flush
    del src, dst
    refs = {}
    progress("GPU work done")
    if not args.no_cpu_baseline:
        # with stored oracle values the sample needs no reference: one matrix
        sample = check_ids[:1] if ref[0] == "golden" else check_ids
        out["cpu_baseline"], refs = cpu_baseline(wl, plan, hp, sample, args.cpu_budget)
    if ref[0] == "golden" or refs:
        out["detail"]["check"] = check_result(wl, plan, hp, snap, snap_o, host, ref, refs)
    else:
        out["detail"]["check"] = {"reference": None, "ok": None,
                                  "note": "no oracle reference without the cpu_baseline leg"}
    print(json.dumps(out), flush=True)
    if out["detail"]["check"]["ok"] is False:
        print("bench: the timed step's result is outside the oracle bound: " + json.dumps(out["detail"]["check"]),
              file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
