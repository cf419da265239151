"""Writes full_size_samples.npz: oracle values at seeded positions of every
matrix of the full-size batches the GPU parity tests run for the 32-layer
decoder (the smallest plan batch of each of its three shapes: 32 x 4096x4096,
10 x 11008x4096 through the transpose path, 10 x 4096x11008) and for the MoE
expert tensor [64, 2048, 7168] (both of its plan batches).

The float64 oracle takes seconds to tens of seconds per matrix here, too slow
to run for every matrix on each test run, so its output is stored: O (the
orthogonalised direction) and W' (the updated parameter) at SAMPLES positions
per matrix, drawn from default_rng(seed) with the seed listed per matrix.
The GPU test runs the same seeded inputs through the library and compares
those positions.

Calls only the oracle and the seeded input generator:
    python tests/golden/full_size_samples.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from matrix_optimizer_amd import workloads as WL  # noqa: E402
from oracle import muon_oracle as ORC  # noqa: E402
from oracle import plan_oracle as PO  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "full_size_samples.npz")
SAMPLES = 1024


def f32(x):
    return float(np.float32(x))


def chosen_batches(wl):
    """Per batch the GPU test runs, its (param, matrix) list in batch order, from the
    plan oracle's bucketing (the library's planner is pinned to it)."""
    plan = PO.plan([p.shape for p in wl.params])
    if wl.name == "decoder32_h4096_f11008":
        pick = {}
        for b in plan:
            if (b.M, b.N) not in pick or b.count < pick[(b.M, b.N)].count:
                pick[(b.M, b.N)] = b
        chosen = [pick[k] for k in sorted(pick)]
    else:
        chosen = [b for b in plan if b.M == 2048]
    return [[(s.param_index, s.first_matrix + q) for s in b.segments for q in range(s.num_matrices)]
            for b in chosen]


def main():
    out = {}
    meta = {"samples": SAMPLES, "entries": []}
    t0 = time.time()
    for name in ("decoder32_h4096_f11008", "moe_experts"):
        wl = WL.WORKLOADS[name]
        hp = wl.hp
        kw = dict(lr=f32(hp.lr), momentum=f32(hp.momentum), weight_decay=f32(hp.weight_decay), eps=f32(hp.eps),
                  nesterov=hp.nesterov, ns_steps=hp.ns_steps, coeffs=tuple(f32(c) for c in hp.coeffs),
                  scale=hp.scale)
        for mats in chosen_batches(wl):
            for (pi, mi) in mats:
                spec = wl.params[pi]
                W0 = WL.decode(wl.matrix(pi, mi, "param"), spec.dtype)
                G = WL.decode(wl.matrix(pi, mi, "grad"), spec.dtype)
                M0 = wl.matrix(pi, mi, "momentum").astype(np.float64)
                ref = ORC.muon_step_matrix(W0, G, M0, **kw)
                seed = 50000 + 1000 * (name == "moe_experts") + len(meta["entries"])
                rng = np.random.default_rng(seed)
                rows = rng.integers(0, W0.shape[0], SAMPLES)
                cols = rng.integers(0, W0.shape[1], SAMPLES)
                key = f"e{len(meta['entries'])}"
                out[key + "_O"] = ref["O"][rows, cols].astype(np.float32)
                out[key + "_W"] = ref["W"][rows, cols].astype(np.float32)
                meta["entries"].append({"workload": name, "param": pi, "matrix": mi, "shape": list(W0.shape),
                                        "seed": seed, "key": key, "hparams": kw})
                print(f"{name} param {pi} matrix {mi} {W0.shape}: {time.time() - t0:.0f} s", flush=True)
                del W0, G, M0, ref
    out["meta"] = np.array(json.dumps(meta))
    np.savez_compressed(OUT, **out)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
