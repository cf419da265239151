"""Writes large_8192x28672_samples.npz: oracle values at sampled positions of
the first matrix of each orientation of the 16 x 8192x28672 + 16 x
28672x8192 workload (rank-64 plus noise gradients, zero momentum), and, with
the argument "extra", large_8192x28672_extra_samples.npz for the second
matrix of each orientation (the other matrix of the same plan batches; the
GPU test checks both files, the benchmark only the first).

The float64 oracle needs about 44 TFLOP per matrix here, too slow for a test
run, so its output is stored at 4096 seeded positions per matrix: O (the
orthogonalised direction) and W' (the updated parameter).  The GPU test runs
the same seeded inputs through the library and compares those positions.

Calls only the oracle and the seeded input generator:
    python tests/golden/large_8192x28672_samples.py [extra]
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from matrix_optimizer_amd import workloads as WL  # noqa: E402
from oracle import muon_oracle as ORC  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
SAMPLES = 4096
# (parameters, output): the first [8192, 28672] and [28672, 8192] parameters, or the second ones (extra);
# each parameter is one matrix (matrix 0)
SETS = {"main": ((0, 16), os.path.join(HERE, "large_8192x28672_samples.npz")),
        "extra": ((1, 17), os.path.join(HERE, "large_8192x28672_extra_samples.npz"))}


def f32(x):
    return float(np.float32(x))


def main(which="main"):
    PARAMS, OUT = SETS[which]
    wl = WL.WORKLOADS["large_8192x28672"]
    hp = wl.hp
    # the fp32 values the kernels receive
    kw = dict(lr=f32(hp.lr), momentum=f32(hp.momentum), weight_decay=f32(hp.weight_decay), eps=f32(hp.eps),
              nesterov=hp.nesterov, ns_steps=hp.ns_steps, coeffs=tuple(f32(c) for c in hp.coeffs), scale=hp.scale)
    out = {}
    meta = {"workload": wl.name, "params": list(PARAMS), "matrix": 0, "samples": SAMPLES, "hparams": kw}
    for pi in PARAMS:
        W0 = WL.decode(wl.matrix(pi, 0, "param"), wl.params[pi].dtype)
        G = WL.decode(wl.matrix(pi, 0, "grad"), wl.params[pi].dtype)
        M0 = wl.matrix(pi, 0, "momentum").astype(np.float64)
        ref = ORC.muon_step_matrix(W0, G, M0, **kw)
        rng = np.random.default_rng(1000 + pi)
        rows = rng.integers(0, W0.shape[0], SAMPLES)
        cols = rng.integers(0, W0.shape[1], SAMPLES)
        out[f"p{pi}_rows"] = rows
        out[f"p{pi}_cols"] = cols
        out[f"p{pi}_O"] = ref["O"][rows, cols]
        out[f"p{pi}_W"] = ref["W"][rows, cols]
        out[f"p{pi}_O_fro"] = np.array([np.linalg.norm(ref["O"])])
        print(f"param {pi} {W0.shape}: ||O||_F = {out[f'p{pi}_O_fro'][0]:.6g}", flush=True)
        del W0, G, M0, ref
    out["meta"] = np.array(json.dumps(meta))
    np.savez_compressed(OUT, **out)
    print("wrote", OUT)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "main")
