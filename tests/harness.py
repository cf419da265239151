"""Shared helpers for the parity tests: build batch buffers from the seeded
generator, run the HIP path through the C ABI, run the oracle on the same
stored values, and compare."""
from __future__ import annotations

from dataclasses import replace
from typing import Dict, Iterable, List, Optional

import numpy as np

from matrix_optimizer_amd import binding as B
from matrix_optimizer_amd import workloads as WL

F32_EPS = np.finfo(np.float32).eps


def f32(x: float) -> float:
    """The value a hyperparameter takes once it crosses the ABI as a float."""
    return float(np.float32(x))


def c_hparams(hp: WL.HParams, **over) -> B.HParams:
    d = dict(lr=hp.lr, momentum=hp.momentum, weight_decay=hp.weight_decay, eps=hp.eps, nesterov=hp.nesterov,
             ns_steps=hp.ns_steps, coeffs=tuple(hp.coeffs), scale=hp.scale, precision=hp.precision)
    d.update(over)
    return B.HParams(**d)


def oracle_kwargs(h: B.HParams, M: int, N: int) -> Dict:
    """Oracle hyperparameters equal to what the kernels see (fp32-rounded)."""
    return dict(lr=f32(h.lr), momentum=f32(h.momentum), weight_decay=f32(h.weight_decay), eps=f32(h.eps),
                nesterov=h.nesterov, ns_steps=h.ns_steps, coeffs=tuple(f32(c) for c in h.coeffs),
                scale=h.scale)


def oracle_scale(h: B.HParams, M: int, N: int) -> float:
    """The scale s as the library passes it (computed in double, then float)."""
    if h.scale == "none":
        return 1.0
    return f32(0.2 * np.sqrt(max(M, N)))


def batch_arrays(wl: WL.Workload, binfo: B.BatchInfo, kinds=("param", "grad", "momentum")) -> Dict[str, np.ndarray]:
    """Stored encodings [count, M, N] of one plan batch, filled segment by segment."""
    out = {}
    for kind in kinds:
        arr = None
        for (pi, first, num, off) in binfo.segments:
            for q in range(num):
                mat = wl.matrix(pi, first + q, kind)
                if arr is None:
                    arr = np.empty((binfo.count, binfo.M, binfo.N), dtype=mat.dtype)
                arr[off // (binfo.M * binfo.N) + q] = mat
        out[kind] = arr
    return out


def matrix_ids(binfo: B.BatchInfo) -> List[tuple]:
    """(param_index, matrix_index) of every matrix of a batch, in batch order."""
    ids = []
    for (pi, first, num, off) in binfo.segments:
        ids += [(pi, first + q) for q in range(num)]
    return ids


def to_device(arr: np.ndarray, dtype: str):
    import torch
    if dtype == WL.BF16:
        return torch.from_numpy(arr.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def decode(arr: np.ndarray) -> np.ndarray:
    return WL.bf16_bits_to_f64(arr) if arr.dtype == np.uint16 else arr.astype(np.float64)


def run_gpu_step(plan: B.Plan, binfo: B.BatchInfo, arrays: Dict[str, np.ndarray], dtype: str, h: B.HParams,
                 want_o: bool = True, repeat: int = 1):
    """muon_step through the C ABI; returns host copies (W', M', O)."""
    import torch
    p = to_device(arrays["param"], dtype)
    g = to_device(arrays["grad"], dtype)
    m = to_device(arrays["momentum"], WL.F32)
    o = torch.empty((binfo.count, binfo.M, binfo.N), dtype=torch.float32, device="cuda") if want_o else None
    ws = torch.empty(max(plan.workspace_bytes(binfo.index, h.precision), 256), dtype=torch.uint8, device="cuda")
    for _ in range(repeat):
        B.muon_step(plan, binfo.index, p, g, m, h, ws, ns_out=o)
    torch.cuda.synchronize()
    return to_host(p), to_host(m), (to_host(o) if want_o else None)


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def check_momentum(M_gpu: np.ndarray, M_old: np.ndarray, G: np.ndarray, mu: float, tol: float = 1e-6):
    """Elementwise, cancellation-safe: |M'_gpu - M'_ref| <= tol (|mu M| + |G|)."""
    ref = mu * M_old + G
    bound = tol * (np.abs(mu * M_old) + np.abs(G)) + 1e-30
    err = np.abs(M_gpu.astype(np.float64) - ref)
    assert np.all(err <= bound), f"momentum mismatch: max ratio {np.max(err / bound):.3g}"


def check_update(W_gpu_stored: np.ndarray, W_old: np.ndarray, O: np.ndarray, lr: float, wd: float, s: float,
                 tol: float = 1e-6):
    """W' against W - lr (wd W + s O) with the GPU's own O (identical inputs).
    fp32 W: elementwise <= tol (|W| + lr|wd W| + lr|s O|).  bf16 W: within one
    bf16 ulp of the exact value (the store rounds to nearest even)."""
    ref = W_old - lr * (wd * W_old + s * O)
    Wg = decode(W_gpu_stored)
    if W_gpu_stored.dtype == np.uint16:
        ulp = np.maximum(np.abs(ref), 1e-38)
        ulp = 2.0 ** (np.floor(np.log2(ulp)) - 7)
        bound = ulp * 1.0 + tol * (np.abs(W_old) + lr * np.abs(wd * W_old) + lr * np.abs(s * O))
    else:
        bound = tol * (np.abs(W_old) + lr * np.abs(wd * W_old) + lr * np.abs(s * O)) + 1e-30
    err = np.abs(Wg - ref)
    assert np.all(err <= bound), f"update mismatch: max ratio {np.max(err / bound):.3g}"


def o_tolerance(precision: str) -> float:
    return 1e-5 if precision == "f32" else 3e-2
