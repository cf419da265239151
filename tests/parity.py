"""The parity bars of the GPU tests, for one matrix at a time: the HIP path's
result against the float64 oracle on the same stored inputs.

Bars (per matrix):
* O (the orthogonalised direction): relative Frobenius error <= 3e-2 for the
  bf16 MFMA modes, <= 1e-5 for the fp32 check path;
* M' (momentum): elementwise |gpu - ref| <= 1e-6 (|mu M| + |G|);
* W' given the GPU's own O: elementwise <= 1e-6 (|W| + lr|wd W| + lr|s O|)
  for fp32 W, within one bf16 ulp for bf16 W (round-to-nearest-even store);
* W' - W end to end against the oracle: the O bound plus the bf16 rounding
  of the stored W' (derived per matrix from half an ulp of every element).
Hyperparameters are handed to the oracle as the fp32 values the kernels see.
"""
from __future__ import annotations

import numpy as np

from matrix_optimizer_amd import binding as B
from oracle import muon_oracle as ORC
from tests import harness as H


def check_matrix(W0s, Gs, M0s, Wp, Mp, O, h: B.HParams, where: str = "") -> float:
    """One matrix: stored inputs W0s, Gs (uint16 bf16 bits or float32) and M0s
    (float32), and the GPU's stored W' (Wp), M' (Mp) and O, all [M, N] in W's
    orientation.  O may be None (the update is then checked end to end only).
    Returns the O error (or the W' - W error without O)."""
    M, N = W0s.shape
    kw = H.oracle_kwargs(h, M, N)
    s = H.oracle_scale(h, M, N)
    W0, G = H.decode(W0s), H.decode(Gs)
    M0 = np.asarray(M0s).astype(np.float64)
    ref = ORC.muon_step_matrix(W0, G, M0, **kw)
    H.check_momentum(Mp, M0, G, kw["momentum"])
    tol = H.o_tolerance(h.precision)
    e = None
    if O is not None:
        Oq = np.asarray(O).astype(np.float64)
        assert np.all(np.isfinite(Oq)), f"{where}: non-finite O"
        e = H.rel_fro(Oq, ref["O"])
        assert e <= tol, f"{where}: O error {e:.3g} > {tol}"
        H.check_update(Wp, W0, Oq, kw["lr"], kw["weight_decay"], s)
    dW_ref = ref["W"] - W0
    dW = H.decode(Wp) - W0
    if np.linalg.norm(dW_ref) > 0:
        slack = 0.0
        if Wp.dtype == np.uint16:
            half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref["W"]), 1e-38))) - 8)
            slack = np.linalg.norm(half_ulp) / np.linalg.norm(dW_ref)
        ew = H.rel_fro(dW, dW_ref)
        assert ew <= tol + slack + 1e-6, f"{where}: W' - W error {ew:.3g}"
        if e is None:
            e = ew
    return 0.0 if e is None else e
