"""Float64 CPU oracle of the owner-side Muon step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or runs
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may.  It shares no code with the HIP
library (no kernels, headers, helpers or constants) and imports nothing from
the ``matrix_optimizer_amd`` package.

It is plain NumPy in float64, one logical matrix at a time, with every step
written in the order and notation of the pages:

* momentum, then orthogonalise, then update -- DMuon-2 §2.1 (the momentum
  recurrence M_t = mu M_{t-1} + G and the update W_{t+1} = W_t - eta NS(M_t)),
  with the Nesterov variant that page says its implementation uses;
* X_0 = G / (||G||_F + eps) and the quintic step
  X_{k+1} = a_k X_k + b_k (X_k X_k^T) X_k + c_k (X_k X_k^T)^2 X_k --
  HyperParallel-FSDP §2.3, Eq. (1);
* the transpose-first rule when rows exceed columns -- HyperParallel-FSDP §6.6
  and Figure 10(a);
* the RMS-matched scale 0.2 sqrt(max(m, n)) -- HyperParallel-FSDP §2.3;
* decoupled (AdamW-style) weight decay -- HyperParallel-FSDP §6.3 / Figure 8
  and §6.4 step (4); HyperParallel RFC item 6;
* 3-D expert tensors are E independent matrices -- HyperParallel-FSDP §6.3;
  DMuon-2 Appendix C.5.

Readings taken where the pages are silent:

* Nesterov form: U = G + mu * M_t, with M_t = mu M_{t-1} + G.
* The normalised quantity is the NS input U.
* eps = 1e-7 by default; when ||U||_F + eps == 0 the direction is zero.
* Decay and the orthogonal update both use W_t: W' = W - eta (lambda W + s O).
* Square matrices are not transposed (the rule is "rows > cols").

Parity status: every function here is pinned by tests/test_oracle.py against
closed forms (SVD identity, diagonal and orthonormal inputs), invariances,
exact rational arithmetic on the elementwise stages and the sharding criterion
of DMuon-2 Appendix A.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np


def momentum_update(M: np.ndarray, G: np.ndarray, mu: float, nesterov: bool = True):
    """DMuon-2 §2.1: M_t = mu M_{t-1} + G(W).  Returns (M_t, U).

    U is the quantity Newton-Schulz orthogonalises.  The page says its
    implementation uses the Nesterov variant without printing it; the reading
    taken is U = G + mu M_t.  Without Nesterov, U = M_t.
    """
    M_new = mu * M + G
    U = G + mu * M_new if nesterov else M_new
    return M_new, U


def frobenius_normalize(U: np.ndarray, eps: float) -> np.ndarray:
    """HyperParallel-FSDP §2.3: X_0 = G / (||G||_F + eps), with G the momentum
    direction.  A zero denominator (zero input, eps = 0) gives X_0 = 0."""
    nu = math.sqrt(float(np.sum(U * U)))
    den = nu + eps
    if den == 0.0:
        return np.zeros_like(U)
    return U / den


def ns_coefficients(coeffs: Sequence[float], steps: int):
    """One (a, b, c) for every step (constant quintic) or one per step."""
    c = list(coeffs)
    if len(c) == 3:
        return [tuple(c)] * steps
    if len(c) == 3 * steps:
        return [tuple(c[3 * k:3 * k + 3]) for k in range(steps)]
    raise ValueError("coefficient count must be 3 or 3*steps")


def newton_schulz(X0: np.ndarray, coeffs: Sequence[float], steps: int) -> np.ndarray:
    """HyperParallel-FSDP Eq. (1): X_{k+1} = a X + b (X X^T) X + c (X X^T)^2 X.

    X0 is taken in the orientation it is given (rows <= cols is the caller's
    business, see ``orthogonalize``)."""
    X = np.array(X0, dtype=np.float64, copy=True)
    for a, b, c in ns_coefficients(coeffs, steps):
        A = X @ X.T
        X = a * X + b * (A @ X) + c * ((A @ A) @ X)
    return X


def orthogonalize(U: np.ndarray, coeffs: Sequence[float], steps: int, eps: float) -> np.ndarray:
    """Normalise, transpose if rows > cols (HyperParallel-FSDP §6.6), iterate,
    and return the result in U's own orientation."""
    X = frobenius_normalize(U, eps)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = newton_schulz(X, coeffs, steps)
    return X.T if tall else X


def rms_scale(M: int, N: int, mode: str = "rms") -> float:
    """HyperParallel-FSDP §2.3 (and DMuon-2 Appendix D.9): RMS-matched scale
    0.2 sqrt(max(m, n)); mode "none" gives 1."""
    if mode == "rms":
        return 0.2 * math.sqrt(max(M, N))
    if mode == "none":
        return 1.0
    raise ValueError(mode)


def apply_update(W: np.ndarray, O: np.ndarray, lr: float, wd: float, s: float) -> np.ndarray:
    """Decoupled weight decay plus the orthogonal update, both from W_t:
    W' = W - eta (lambda W + s O)."""
    return W - lr * (wd * W + s * O)


def muon_step_matrix(W: np.ndarray, G: np.ndarray, M: np.ndarray, *, lr: float, momentum: float,
                     weight_decay: float, eps: float = 1e-7, nesterov: bool = True,
                     ns_steps: int = 5, coeffs: Sequence[float] = (3.4445, -4.7750, 2.0315),
                     scale: str = "rms") -> Dict[str, np.ndarray]:
    """One Muon step on one [M,N] matrix.  Returns W', M', U and O."""
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    M_new, U = momentum_update(M, G, momentum, nesterov)
    O = orthogonalize(U, coeffs, ns_steps, eps)
    s = rms_scale(W.shape[0], W.shape[1], scale)
    W_new = apply_update(W, O, lr, weight_decay, s)
    return {"W": W_new, "M": M_new, "U": U, "O": O}


def matrices_of(t: np.ndarray) -> np.ndarray:
    """View a parameter tensor as its stack of logical matrices:
    [M,N] -> 1 matrix, [M,1,N] -> 1 matrix, [E,M,N] -> E matrices
    (HyperParallel-FSDP §6.6 / Figure 10(a); §6.3 for experts)."""
    if t.ndim == 2:
        return t[None]
    if t.ndim == 3 and t.shape[1] == 1:
        return t[:, 0, :][None]
    if t.ndim == 3:
        return t
    raise ValueError("Muon takes 2-D and 3-D parameters only")


def muon_step_tensor(W: np.ndarray, G: np.ndarray, M: np.ndarray, **hp) -> Dict[str, np.ndarray]:
    """One Muon step on a whole parameter tensor, matrix by matrix."""
    Ws, Gs, Ms = matrices_of(W), matrices_of(G), matrices_of(M)
    outs = [muon_step_matrix(Ws[i], Gs[i], Ms[i], **hp) for i in range(Ws.shape[0])]
    res = {}
    for k in ("W", "M", "U", "O"):
        res[k] = np.stack([o[k] for o in outs]).reshape(W.shape)
    return res

