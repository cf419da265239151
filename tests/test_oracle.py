"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each one checks it against a
different computation -- an SVD with the scalar map applied to each singular
value, exact rational arithmetic, an invariance, or the sharding criterion of
DMuon-2 Appendix A.  ``test_pins_catch_planted_mistakes`` plants plausible
mistakes into a copy of the oracle (on the CPU) and shows that some pin fails
for each.
"""
import inspect
import math
import types
from fractions import Fraction

import numpy as np
import pytest

from oracle import muon_oracle as ORC

COEFFS = (3.4445, -4.7750, 2.0315)
STEPS = 5


# --------------------------------------------------------------------------
# independent closed forms used by the pins
# --------------------------------------------------------------------------
def scalar_map_exact(x: Fraction, coeffs, steps) -> Fraction:
    """What NS does to one singular value, in exact rational arithmetic
    (HyperParallel-FSDP Eq. (1) restricted to a 1x1 matrix)."""
    cs = [Fraction(str(c)) for c in coeffs]
    sets = [cs] * steps if len(cs) == 3 else [cs[3 * k:3 * k + 3] for k in range(steps)]
    for a, b, c in sets:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def scalar_map_float(x: float, coeffs, steps) -> float:
    """The same scalar map in float64 (used on many singular values)."""
    cs = list(coeffs)
    sets = [cs] * steps if len(cs) == 3 else [cs[3 * k:3 * k + 3] for k in range(steps)]
    for a, b, c in sets:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def svd_reference(G: np.ndarray, coeffs, steps, eps) -> np.ndarray:
    """O = U_s diag(p^K(sigma_i / (||G||_F + eps))) V_s^T: NS is a polynomial in
    X X^T times X, so it acts on the singular values only."""
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    den = np.linalg.norm(G) + eps
    ps = np.array([scalar_map_float(float(si / den), coeffs, steps) for si in s])
    return (U * ps) @ Vt


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------------
# pin checks, each taking the oracle module so planted mistakes can be run
# --------------------------------------------------------------------------
def check_svd_identity(orc):
    rng = np.random.default_rng(11)
    for shape in [(7, 11), (11, 7), (5, 5), (1, 9), (9, 1), (16, 40)]:
        G = rng.standard_normal(shape)
        O = orc.orthogonalize(G, COEFFS, STEPS, 1e-7)
        ref = svd_reference(G, COEFFS, STEPS, 1e-7)
        assert rel(O, ref) < 1e-12, shape
    # a per-step coefficient schedule goes through the same identity
    sched = (3.0, -3.2, 1.2, 3.4445, -4.7750, 2.0315, 2.0, -1.5, 0.5)
    G = rng.standard_normal((6, 10))
    assert rel(orc.orthogonalize(G, sched, 3, 0.0), svd_reference(G, sched, 3, 0.0)) < 1e-12


def check_diagonal_rational(orc):
    # G = [[3,0,0],[0,4,0]]: ||G||_F = 5, singular values 3 and 4 -> X0 = diag(0.6, 0.8)
    G = np.array([[3.0, 0, 0], [0, 4.0, 0]])
    O = orc.orthogonalize(G, COEFFS, STEPS, 0.0)
    e06 = float(scalar_map_exact(Fraction(3, 5), COEFFS, STEPS))
    e08 = float(scalar_map_exact(Fraction(4, 5), COEFFS, STEPS))
    ref = np.array([[e06, 0, 0], [0, e08, 0]])
    assert np.max(np.abs(O - ref)) < 1e-14
    # and transposed: the tall orientation goes through the transpose-first rule
    assert np.max(np.abs(orc.orthogonalize(G.T, COEFFS, STEPS, 0.0) - ref.T)) < 1e-14


def check_orthonormal_rows(orc):
    rng = np.random.default_rng(5)
    for m, n in [(4, 12), (24, 64), (8, 8)]:
        Q, _ = np.linalg.qr(rng.standard_normal((n, m)))
        Q = Q.T                                          # m x n with Q Q^T = I
        O = orc.orthogonalize(Q, COEFFS, STEPS, 0.0)
        f = scalar_map_float(1.0 / math.sqrt(m), COEFFS, STEPS)
        assert rel(O, f * Q) < 1e-12


def check_invariances(orc):
    rng = np.random.default_rng(7)
    G = rng.standard_normal((6, 14))
    O = orc.orthogonalize(G, COEFFS, STEPS, 0.0)
    # scale invariance (eps = 0)
    assert rel(orc.orthogonalize(37.5 * G, COEFFS, STEPS, 0.0), O) < 1e-12
    # orthogonal equivariance NS(P G Q) = P NS(G) Q
    P, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    Qm, _ = np.linalg.qr(rng.standard_normal((14, 14)))
    assert rel(orc.orthogonalize(P @ G @ Qm, COEFFS, STEPS, 0.0), P @ O @ Qm) < 1e-12
    # transpose: NS(G^T) = NS(G)^T
    assert rel(orc.orthogonalize(G.T, COEFFS, STEPS, 0.0), O.T) < 1e-12


def check_sharding_criterion(orc):
    """DMuon-2 §2.1 and Appendix A: row shards orthogonalised separately agree
    with the whole matrix iff rows of different shards are orthogonal."""
    rng = np.random.default_rng(3)
    n = 20
    basis, _ = np.linalg.qr(rng.standard_normal((n, n)))
    # M1 rows in span(basis[:, :6]), M2 rows in span(basis[:, 6:12]) -> M1 M2^T = 0
    M1 = rng.standard_normal((4, 6)) @ basis[:, :6].T
    M2 = rng.standard_normal((5, 6)) @ basis[:, 6:12].T
    Mw = np.vstack([M1, M2])
    assert np.max(np.abs(M1 @ M2.T)) < 1e-12

    def polar(X):
        U, _, Vt = np.linalg.svd(X, full_matrices=False)
        return U @ Vt

    assert rel(np.vstack([polar(M1), polar(M2)]), polar(Mw)) < 1e-12
    # NS with the same (global) normalisation splits exactly as well ...
    nrm = np.linalg.norm(Mw)
    whole = orc.newton_schulz(Mw / nrm, COEFFS, STEPS)
    split = np.vstack([orc.newton_schulz(M1 / nrm, COEFFS, STEPS),
                       orc.newton_schulz(M2 / nrm, COEFFS, STEPS)])
    assert rel(split, whole) < 1e-12
    # ... and the oracle's whole-matrix step agrees with it
    assert rel(orc.orthogonalize(Mw, COEFFS, STEPS, 0.0), whole) < 1e-12
    # generic Gaussian rows: shards differ from the whole by O(1)
    G = rng.standard_normal((9, n))
    whole = orc.orthogonalize(G, COEFFS, STEPS, 0.0)
    split = np.vstack([orc.orthogonalize(G[:4], COEFFS, STEPS, 0.0),
                       orc.orthogonalize(G[4:], COEFFS, STEPS, 0.0)])
    assert rel(split, whole) > 0.1


def check_elementwise_rational(orc):
    """Momentum, Nesterov direction and update on dyadic inputs, where float64
    is exact, against Fraction arithmetic of the same readings."""
    Mv = np.array([[2.0, -1.5], [0.25, 8.0]])
    Gv = np.array([[1.0, 0.5], [-3.0, 0.125]])
    mu = 0.5
    M_new, U = orc.momentum_update(Mv, Gv, mu, True)
    for i in range(2):
        for j in range(2):
            fm = Fraction(mu) * Fraction(Mv[i, j]) + Fraction(Gv[i, j])
            assert M_new[i, j] == float(fm)
            assert U[i, j] == float(Fraction(Gv[i, j]) + Fraction(mu) * fm)
    M_plain, U_plain = orc.momentum_update(Mv, Gv, mu, False)
    assert np.array_equal(U_plain, M_plain)
    W = np.array([[1.0, -2.0], [0.5, 4.0]])
    O = np.array([[0.25, 0.5], [-1.0, 2.0]])
    lr, wd, s = 0.25, 0.5, 2.0
    Wn = orc.apply_update(W, O, lr, wd, s)
    for i in range(2):
        for j in range(2):
            ref = Fraction(W[i, j]) - Fraction(lr) * (Fraction(wd) * Fraction(W[i, j]) + Fraction(s) * Fraction(O[i, j]))
            assert Wn[i, j] == float(ref)


def check_special_cases(orc):
    rng = np.random.default_rng(1)
    W = rng.standard_normal((6, 9))
    Z = np.zeros((6, 9))
    hp = dict(lr=0.02, momentum=0.95, weight_decay=0.1, eps=1e-7)
    r = orc.muon_step_matrix(W, Z, Z, **hp)
    assert np.all(np.isfinite(r["O"])) and np.max(np.abs(r["O"])) == 0.0
    assert np.array_equal(r["W"], W - 0.02 * (0.1 * W + 0.0))
    # eps = 0 with a zero direction still gives zero, not NaN
    r0 = orc.muon_step_matrix(W, Z, Z, **dict(hp, eps=0.0))
    assert np.max(np.abs(r0["O"])) == 0.0
    G = rng.standard_normal((6, 9))
    Mv = rng.standard_normal((6, 9))
    r = orc.muon_step_matrix(W, G, Mv, **dict(hp, momentum=0.0))
    assert np.array_equal(r["U"], G) and np.array_equal(r["M"], G)
    r = orc.muon_step_matrix(W, G, Mv, **dict(hp, lr=0.0))
    assert np.array_equal(r["W"], W)


def check_rms_scale(orc):
    """HyperParallel-FSDP §2.3: the scale makes the update RMS 0.2 for an exact
    semi-orthogonal factor (RMS 1/sqrt(max(m, n)))."""
    rng = np.random.default_rng(2)
    for M, N in [(24, 160), (160, 24), (16, 16)]:
        U, _, Vt = np.linalg.svd(rng.standard_normal((M, N)), full_matrices=False)
        Q = U @ Vt
        s = orc.rms_scale(M, N, "rms")
        assert abs(np.sqrt(np.mean((s * Q) ** 2)) - 0.2) < 1e-12
    assert orc.rms_scale(3, 7, "none") == 1.0


def check_expert_independence(orc):
    """HyperParallel-FSDP §6.3: an [E,M,N] tensor is E independent matrices,
    never one flattened [E, M*N] matrix."""
    rng = np.random.default_rng(4)
    E, M, N = 3, 5, 8
    W = rng.standard_normal((E, M, N))
    G = rng.standard_normal((E, M, N))
    Mv = rng.standard_normal((E, M, N))
    hp = dict(lr=0.02, momentum=0.95, weight_decay=0.1, eps=1e-7)
    r = orc.muon_step_tensor(W, G, Mv, **hp)
    for e in range(E):
        one = orc.muon_step_matrix(W[e], G[e], Mv[e], **hp)
        U = G[e] + 0.95 * (0.95 * Mv[e] + G[e])
        assert rel(r["O"][e], svd_reference(U, COEFFS, STEPS, 1e-7)) < 1e-12
        assert rel(r["W"][e], one["W"]) == 0.0
    # [M,1,N] is one matrix
    r1 = orc.muon_step_tensor(W[0][:, None, :], G[0][:, None, :], Mv[0][:, None, :], **hp)
    assert rel(r1["W"][:, 0, :], r["W"][0]) == 0.0


PIN_CHECKS = [check_svd_identity, check_diagonal_rational, check_orthonormal_rows,
              check_invariances, check_sharding_criterion, check_elementwise_rational,
              check_special_cases, check_rms_scale, check_expert_independence]


@pytest.mark.parametrize("check", PIN_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(ORC)


# --------------------------------------------------------------------------
# planted mistakes (run on the CPU, in a copy of the oracle)
# --------------------------------------------------------------------------
def _mutant(**overrides):
    """A fresh copy of the oracle module with some functions replaced."""
    m = types.ModuleType("oracle_mutant")
    exec(compile(inspect.getsource(ORC), ORC.__file__, "exec"), m.__dict__)
    m.__dict__.update(overrides)
    return m


def _ns_dropped_c(X0, coeffs, steps):
    X = np.array(X0, dtype=np.float64)
    for a, b, c in ORC.ns_coefficients(coeffs, steps):
        A = X @ X.T
        X = a * X + b * (A @ X)
    return X


def _ns_wrong_sign(X0, coeffs, steps):
    X = np.array(X0, dtype=np.float64)
    for a, b, c in ORC.ns_coefficients(coeffs, steps):
        A = X @ X.T
        X = a * X - b * (A @ X) + c * ((A @ A) @ X)
    return X


def _ns_extra_gram_power(X0, coeffs, steps):
    X = np.array(X0, dtype=np.float64)
    for a, b, c in ORC.ns_coefficients(coeffs, steps):
        A = X @ X.T
        X = a * X + b * (A @ X) + c * ((A @ A @ A) @ X)
    return X


def _ortho_no_transpose_back(U, coeffs, steps, eps):
    X = ORC.frobenius_normalize(U, eps)
    if X.shape[0] > X.shape[1]:
        X = X.T
    return ORC.newton_schulz(X, coeffs, steps)


def _norm_squared(U, eps):
    return U / (float(np.sum(U * U)) + eps)


def _norm_max(U, eps):
    return U / (float(np.max(np.abs(U))) + eps)


def _mom_old(M, G, mu, nesterov=True):
    return mu * M + G, G + mu * M


def _mom_no_grad(M, G, mu, nesterov=True):
    Mn = mu * M + G
    return Mn, mu * Mn


def _update_sign(W, O, lr, wd, s):
    return W - lr * (wd * W - s * O)


def _update_coupled(W, O, lr, wd, s):
    return W - lr * s * O - wd * W


def _scale_linear(M, N, mode="rms"):
    return 0.2 * max(M, N) if mode == "rms" else 1.0


def _matrices_flat(t):
    if t.ndim == 3 and t.shape[1] != 1:
        return t.reshape(1, t.shape[0] * t.shape[1], t.shape[2])
    return ORC.matrices_of(t)


def _coeffs_reversed(coeffs, steps):
    c = list(coeffs)
    sets = [tuple(c)] * steps if len(c) == 3 else [tuple(c[3 * k:3 * k + 3]) for k in range(steps)]
    return sets[::-1]


MUTANTS = {
    "dropped_quintic_term": dict(newton_schulz=_ns_dropped_c),
    "wrong_sign_cubic": dict(newton_schulz=_ns_wrong_sign),
    "extra_gram_power": dict(newton_schulz=_ns_extra_gram_power),
    "no_transpose_back": dict(orthogonalize=_ortho_no_transpose_back),
    "norm_squared": dict(frobenius_normalize=_norm_squared),
    "norm_max": dict(frobenius_normalize=_norm_max),
    "nesterov_old_momentum": dict(momentum_update=_mom_old),
    "nesterov_no_grad": dict(momentum_update=_mom_no_grad),
    "update_sign": dict(apply_update=_update_sign),
    "decay_coupled": dict(apply_update=_update_coupled),
    "scale_without_sqrt": dict(rms_scale=_scale_linear),
    "experts_flattened": dict(matrices_of=_matrices_flat),
    "schedule_reversed": dict(ns_coefficients=_coeffs_reversed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    mut = _mutant(**MUTANTS[name])
    failures = 0
    for check in PIN_CHECKS:
        try:
            check(mut)
        except (AssertionError, ValueError, np.linalg.LinAlgError):
            failures += 1
    assert failures >= 1, f"no pin catches the planted mistake {name}"
