"""The step with a per-step minimax coefficient schedule (muon_ns_schedule)
on inputs whose singular values are known.

X_0 = U / ||U||_F has singular values s_i / ||s||_2; an odd polynomial step
maps each to p_k(s), so after K steps every singular value of O lies in the
interval the schedule states for step K, whatever the shape or kernel.  Five
steps from these inputs' own lower bounds (2e-3 to 6e-3) leave them within
1.8e-2 of 1 (1.5e-4 for the 24-row case); ten steps make O orthogonal to float
precision.  fp32 precision, so the only slack is float rounding: 1e-4.
Parity with the oracle under the same schedule is in test_gpu_parity.py
(hyperparameter variants).
"""
import numpy as np
import pytest

from matrix_optimizer_amd import binding as B

pytestmark = pytest.mark.gpu

CASES = [((24, 2000), 1), ((24, 2000), 2), ((200, 600), 0), ((600, 200), 0), ((20, 700), 1)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _known_spectrum(M, N, seed):
    """G = Q1 diag(s) Q2^T with s geometric from 5 down to 0.05."""
    rng = np.random.default_rng(seed)
    m = min(M, N)
    q1, _ = np.linalg.qr(rng.standard_normal((M, m)))
    q2, _ = np.linalg.qr(rng.standard_normal((N, m)))
    s = 5.0 * np.geomspace(1.0, 1e-2, m)
    return (q1 * s) @ q2.T, s


@pytest.mark.parametrize("steps", [5, 10])
@pytest.mark.parametrize("shape,kernel", CASES, ids=[f"{c[0][0]}x{c[0][1]}-k{c[1]}" for c in CASES])
def test_schedule_bounds_singular_values(shape, kernel, steps):
    import torch
    M, N = shape
    G, s = _known_spectrum(M, N, seed=M * 7 + N)
    lower = float(s.min() / np.linalg.norm(s)) * (1 - 1e-3)
    coeffs, bounds = B.ns_schedule(steps, lower)
    lo, hi = bounds[-1]
    plan = B.Plan([shape], skinny_kernel=kernel)
    b = plan.batches[0]
    h = B.HParams(ns_steps=steps, coeffs=coeffs, precision="f32", lr=0.0, weight_decay=0.0)
    p = torch.zeros(1, M, N, dtype=torch.float32, device="cuda")
    g = torch.from_numpy(G.astype(np.float32)).reshape(1, M, N).cuda()
    mom = torch.zeros_like(p)
    o = torch.empty_like(p)
    ws = torch.empty(max(plan.workspace_bytes(b.index, "f32"), 256), dtype=torch.uint8, device="cuda")
    B.muon_step(plan, b.index, p, g, mom, h, ws, ns_out=o)
    torch.cuda.synchronize()
    sv = np.linalg.svd(o[0].cpu().numpy().astype(np.float64), compute_uv=False)
    assert sv.size == min(M, N)
    assert sv.min() >= lo - 1e-4 and sv.max() <= hi + 1e-4, (sv.min(), sv.max(), lo, hi)
    if steps == 10:
        assert hi - lo <= 1e-6
        assert np.max(np.abs(sv - 1.0)) <= 1e-4
    else:
        assert hi - lo < 0.25
