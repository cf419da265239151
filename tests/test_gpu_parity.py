"""Parity of the HIP path (through the C ABI) with the float64 oracle, per
matrix, with the bars stated in tests/parity.py: O within 3e-2 (bf16 modes)
or 1e-5 (fp32) relative Frobenius error, M' within 1e-6 elementwise, W'
within one bf16 ulp (or 1e-6) given the GPU's O, and W' - W end to end.
Hyperparameters are handed to the oracle as the fp32 values the kernels see.
"""
import numpy as np
import pytest

from matrix_optimizer_amd import binding as B
from matrix_optimizer_amd import workloads as WL
from oracle import muon_oracle as ORC
from tests import harness as H
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def check_batch(wl, h: B.HParams, dtype: str, select=None, plan=None, batches=None, skinny_kernel=0):
    """Run every (or the chosen) batch of wl's plan and compare the selected
    matrices with the oracle (tests/parity.py).  Returns the list of O errors."""
    plan = plan or B.Plan([p.shape for p in wl.params], skinny_kernel=skinny_kernel)
    errs = []
    for binfo in plan.batches:
        if batches is not None and binfo.index not in batches:
            continue
        arrays = H.batch_arrays(wl, binfo)
        Wp, Mp, O = H.run_gpu_step(plan, binfo, arrays, dtype, h)
        sel = range(binfo.count) if select is None else select(binfo)
        for q in sel:
            errs.append(P.check_matrix(arrays["param"][q], arrays["grad"][q], arrays["momentum"][q], Wp[q], Mp[q],
                                       O[q], h, f"batch {binfo.index} matrix {q}"))
    return errs


PRECS = ["bf16", "bf16_x32", "bf16_x32c", "f32"]


# --------------------------------------------------------------------------
# the single 128x256 fp32 matrix (seed 0)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("prec", PRECS)
def test_single_128x256(prec):
    wl = WL.WORKLOADS["single_128x256_f32"]
    errs = check_batch(wl, H.c_hparams(wl.hp, precision=prec), WL.F32)
    print(f"single_128x256 {prec}: O error {errs}")


# --------------------------------------------------------------------------
# ragged and degenerate shapes, both paths, all precisions and dtypes
# --------------------------------------------------------------------------
SHAPE_SETS = {
    "skinny_ragged": [(24, 333), (24, 333)],
    "skinny_tall": [(333, 24)],
    "skinny_mixed_forms": [(7, 1000), (7, 1, 1000), (3, 7, 1000)],
    "skinny_32": [(32, 2049)],
    "row_vector": [(1, 50)],
    "col_vector": [(50, 1)],
    "tiny": [(2, 3), (3, 2)],
    "square_33": [(33, 33)],
    "tiled_wide": [(100, 300)],
    "tiled_tall": [(300, 100)],
    "tiled_square": [(130, 130)],
    "tiled_multi_tile": [(129, 400), (2, 129, 400)],
    "tiled_experts_tall": [(2, 300, 40)],
    "tiled_256_tiles": [(256, 768), (2, 512, 256)],
    # 256 x 256 tiles over 3 x 4 tile grids with ragged edges: off-diagonal
    # triangle tiles, several tiles per workgroup, both orientations
    "tiled_256_ragged": [(700, 900), (2, 900, 700)],
    # the same with stored rows a multiple of 8 long: the first pass moves
    # 16-byte runs (16 x 256 regions for the wide form, 64 x 64 through the
    # LDS transpose for the tall one) and must zero the ragged padding
    "tiled_256_ragged_vec": [(696, 904), (2, 904, 696)],
}


def _skinny(name):
    return all(min(WL.ParamSpec("x", tuple(s)).matrix_shape) <= 32 for s in SHAPE_SETS[name])


# skinny shapes run through every Newton-Schulz form: 0 = Gram space, one launch for the
# iteration and the apply (bf16 precision), 1 = Gram space in three launches, 2 = step by step
SHAPE_CASES = [(n, k) for n in sorted(SHAPE_SETS) for k in ((0, 1, 2) if _skinny(n) else (0,))]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("dtype", [WL.BF16, WL.F32])
@pytest.mark.parametrize("name,kernel", SHAPE_CASES, ids=[f"{n}-k{k}" for n, k in SHAPE_CASES])
def test_small_shapes(name, kernel, dtype, prec):
    wl = WL.small_workload(name, SHAPE_SETS[name], dtype=dtype, momentum_recipe="normal",
                           wid=200 + sorted(SHAPE_SETS).index(name))
    check_batch(wl, H.c_hparams(wl.hp, precision=prec), dtype, skinny_kernel=kernel)


# --------------------------------------------------------------------------
# hyperparameter variants
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shapes", [[(24, 500)], [(160, 200)]], ids=["skinny", "tiled"])
@pytest.mark.parametrize("variant", ["one_step", "schedule", "c_zero", "c_tiny", "no_nesterov", "no_scale", "eps_zero",
                                     "seven_steps", "minimax_schedule"])
def test_hparam_variants(shapes, variant):
    wl = WL.small_workload("v", shapes, momentum_recipe="normal", wid=300)
    over = {
        "one_step": dict(ns_steps=1),
        "schedule": dict(ns_steps=3, coeffs=(3.0, -3.2, 1.2, 3.4445, -4.7750, 2.0315, 2.0, -1.5, 0.5)),
        # a cubic step (c = 0) between quintic ones: the tiled bf16 poly then
        # takes b A from the fp32 copy of A instead of its operand tiles
        "c_zero": dict(ns_steps=3, coeffs=(3.4445, -4.7750, 2.0315, 1.5, -0.5, 0.0, 3.4445, -4.7750, 2.0315)),
        # a nonzero but subnormal c: b / c would overflow, so the same fp32-A
        # fallback must take it
        "c_tiny": dict(ns_steps=3, coeffs=(3.4445, -4.7750, 2.0315, 1.5, -0.5, 1e-39, 3.4445, -4.7750, 2.0315)),
        "no_nesterov": dict(nesterov=False),
        "no_scale": dict(scale="none"),
        "eps_zero": dict(eps=0.0),
        "seven_steps": dict(ns_steps=7),
        # five greedy minimax steps from a 1e-3 singular-value bound, with
        # the safety factor 1.01 and cushion 0.02 that bf16 operands need
        # (first step a = 7.63, b = -21.5, c = 15.5; without them, a = 8.47
        # amplifies operand rounding past the bf16 bound on 160 x 200)
        "minimax_schedule": dict(ns_steps=5, coeffs=B.ns_schedule(5, 1e-3, 1.01, 0.02)[0]),
    }[variant]
    for prec in PRECS:
        for kernel in (0, 1, 2):
            check_batch(wl, H.c_hparams(wl.hp, precision=prec, **over), WL.BF16, skinny_kernel=kernel)


# --------------------------------------------------------------------------
# special cases
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shapes,kernel", [([(24, 700)], 1), ([(24, 700)], 2), ([(200, 72)], 0)],
                         ids=["skinny-gram", "skinny-stepwise", "tiled"])
def test_zero_gradient_and_zero_lr(shapes, kernel):
    import torch
    plan = B.Plan(shapes, skinny_kernel=kernel)
    b = plan.batches[0]
    wl = WL.small_workload("z", shapes, dtype=WL.F32, momentum_recipe="zeros", wid=301)
    arrays = H.batch_arrays(wl, b)
    arrays["grad"] = np.zeros_like(arrays["grad"])
    for prec in PRECS:
        h = H.c_hparams(wl.hp, precision=prec)
        Wp, Mp, O = H.run_gpu_step(plan, b, arrays, WL.F32, h)
        assert np.all(O == 0) and np.all(Mp == 0)
        W0 = arrays["param"].astype(np.float32)
        lr, wd = np.float32(h.lr), np.float32(h.weight_decay)
        ref = W0 - lr * (wd * W0 + np.float32(0) * np.float32(0))
        assert np.max(np.abs(Wp - ref)) <= 1e-7 * np.max(np.abs(W0))
        # lr = 0 leaves W bitwise unchanged
        h0 = H.c_hparams(wl.hp, precision=prec, lr=0.0)
        arrays2 = H.batch_arrays(wl, b)
        Wp0, _, _ = H.run_gpu_step(plan, b, arrays2, WL.F32, h0)
        assert np.array_equal(Wp0, arrays2["param"])


# --------------------------------------------------------------------------
# determinism, batch independence, transpose symmetry
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shapes,kernel", [([(24, 3000)] * 3, 0), ([(24, 3000)] * 3, 1), ([(24, 3000)] * 3, 2),
                                           ([(300, 500)] * 3, 0)],
                         ids=["skinny-fused", "skinny-gram", "skinny-stepwise", "tiled"])
@pytest.mark.parametrize("prec", PRECS)
def test_deterministic_and_batch_independent(shapes, kernel, prec):
    wl = WL.small_workload("d", shapes, momentum_recipe="normal", wid=302)
    h = H.c_hparams(wl.hp, precision=prec)
    plan = B.Plan(shapes, skinny_kernel=kernel)
    b = plan.batches[0]
    arrays = H.batch_arrays(wl, b)
    r1 = H.run_gpu_step(plan, b, arrays, WL.BF16, h)
    r2 = H.run_gpu_step(plan, b, arrays, WL.BF16, h)
    for x, y in zip(r1, r2):
        assert np.array_equal(x, y), "run-to-run results differ"
    # each matrix alone gives bitwise the batched result
    single = B.Plan([shapes[0]], skinny_kernel=kernel)
    for q in range(len(shapes)):
        one = {k: v[q:q + 1].copy() for k, v in arrays.items()}
        Wq, Mq, Oq = H.run_gpu_step(single, single.batches[0], one, WL.BF16, h)
        assert np.array_equal(Oq[0], r1[2][q]) and np.array_equal(Wq[0], r1[0][q])


@pytest.mark.parametrize("shape,kernel", [((24, 900), 1), ((24, 900), 2), ((96, 260), 0)],
                         ids=["skinny-gram", "skinny-stepwise", "tiled"])
def test_transpose_symmetry(shape, kernel):
    """NS(G^T) = NS(G)^T: the tall matrix runs on the transpose."""
    wl = WL.small_workload("t", [shape], dtype=WL.F32, momentum_recipe="normal", wid=303)
    plan = B.Plan([shape], skinny_kernel=kernel)
    planT = B.Plan([shape[::-1]], skinny_kernel=kernel)
    arrays = H.batch_arrays(wl, plan.batches[0])
    arraysT = {k: np.ascontiguousarray(np.swapaxes(v, 1, 2)) for k, v in arrays.items()}
    for prec in ("bf16", "f32"):
        h = H.c_hparams(wl.hp, precision=prec)
        _, _, O = H.run_gpu_step(plan, plan.batches[0], arrays, WL.F32, h)
        _, _, OT = H.run_gpu_step(planT, planT.batches[0], arraysT, WL.F32, h)
        assert H.rel_fro(OT[0].T.astype(np.float64), O[0].astype(np.float64)) <= (1e-6 if prec == "f32" else 2e-2)


# --------------------------------------------------------------------------
# stage entry points
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shapes,kernel", [([(24, 1500), (24, 1500)], 1), ([(24, 1500), (24, 1500)], 2),
                                           ([(150, 260)], 0), ([(260, 150)], 0)],
                         ids=["skinny-gram", "skinny-stepwise", "tiled", "tiled_tall"])
def test_stage_entry_points(shapes, kernel):
    import torch
    wl = WL.small_workload("s", shapes, dtype=WL.BF16, momentum_recipe="normal", wid=304)
    plan = B.Plan(shapes, skinny_kernel=kernel)
    b = plan.batches[0]
    arrays = H.batch_arrays(wl, b)
    for prec in PRECS:
        h = H.c_hparams(wl.hp, precision=prec)
        kw = H.oracle_kwargs(h, b.M, b.N)
        g = H.to_device(arrays["grad"], WL.BF16)
        m = H.to_device(arrays["momentum"], WL.F32)
        u = torch.empty((b.count, b.M, b.N), dtype=torch.float32, device="cuda")
        B.muon_stage_momentum(plan, b.index, g, m, u, h)
        o = torch.empty_like(u)
        ws = torch.empty(plan.workspace_bytes(b.index, prec), dtype=torch.uint8, device="cuda")
        B.muon_stage_ns(plan, b.index, u, o, h, ws)
        p = H.to_device(arrays["param"], WL.BF16)
        B.muon_stage_update(plan, b.index, p, o, h)
        torch.cuda.synchronize()
        U, Mn, O, Wn = H.to_host(u), H.to_host(m), H.to_host(o), H.to_host(p)
        for q in range(b.count):
            G = H.decode(arrays["grad"][q])
            M0 = arrays["momentum"][q].astype(np.float64)
            H.check_momentum(Mn[q], M0, G, kw["momentum"])
            mu = kw["momentum"]
            Uref = G + mu * Mn[q].astype(np.float64)
            assert np.all(np.abs(U[q] - Uref) <= 1e-6 * (np.abs(G) + np.abs(mu * Mn[q])) + 1e-30)
            Oref = ORC.orthogonalize(U[q].astype(np.float64), kw["coeffs"], h.ns_steps, kw["eps"])
            assert H.rel_fro(O[q].astype(np.float64), Oref) <= H.o_tolerance(prec)
            H.check_update(Wn[q], H.decode(arrays["param"][q]), O[q].astype(np.float64), kw["lr"],
                           kw["weight_decay"], H.oracle_scale(h, b.M, b.N))


# --------------------------------------------------------------------------
# the workloads at full size
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kernel", [0, 1, 2], ids=["gram-fused", "gram", "stepwise"])
def test_fused_74x24x10240_full(kernel):
    wl = WL.WORKLOADS["fused_74x24x10240"]
    errs = check_batch(wl, H.c_hparams(wl.hp), WL.BF16, skinny_kernel=kernel)
    print(f"fused_74x24x10240 kernel {kernel}: max O error {max(errs):.3g} over {len(errs)} matrices")


def test_moe_experts_skinny_full():
    wl = WL.WORKLOADS["moe_experts"]
    plan = B.Plan([p.shape for p in wl.params])
    idx = [b.index for b in plan.batches if b.M == 24]
    errs = check_batch(wl, H.c_hparams(wl.hp), WL.BF16, plan=plan, batches=idx)
    print(f"moe [32,24,10240]: max O error {max(errs):.3g}")


def check_batch_golden(wl, plan, binfo, h, full):
    """Run one full-size batch; every matrix of it is compared at the positions
    tests/golden/full_size_samples.py stored oracle values for (O, and W' with
    the bf16 rounding of the stored W' as slack), its M' in full against the
    momentum update; the matrices `full` picks also against the whole oracle
    output.  Returns (sampled O errors, full O errors)."""
    import json
    import os
    gold = np.load(os.path.join(os.path.dirname(__file__), "golden", "full_size_samples.npz"))
    meta = json.loads(str(gold["meta"]))
    entries = {(e["workload"], e["param"], e["matrix"]): e for e in meta["entries"]}
    arrays = H.batch_arrays(wl, binfo)
    Wp, Mp, O = H.run_gpu_step(plan, binfo, arrays, WL.BF16, h)
    kw = H.oracle_kwargs(h, binfo.M, binfo.N)
    tol = H.o_tolerance(h.precision)
    sampled = []
    for q, (pi, mi) in enumerate(H.matrix_ids(binfo)):
        e = entries[(wl.name, pi, mi)]
        assert e["hparams"] == {k: (list(v) if isinstance(v, tuple) else v) for k, v in kw.items()}
        assert e["shape"] == [binfo.M, binfo.N]
        rng = np.random.default_rng(e["seed"])
        rows = rng.integers(0, binfo.M, meta["samples"])
        cols = rng.integers(0, binfo.N, meta["samples"])
        assert np.all(np.isfinite(O[q]))
        err = H.rel_fro(O[q][rows, cols].astype(np.float64), gold[e["key"] + "_O"].astype(np.float64))
        assert err <= tol, f"{wl.name} param {pi} matrix {mi}: sampled O error {err:.3g}"
        H.check_momentum(Mp[q], arrays["momentum"][q].astype(np.float64), H.decode(arrays["grad"][q]),
                         kw["momentum"])
        W_ref = gold[e["key"] + "_W"].astype(np.float64)
        W0 = H.decode(arrays["param"][q][rows, cols])
        dW_ref = W_ref - W0
        half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(W_ref), 1e-38))) - 8)
        # the stored reference W' is rounded to fp32 (2^-24 relative) on top of the bf16 slack
        slack = (np.linalg.norm(half_ulp) + 2.0 ** -24 * np.linalg.norm(W_ref)) / np.linalg.norm(dW_ref)
        ew = H.rel_fro(H.decode(Wp[q][rows, cols]) - W0, dW_ref)
        assert ew <= tol + slack + 1e-6, f"{wl.name} param {pi} matrix {mi}: sampled W' - W error {ew:.3g}"
        sampled.append(err)
    whole = [P.check_matrix(arrays["param"][q], arrays["grad"][q], arrays["momentum"][q], Wp[q], Mp[q], O[q], h,
                            f"batch {binfo.index} matrix {q}") for q in full(binfo)]
    return sampled, whole


def test_moe_experts_2048x7168_sampled():
    """Both [32, 2048, 7168] batches of the MoE expert tensor at full size: all
    64 experts at stored oracle positions, three of them against the whole
    oracle output."""
    wl = WL.WORKLOADS["moe_experts"]
    plan = B.Plan([p.shape for p in wl.params])
    rng = np.random.default_rng(7)
    for b in [b for b in plan.batches if b.M == 2048]:
        sampled, whole = check_batch_golden(wl, plan, b, H.c_hparams(wl.hp),
                                            lambda b: sorted({0, b.count - 1, int(rng.integers(1, b.count - 1))}))
        print(f"moe batch {b.index} [{b.count},2048,7168]: sampled O errors max {max(sampled):.3g} "
              f"over {len(sampled)}, whole-matrix O errors {whole}")


# --------------------------------------------------------------------------
# full-size configurations, sampled
# --------------------------------------------------------------------------
def test_decoder_full_size_sampled():
    """One full-size batch per decoder shape (32 x 4096x4096, 10 x 11008x4096
    through the transpose path, 10 x 4096x11008), as the plan cuts them: every
    matrix at stored oracle positions, the last of each against the whole
    oracle output."""
    wl = WL.WORKLOADS["decoder32_h4096_f11008"]
    plan = B.Plan([p.shape for p in wl.params])
    pick = {}
    for b in plan.batches:
        if (b.M, b.N) not in pick or b.count < pick[(b.M, b.N)].count:
            pick[(b.M, b.N)] = b
    assert len(pick) == 3
    for b in pick.values():
        sampled, whole = check_batch_golden(wl, plan, b, H.c_hparams(wl.hp), lambda b: [b.count - 1])
        print(f"decoder batch {b.index} [{b.count},{b.M},{b.N}]: sampled O errors max {max(sampled):.3g} "
              f"over {len(sampled)}, whole-matrix O errors {whole}")


@pytest.mark.parametrize("prec", ["bf16_x32", "bf16_x32c"])
def test_large_8192x28672_golden_samples(prec):
    """The first batch of each orientation of the 8192x28672 workload at full
    size (two matrices each, bf16 products with the master of X, and with the
    compensating half); both matrices of each are compared at 4096 positions
    with oracle values stored by tests/golden/large_8192x28672_samples.py (O
    and W'; the main file holds matrix 0 of each batch, the extra file matrix
    1), and their M' in full against the momentum update."""
    import json
    import os
    here = os.path.join(os.path.dirname(__file__), "golden")
    golds = [np.load(os.path.join(here, f)) for f in ("large_8192x28672_samples.npz",
                                                      "large_8192x28672_extra_samples.npz")]
    per_param = {}
    for gold in golds:
        meta = json.loads(str(gold["meta"]))
        for pi in meta["params"]:
            per_param[pi] = (gold, meta)
    wl = WL.WORKLOADS[meta["workload"]]
    h = H.c_hparams(wl.hp, precision=prec)
    plan = B.Plan([p.shape for p in wl.params])
    by_batch = {}
    for pi, (gold, meta) in per_param.items():
        assert meta["hparams"] == {k: (list(v) if isinstance(v, tuple) else v)
                                   for k, v in H.oracle_kwargs(h, 8192, 28672).items()}
        binfo = next(b for b in plan.batches if any(s[0] == pi and s[1] == 0 for s in b.segments))
        by_batch.setdefault(binfo.index, (binfo, []))[1].append(pi)
    assert len(by_batch) == 2 and all(len(v[1]) == 2 for v in by_batch.values())
    for binfo, params in by_batch.values():
        arrays = H.batch_arrays(wl, binfo)
        Wp, Mp, O = H.run_gpu_step(plan, binfo, arrays, WL.BF16, h)
        for pi in params:
            gold, meta = per_param[pi]
            q = next(s[3] // (binfo.M * binfo.N) for s in binfo.segments if s[0] == pi and s[1] == 0)
            # M' over the whole matrix (the oracle's momentum update is elementwise)
            H.check_momentum(Mp[q], arrays["momentum"][q].astype(np.float64), H.decode(arrays["grad"][q]),
                             H.f32(h.momentum))
            rows, cols = gold[f"p{pi}_rows"], gold[f"p{pi}_cols"]
            o = O[q][rows, cols].astype(np.float64)
            e = H.rel_fro(o, gold[f"p{pi}_O"])
            print(f"large param {pi} ({binfo.M}x{binfo.N}, batch of {binfo.count}): sampled O error {e:.3g}")
            assert np.all(np.isfinite(O[q]))
            assert e <= H.o_tolerance(h.precision)
            W0 = H.decode(arrays["param"][q][rows, cols])
            dW = H.decode(Wp[q][rows, cols]) - W0
            dW_ref = gold[f"p{pi}_W"] - W0
            half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(gold[f"p{pi}_W"]), 1e-38))) - 8)
            slack = np.linalg.norm(half_ulp) / np.linalg.norm(dW_ref)
            assert H.rel_fro(dW, dW_ref) <= H.o_tolerance(h.precision) + slack + 1e-6
        del arrays, Wp, Mp, O
