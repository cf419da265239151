"""The fused Gram-space form (plan option skinny_kernel = 3, the default's
form: the Newton-Schulz on the Gram matrix and the apply in one launch) gives
bitwise the parameters, momentum and O of the three-launch form
(skinny_kernel = 1), which the parity tests check against the oracle.  Both
form Q and apply it with the same arithmetic; only the launch structure
differs.

Cases: wide shapes with full and ragged 64-column units, an odd unit count,
rows that are not a multiple of 8 (no 16-byte vectors), a single unit, 1 and
32 rows, expert tensors, batches large enough that each matrix gets one
workgroup (16-wave workgroups) and small ones (8-wave), tall shapes (W stored
as the transpose of U: short sides that are and are not a multiple of 4, 32
rows, many matrices), all three precisions (8-wave workgroups for the fp32
operands), bf16 and fp32 parameters; the update without O, O without the
update (the stage call), pointer tables and row tables of both orientations.
"""
import numpy as np
import pytest

from matrix_optimizer_amd import binding as B

pytestmark = pytest.mark.gpu

CASES = [
    ("wide", [(24, 10240)] * 5),
    ("ragged", [(24, 1000)] * 3),
    ("odd_units", [(20, 2100)] * 2),
    ("not_vec", [(7, 333)] * 4),
    ("one_unit", [(24, 64)] * 3),
    ("one_row", [(1, 50)] * 2),
    ("rows32", [(32, 4096)] * 2),
    ("experts", [(3, 17, 2000)]),
    ("many", [(8, 256)] * 600),
    ("tall", [(700, 20)] * 2),
    ("tall_not_vec", [(500, 7)] * 3),
    ("tall_rows32", [(2048, 32)] * 2),
    ("tall_many", [(300, 8)] * 300),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _inputs(b, dt, seed):
    import torch
    gen = torch.Generator(device="cuda").manual_seed(seed)
    P = torch.randn(b.count, b.M, b.N, device="cuda", generator=gen).mul_(0.02).to(dt)
    G = torch.randn(b.count, b.M, b.N, device="cuda", generator=gen).to(dt)
    Mo = torch.randn(b.count, b.M, b.N, device="cuda", generator=gen)
    return P, G, Mo


def _run(kernel, shapes, prec, dt, seed, with_o=True, with_p=True):
    import torch
    plan = B.Plan(shapes, skinny_kernel=kernel)
    hp = B.HParams(precision=prec)
    out = []
    for b in plan.batches:
        P, G, Mo = _inputs(b, dt, seed + b.index)
        O = torch.zeros(b.count, b.M, b.N, device="cuda") if with_o else None
        ws = torch.empty(plan.workspace_bytes(b.index, prec), dtype=torch.uint8, device="cuda")
        if with_p:
            B.muon_step(plan, b.index, P, G, Mo, hp, ws, ns_out=O)
        else:
            U = (G.float() + Mo)
            B.muon_stage_ns(plan, b.index, U, O, hp, ws)
        out.append((P, Mo, O))
    torch.cuda.synchronize()
    return plan, out


@pytest.mark.parametrize("prec", ["bf16", "bf16_x32", "f32"])
@pytest.mark.parametrize("pdtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,shapes", CASES, ids=[c[0] for c in CASES])
def test_fused_matches_three_launches(name, shapes, pdtype, prec):
    import torch
    dt = torch.bfloat16 if pdtype == "bf16" else torch.float32
    p1, r1 = _run(1, shapes, prec, dt, seed=5)
    p3, r3 = _run(3, shapes, prec, dt, seed=5)
    assert [(b.M, b.N, b.count, b.path) for b in p1.batches] == [(b.M, b.N, b.count, b.path) for b in p3.batches]
    for (Pa, Ma, Oa), (Pb, Mb, Ob) in zip(r1, r3):
        assert torch.equal(Pa, Pb) and torch.equal(Ma, Mb) and torch.equal(Oa, Ob), name


@pytest.mark.parametrize("name,shapes", [CASES[0], CASES[1], CASES[3]], ids=["wide", "ragged", "not_vec"])
def test_fused_update_only_and_o_only(name, shapes):
    import torch
    for prec in ("bf16", "f32"):
        _, r1 = _run(1, shapes, prec, torch.bfloat16, seed=9, with_o=False)
        _, r3 = _run(3, shapes, prec, torch.bfloat16, seed=9, with_o=False)
        for (Pa, Ma, _), (Pb, Mb, _) in zip(r1, r3):
            assert torch.equal(Pa, Pb) and torch.equal(Ma, Mb)
        _, r1 = _run(1, shapes, prec, torch.bfloat16, seed=9, with_p=False)
        _, r3 = _run(3, shapes, prec, torch.bfloat16, seed=9, with_p=False)
        for (_, _, Oa), (_, _, Ob) in zip(r1, r3):
            assert torch.equal(Oa, Ob)


def _scattered(count, M, N, dtype, gap=64):
    import torch
    per = ((M * N + 7) // 8) * 8 + gap
    base = torch.empty(count * per + gap, dtype=dtype, device="cuda")
    return [base[(count - 1 - i) * per + gap:(count - 1 - i) * per + gap + M * N].view(M, N) for i in range(count)]


@pytest.mark.parametrize("prec", ["bf16", "bf16_x32", "f32"])
@pytest.mark.parametrize("shape", [(24, 3000), (3000, 24)], ids=["wide", "tall"])
def test_fused_pointer_and_row_tables(prec, shape):
    """Pointer tables and row tables (rows in reverse order, gaps between
    them) through the fused launch equal the packed three-launch step."""
    import torch
    shapes = [shape] * 3
    hp = B.HParams(precision=prec)
    p1 = B.Plan(shapes, skinny_kernel=1)
    p3 = B.Plan(shapes, skinny_kernel=3)
    b = p1.batches[0]
    P, G, Mo = _inputs(b, torch.bfloat16, 21)
    ws = torch.empty(p1.workspace_bytes(0, prec), dtype=torch.uint8, device="cuda")
    ref = [P.clone(), Mo.clone()]
    B.muon_step(p1, 0, ref[0], G, ref[1], hp, ws)
    # pointer tables
    ps, gs, ms = (_scattered(b.count, b.M, b.N, torch.bfloat16), _scattered(b.count, b.M, b.N, torch.bfloat16),
                  _scattered(b.count, b.M, b.N, torch.float32))
    for i in range(b.count):
        ps[i].copy_(P[i]); gs[i].copy_(G[i]); ms[i].copy_(Mo[i])
    ws3 = torch.empty(p3.workspace_bytes(0, prec), dtype=torch.uint8, device="cuda")
    B.muon_step_ptrs(p3, 0, ps, gs, ms, hp, ws3)
    # row tables: every stored row at its own address, rows of a matrix in reverse order
    Wrows = torch.empty(b.count * b.M, b.N + 16, dtype=torch.bfloat16, device="cuda")
    Grows = torch.empty_like(Wrows)
    wv = [[Wrows[i * b.M + (b.M - 1 - r), 8:8 + b.N] for r in range(b.M)] for i in range(b.count)]
    gv = [[Grows[i * b.M + (b.M - 1 - r), 8:8 + b.N] for r in range(b.M)] for i in range(b.count)]
    for i in range(b.count):
        for r in range(b.M):
            wv[i][r].copy_(P[i, r]); gv[i][r].copy_(G[i, r])
    M2 = Mo.clone()
    ws4 = torch.empty_like(ws3)
    tw = torch.tensor([t.data_ptr() for rows in wv for t in rows], dtype=torch.int64, device="cuda")
    tg = torch.tensor([t.data_ptr() for rows in gv for t in rows], dtype=torch.int64, device="cuda")
    B.muon_step_rows(p3, 0, tw, tg, M2, hp, ws4, "bf16", "bf16")
    torch.cuda.synchronize()
    for i in range(b.count):
        assert torch.equal(ps[i], ref[0][i]) and torch.equal(ms[i], ref[1][i])
        assert torch.equal(torch.stack(wv[i]), ref[0][i]) and torch.equal(M2[i], ref[1][i])
