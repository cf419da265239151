"""muon_step_rows: logical matrices that are row-level views of fused
physical parameters (the model-adapter views of HyperParallel-FSDP §6.6).

The physical parameters and gradients, and the logical matrices' momentum,
come from the seeded generator (workloads.py).  The logical matrices' W', M'
and O are checked against the float64 oracle (tests/parity.py bars) and
bitwise against muon_step on the same matrices packed, and every physical
element outside them must be untouched.

Layouts: a fused QKV weight with heads interleaved, column splits with gaps
(square, and tall on 256 x 256 tiles),
an MoE FC1 weight with gate and up rows interleaved (tall matrices), and row
and column splits of skinny matrices; bf16 and fp32 parameters, all
precisions, both skinny Newton-Schulz forms.
"""
import pytest

from matrix_optimizer_amd import binding as B
from matrix_optimizer_amd import workloads as WL
from tests import harness as H
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _qkv_interleaved(t):
    """[3H, H] with rows [head][q|k|v][d]: heads 4, d 64 -> three [256, 256]."""
    v = t.view(4, 3, 64, t.shape[-1])
    return [v[:, k] for k in range(3)]


def _column_split_gaps(t):
    """[200, 616]: columns 0..199, 208..407, 416..615 -> three [200, 200]."""
    return [t[:, 208 * k:208 * k + 200] for k in range(3)]


def _gate_up_interleaved(t):
    """[2 experts, 2 x 300, 72], gate and up rows alternating -> four [300, 72]."""
    return [t[e, k::2] for e in range(2) for k in range(2)]


def _skinny_rows(t):
    """[72, 1000] -> three [24, 1000] row blocks."""
    return [t[24 * k:24 * k + 24] for k in range(3)]


def _skinny_columns_tall(t):
    """[1000, 72] -> three [1000, 24] column ranges (tall: stored rows are 24 long)."""
    return [t[:, 24 * k:24 * k + 24] for k in range(3)]


def _tall_column_split(t):
    """[768, 528]: columns 0..255 and 272..527 -> two tall [768, 256] (256 x 256
    tiles, W stored as the transpose of X)."""
    return [t[:, 0:256], t[:, 272:528]]


CASES = [
    ("qkv_interleaved", (768, 256), _qkv_interleaved, (256, 256), (0,)),
    ("tall_column_split", (768, 528), _tall_column_split, (768, 256), (0,)),
    ("column_split_gaps", (200, 616), _column_split_gaps, (200, 200), (0,)),
    ("gate_up_interleaved", (2, 600, 72), _gate_up_interleaved, (300, 72), (0,)),
    ("skinny_rows", (72, 1000), _skinny_rows, (24, 1000), (0, 2)),
    ("skinny_columns_tall", (1000, 72), _skinny_columns_tall, (1000, 24), (0, 2)),
]


@pytest.mark.parametrize("prec", ["bf16", "bf16_x32", "bf16_x32c", "f32"])
@pytest.mark.parametrize("pdtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,phys,split,mshape,kernels", CASES, ids=[c[0] for c in CASES])
def test_step_rows_matches_oracle_and_packed(name, phys, split, mshape, kernels, pdtype, prec):
    import numpy as np
    import torch
    dt = torch.bfloat16 if pdtype == "bf16" else torch.float32
    wdt = WL.BF16 if pdtype == "bf16" else WL.F32
    case = [c[0] for c in CASES].index(name)
    for kernel in kernels:
        wl = WL.small_workload(name, [phys], dtype=wdt, wid=530 + 10 * case + kernel)
        Wp = H.to_device(wl.tensor(0, "param"), wdt)
        Gp = H.to_device(wl.tensor(0, "grad"), wdt)
        assert Wp.dtype == dt and tuple(Wp.shape) == tuple(phys)
        W0 = Wp.clone()
        views_w, views_g = split(Wp), split(Gp)
        count = len(views_w)
        M, N = mshape
        assert all(tuple(v.reshape(-1, v.shape[-1]).shape) == (M, N) for v in views_w)
        plan = B.Plan([mshape] * count, skinny_kernel=kernel)
        assert len(plan.batches) == 1 and plan.batches[0].count == count
        hp = B.HParams(precision=prec)
        Pk = torch.stack([v.reshape(M, N) for v in views_w])   # packed copies
        G = torch.stack([v.reshape(M, N) for v in views_g])
        wlm = WL.small_workload(name + "_momentum", [mshape] * count, momentum_recipe="normal",
                                wid=531 + 10 * case + kernel)
        M0 = np.stack([wlm.matrix(i, 0, "momentum") for i in range(count)])
        Mo = H.to_device(M0, WL.F32)
        W0s, G0s = H.to_host(Pk), H.to_host(G)
        Mo2 = Mo.clone()
        O, O2 = torch.zeros_like(Mo), torch.zeros_like(Mo)
        ws = torch.zeros(plan.workspace_bytes(0, prec), dtype=torch.uint8, device="cuda")
        ws2 = torch.zeros_like(ws)
        B.muon_step(plan, 0, Pk, G, Mo, hp, ws, ns_out=O)
        tw, tg = B.row_table(views_w), B.row_table(views_g)
        B.muon_step_rows(plan, 0, tw, tg, Mo2, hp, ws2, pdtype, pdtype, ns_out=O2)
        torch.cuda.synchronize()
        for i, v in enumerate(views_w):
            assert torch.equal(v.reshape(M, N), Pk[i]), (name, kernel, i, "param")
        assert torch.equal(Mo2, Mo) and torch.equal(O2, O), (name, kernel)
        # the logical matrices as updated in place in the physical parameter
        Wl = H.to_host(torch.stack([v.reshape(M, N) for v in views_w]))
        Ml, Ol = H.to_host(Mo2), H.to_host(O2)
        for i in range(count):
            P.check_matrix(W0s[i], G0s[i], M0[i], Wl[i], Ml[i], Ol[i], hp,
                           f"{name} {pdtype} {prec} kernel {kernel} matrix {i}")
        # physical elements outside every logical matrix are untouched
        mask = torch.ones(phys, dtype=torch.bool, device="cuda")
        for v in split(mask):
            v.fill_(False)
        assert torch.equal(Wp[mask], W0[mask]), (name, kernel, "outside")
        # and the gradient is only read
        assert torch.equal(torch.stack([v.reshape(M, N) for v in views_g]), G)


def test_step_rows_without_ns_out():
    """The update alone (no O written) through row tables, against muon_step."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(5)
    Wp = torch.randn(768, 256, device="cuda", generator=gen).mul_(0.02).to(torch.bfloat16)
    Gp = torch.randn(768, 256, device="cuda", generator=gen).to(torch.bfloat16)
    vw, vg = _qkv_interleaved(Wp), _qkv_interleaved(Gp)
    plan = B.Plan([(256, 256)] * 3)
    hp = B.HParams()
    P = torch.stack([v.reshape(256, 256) for v in vw])
    G = torch.stack([v.reshape(256, 256) for v in vg])
    Mo = torch.zeros(3, 256, 256, device="cuda")
    Mo2 = Mo.clone()
    ws = torch.zeros(plan.workspace_bytes(0), dtype=torch.uint8, device="cuda")
    B.muon_step(plan, 0, P, G, Mo, hp, ws)
    B.muon_step_rows(plan, 0, B.row_table(vw), B.row_table(vg), Mo2, hp, torch.zeros_like(ws), "bf16", "bf16")
    torch.cuda.synchronize()
    for i, v in enumerate(vw):
        assert torch.equal(v.reshape(256, 256), P[i]), i
    assert torch.equal(Mo2, Mo)
