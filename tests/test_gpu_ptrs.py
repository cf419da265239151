"""muon_step_ptrs: a batch whose matrices sit at independent addresses (one
pointer per matrix, no packing).  Inputs come from the seeded generator
(workloads.py); the result is checked against the float64 oracle
(tests/parity.py bars: O, M', W' per matrix) and bitwise against muon_step
on the same values packed into [count, M, N] buffers.

The per-matrix tensors are carved out of one allocation in reverse order with
gaps, so their addresses are neither contiguous nor increasing.  Skinny (both
Newton-Schulz forms, both orientations), 128 x 128 and 256 x 256 tiled
batches, expert tensors, bf16 and fp32 parameters, and all precisions.
"""
import pytest

from matrix_optimizer_amd import binding as B
from matrix_optimizer_amd import workloads as WL
from tests import harness as H
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = [
    ("skinny", [(24, 1000)] * 3, 0),
    ("skinny_stepwise", [(24, 1000)] * 3, 2),
    ("skinny_tall", [(700, 20)] * 2, 0),
    ("tiled_128", [(150, 260), (150, 260)], 0),
    ("tiled_256_tall", [(900, 700), (900, 700)], 0),
    ("experts", [(3, 200, 72)], 0),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _scattered(count, M, N, dtype, gap=64):
    """count [M, N] views of one allocation, in reverse order with gaps
    (16-byte aligned: M N + gap elements apart, both multiples of 8)."""
    import torch
    per = ((M * N + 7) // 8) * 8 + gap
    base = torch.empty(count * per + gap, dtype=dtype, device="cuda")
    return [base[(count - 1 - i) * per + gap:(count - 1 - i) * per + gap + M * N].view(M, N) for i in range(count)]


@pytest.mark.parametrize("prec", ["bf16", "bf16_x32", "bf16_x32c", "f32"])
@pytest.mark.parametrize("pdtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,shapes,kernel", CASES, ids=[c[0] for c in CASES])
def test_step_ptrs_matches_oracle_and_packed(name, shapes, kernel, pdtype, prec):
    import torch
    dt = torch.bfloat16 if pdtype == "bf16" else torch.float32
    wdt = WL.BF16 if pdtype == "bf16" else WL.F32
    plan = B.Plan(shapes, skinny_kernel=kernel)
    hp = B.HParams(precision=prec)
    wl = WL.small_workload(name, shapes, dtype=wdt, momentum_recipe="normal",
                           wid=520 + [c[0] for c in CASES].index(name))
    for bi, b in enumerate(plan.batches):
        cnt, M, N = b.count, b.M, b.N
        arr = H.batch_arrays(wl, b)
        Pk, G, Mo = H.to_device(arr["param"], wdt), H.to_device(arr["grad"], wdt), H.to_device(arr["momentum"], WL.F32)
        O = torch.zeros(cnt, M, N, device="cuda")
        ws = torch.zeros(plan.workspace_bytes(bi, prec), dtype=torch.uint8, device="cuda")

        ps, gs, ms, os_ = (_scattered(cnt, M, N, dt), _scattered(cnt, M, N, dt),
                           _scattered(cnt, M, N, torch.float32), _scattered(cnt, M, N, torch.float32))
        for i in range(cnt):
            ps[i].copy_(Pk[i]); gs[i].copy_(G[i]); ms[i].copy_(Mo[i]); os_[i].zero_()
        ws2 = torch.zeros_like(ws)

        B.muon_step(plan, bi, Pk, G, Mo, hp, ws, ns_out=O)
        B.muon_step_ptrs(plan, bi, ps, gs, ms, hp, ws2, ns_out=os_)
        torch.cuda.synchronize()
        for i in range(cnt):
            assert torch.equal(ps[i], Pk[i]), (name, bi, i, "param")
            assert torch.equal(ms[i], Mo[i]), (name, bi, i, "momentum")
            assert torch.equal(os_[i], O[i]), (name, bi, i, "O")
            P.check_matrix(arr["param"][i], arr["grad"][i], arr["momentum"][i], H.to_host(ps[i]),
                           H.to_host(ms[i]), H.to_host(os_[i]), hp, f"{name} {pdtype} {prec} batch {bi} matrix {i}")


def test_step_ptrs_tables_reused_across_steps():
    """Pointer tables made once serve every later step (they hold addresses,
    not data): two steps through the same tables equal two packed steps."""
    import torch
    shapes = [(24, 3000)] * 2
    plan = B.Plan(shapes)
    hp = B.HParams()
    b = plan.batches[0]
    gen = torch.Generator(device="cuda").manual_seed(3)
    P = torch.randn(b.count, b.M, b.N, device="cuda", generator=gen).mul_(0.02).to(torch.bfloat16)
    Mo = torch.zeros(b.count, b.M, b.N, device="cuda")
    ps, gs, ms = (_scattered(b.count, b.M, b.N, torch.bfloat16), _scattered(b.count, b.M, b.N, torch.bfloat16),
                  _scattered(b.count, b.M, b.N, torch.float32))
    for i in range(b.count):
        ps[i].copy_(P[i]); ms[i].zero_()
    tp, tg, tm = B.pointer_table(ps), B.pointer_table(gs), B.pointer_table(ms)
    ws = torch.zeros(plan.workspace_bytes(0), dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros_like(ws)
    for _ in range(2):
        G = torch.randn(b.count, b.M, b.N, device="cuda", generator=gen).to(torch.bfloat16)
        for i in range(b.count):
            gs[i].copy_(G[i])
        B.muon_step(plan, 0, P, G, Mo, hp, ws)
        B.muon_step_ptrs(plan, 0, tp, tg, tm, hp, ws2, param_dtype="bf16", grad_dtype="bf16")
    torch.cuda.synchronize()
    for i in range(b.count):
        assert torch.equal(ps[i], P[i]) and torch.equal(ms[i], Mo[i])
