"""muon_step_noalloc, the entry point for callers that cannot allocate device
memory: the step with its workspace in the library's static device array.

Two calls in a row through the C ABI, the second on a smaller batch (a
smaller workspace, another path), each against muon_step on the same seeded
inputs with a caller-allocated workspace: bitwise equal W', M' and O, and
within the oracle's parity bars (tests/parity.py).  A batch whose workspace
exceeds the static array is refused with MUON_ERR_WORKSPACE_TOO_SMALL and
leaves its buffers untouched.
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


def _one(shapes, prec, wid):
    import torch
    wl = WL.small_workload("noalloc", shapes, momentum_recipe="normal", wid=wid)
    plan = B.Plan(shapes)
    assert len(plan.batches) == 1
    b = plan.batches[0]
    need = plan.workspace_bytes(0, prec)
    assert need <= B.NOALLOC_SCRATCH_BYTES
    h = B.HParams(precision=prec)
    arr = H.batch_arrays(wl, b)
    ref = [H.to_device(arr["param"], WL.BF16), H.to_device(arr["grad"], WL.BF16), H.to_device(arr["momentum"], WL.F32),
           torch.zeros((b.count, b.M, b.N), dtype=torch.float32, device="cuda")]
    mine = [t.clone() for t in ref]
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    B.muon_step(plan, 0, ref[0], ref[1], ref[2], h, ws, ns_out=ref[3])
    B.muon_step_noalloc(plan, 0, mine[0], mine[1], mine[2], h, ns_out=mine[3])
    torch.cuda.synchronize()
    for k, name in enumerate(("param", "grad", "momentum", "O")):
        assert torch.equal(mine[k], ref[k]), (shapes, prec, name)
    Wp, Mp, O = H.to_host(mine[0]), H.to_host(mine[2]), H.to_host(mine[3])
    for q in range(b.count):
        P.check_matrix(arr["param"][q], arr["grad"][q], arr["momentum"][q], Wp[q], Mp[q], O[q], h,
                       f"noalloc {shapes[0]} {prec} matrix {q}")
    return need


def test_noalloc_two_calls_second_smaller():
    first = _one([(24, 10240)] * 40, "bf16", 600)          # skinny, one launch for the iteration and the apply
    second = _one([(2, 300, 500)], "bf16_x32", 601)         # tiled, smaller workspace
    assert second < first


def test_noalloc_refuses_oversize_batch():
    import torch
    plan = B.Plan([(4096, 4096)])
    assert plan.workspace_bytes(0, "bf16") > B.NOALLOC_SCRATCH_BYTES
    p = torch.full((1, 4096, 4096), 0.5, dtype=torch.bfloat16, device="cuda")
    g = torch.ones_like(p)
    m = torch.zeros((1, 4096, 4096), dtype=torch.float32, device="cuda")
    with pytest.raises(B.MuonError) as ei:
        B.muon_step_noalloc(plan, 0, p, g, m, B.HParams())
    assert ei.value.status == B.MUON_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((p == 0.5).all()) and bool((m == 0).all())
