"""muon_step captured into a HIP graph and replayed.

The captured step is replayed several times with eager work, new gradients
and synchronisations in between, and with new lr / weight-decay values written
to the device scalars (muon_hparams.lr_wd_device) before each replay.  Every
replay is checked two ways:
* against the float64 oracle (tests/parity.py bars: O, M', W') on the
  replay's own inputs, which come from the seeded generator
  (matrix_optimizer_amd/workloads.py) for the first replay and are the
  previous replay's W' and M' with new seeded gradients after that;
* bitwise against the same step run eagerly with those values passed on the
  host.
Skinny (both the Gram-space and the transposed form) and tiled batches are
covered, with the batches on one stream and spread over two
(muon_step_batches: the side stream forks from and joins the capture stream
inside the graph).
"""
import pytest

from matrix_optimizer_amd import binding as B
from matrix_optimizer_amd import workloads as WL
from tests import harness as H
from tests import parity as P

pytestmark = pytest.mark.gpu

SHAPES = [(24, 3000)] * 3 + [(3000, 24)] + [(160, 200)] * 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _fill(bm, wl, kinds):
    """Copy the workload's stored values into a BatchedMuon's batch buffers."""
    for b in bm.plan.batches:
        arr = H.batch_arrays(wl, b, kinds)
        for kind in kinds:
            dst = {"param": bm.params, "grad": bm.grads, "momentum": bm.moms}[kind][b.index]
            dst.copy_(H.to_device(arr[kind], WL.F32 if kind == "momentum" else WL.BF16))


@pytest.mark.parametrize("streams", [1, 2])
@pytest.mark.parametrize("prec", ["bf16", "bf16_x32c", "f32"])
def test_graph_replays_match_eager_and_oracle(prec, streams):
    import torch
    wl = WL.small_workload("graph", SHAPES, momentum_recipe="normal", wid=500)
    lr_wd = torch.tensor([0.02, 0.1], dtype=torch.float32, device="cuda")
    graphed = B.BatchedMuon(SHAPES, torch.bfloat16, B.HParams(precision=prec, lr_wd=lr_wd), streams=streams)
    eager = B.BatchedMuon(SHAPES, torch.bfloat16, B.HParams(precision=prec))
    kinds = ("param", "grad", "momentum")
    _fill(graphed, wl, kinds)
    _fill(eager, wl, kinds)
    outs = [torch.zeros((b.count, b.M, b.N), dtype=torch.float32, device="cuda") for b in graphed.plan.batches]
    graph = graphed.capture_graph(outs)
    torch.cuda.synchronize()
    for i in range(len(graphed.params)):   # capturing runs nothing
        assert torch.equal(graphed.params[i], eager.params[i]) and torch.equal(graphed.moms[i], eager.moms[i])

    for rep, (lr, wd) in enumerate([(0.02, 0.1), (0.05, 0.0), (0.01, 0.3), (0.02, 0.1)]):
        inputs = [(H.to_host(graphed.params[i]), H.to_host(graphed.grads[i]), H.to_host(graphed.moms[i]))
                  for i in range(len(graphed.params))]
        lr_wd.copy_(torch.tensor([lr, wd], dtype=torch.float32))
        graph.replay()
        eager.hp = B.HParams(precision=prec, lr=lr, weight_decay=wd)
        eager.step()
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")   # unrelated eager work
        torch.cuda.synchronize()
        for i in range(len(graphed.params)):
            assert torch.equal(graphed.params[i], eager.params[i]), (prec, streams, rep, i)
            assert torch.equal(graphed.moms[i], eager.moms[i]), (prec, streams, rep, i)
        h = B.HParams(precision=prec, lr=lr, weight_decay=wd)
        for b in graphed.plan.batches:
            W0, G0, M0 = inputs[b.index]
            Wp, Mp, O = H.to_host(graphed.params[b.index]), H.to_host(graphed.moms[b.index]), H.to_host(outs[b.index])
            for q in range(b.count):
                P.check_matrix(W0[q], G0[q], M0[q], Wp[q], Mp[q], O[q], h,
                               f"{prec} streams {streams} replay {rep} batch {b.index} matrix {q}")
        # next step's gradients: a fresh seeded draw
        nxt = WL.small_workload("graph", SHAPES, momentum_recipe="normal", wid=501 + rep)
        _fill(graphed, nxt, ("grad",))
        for i in range(len(graphed.params)):
            eager.grads[i].copy_(graphed.grads[i])
        del junk
