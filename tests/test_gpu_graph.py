"""muon_step captured into a HIP graph and replayed.

The captured step is replayed several times with eager work, new gradients
and synchronisations in between, and with new lr / weight-decay values written
to the device scalars (muon_hparams.lr_wd_device) before each replay; every
replay must leave parameters and momentum bit-identical to the same step run
eagerly with those values passed on the host.  Skinny (both the Gram-space
and the transposed form) and tiled batches are covered, with the batches on
one stream and spread over two (muon_step_batches: the side stream forks from
and joins the capture stream inside the graph).
"""
import pytest

from matrix_optimizer_amd import binding as B

pytestmark = pytest.mark.gpu

SHAPES = [(24, 3000)] * 3 + [(3000, 24)] + [(160, 200)] * 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


@pytest.mark.parametrize("streams", [1, 2])
@pytest.mark.parametrize("prec", ["bf16", "f32"])
def test_graph_replays_match_eager(prec, streams):
    import torch
    gen = torch.Generator(device="cuda").manual_seed(5)
    lr_wd = torch.tensor([0.02, 0.1], dtype=torch.float32, device="cuda")
    graphed = B.BatchedMuon(SHAPES, torch.bfloat16, B.HParams(precision=prec, lr_wd=lr_wd), streams=streams)
    eager = B.BatchedMuon(SHAPES, torch.bfloat16, B.HParams(precision=prec))
    for i in range(len(graphed.params)):
        graphed.params[i].normal_(0.0, 0.02, generator=gen)
        graphed.grads[i].normal_(generator=gen)
        graphed.moms[i].normal_(generator=gen)
        eager.params[i].copy_(graphed.params[i])
        eager.grads[i].copy_(graphed.grads[i])
        eager.moms[i].copy_(graphed.moms[i])
    graph = graphed.capture_graph()
    torch.cuda.synchronize()
    for i in range(len(graphed.params)):   # capturing runs nothing
        assert torch.equal(graphed.params[i], eager.params[i]) and torch.equal(graphed.moms[i], eager.moms[i])

    for rep, (lr, wd) in enumerate([(0.02, 0.1), (0.05, 0.0), (0.01, 0.3), (0.02, 0.1)]):
        lr_wd.copy_(torch.tensor([lr, wd], dtype=torch.float32))
        graph.replay()
        eager.hp = B.HParams(precision=prec, lr=lr, weight_decay=wd)
        eager.step()
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")   # unrelated eager work
        torch.cuda.synchronize()
        for i in range(len(graphed.params)):
            assert torch.equal(graphed.params[i], eager.params[i]), (prec, streams, rep, i)
            assert torch.equal(graphed.moms[i], eager.moms[i]), (prec, streams, rep, i)
        for i in range(len(graphed.params)):   # next step's gradients
            graphed.grads[i].normal_(generator=gen)
            eager.grads[i].copy_(graphed.grads[i])
        del junk
