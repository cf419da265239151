"""muon_step_batches: the batches of a plan spread over several streams.

The plan mixes tiled batches (128 x 128 and 256 x 256 tiles, a transposed
one), skinny batches in both orientations and an expert tensor, with a batch
cap that splits one shape into two batches, so lanes hold batches of every
path.  Inputs come from the seeded generator (workloads.py).  The
multi-stream step is checked against the float64 oracle (tests/parity.py
bars: O, M', W' per matrix) and bitwise against muon_step run on each batch
in turn: lanes run concurrently on separate workspaces, and every kernel's
reductions have a fixed order, so overlap changes no bit.
"""
import pytest

from matrix_optimizer_amd import binding as B
from matrix_optimizer_amd import workloads as WL
from tests import harness as H
from tests import parity as P

pytestmark = pytest.mark.gpu

SHAPES = ([(300, 700)] * 3 + [(24, 1000)] * 4 + [(1000, 20)] + [(3, 200, 72)] + [(512, 768)] * 2
          + [(900, 256)])
CAP = 2 * 300 * 700


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _filled(plan, dtype, seed):
    import torch
    gen = torch.Generator(device="cuda").manual_seed(seed)
    out = []
    for b in plan.batches:
        shp = (b.count, b.M, b.N)
        out.append((torch.randn(shp, device="cuda", generator=gen).mul_(0.02).to(dtype),
                    torch.randn(shp, device="cuda", generator=gen).to(dtype),
                    torch.randn(shp, device="cuda", generator=gen),
                    torch.zeros(shp, device="cuda")))
    return out


def _seeded(plan, wl):
    """Per-batch (param, grad, momentum, O) device buffers holding the seeded
    generator's values, and the stored host arrays they came from."""
    import torch
    dev, host = [], []
    for b in plan.batches:
        arr = H.batch_arrays(wl, b)
        host.append(arr)
        dev.append((H.to_device(arr["param"], WL.BF16), H.to_device(arr["grad"], WL.BF16),
                    H.to_device(arr["momentum"], WL.F32),
                    torch.zeros((b.count, b.M, b.N), dtype=torch.float32, device="cuda")))
    return dev, host


@pytest.mark.parametrize("prec", ["bf16", "bf16_x32", "bf16_x32c", "f32"])
@pytest.mark.parametrize("streams", [2, 3])
def test_step_batches_matches_oracle_and_sequential(streams, prec):
    import torch
    plan = B.Plan(SHAPES, max_batch_elems=CAP)
    assert len(plan.batches) >= 6 and {b.path for b in plan.batches} >= {0, 1}
    hp = B.HParams(precision=prec)
    wl = WL.small_workload("batches", SHAPES, momentum_recipe="normal", wid=510)
    ref, host = _seeded(plan, wl)
    mine = [tuple(t.clone() for t in bufs) for bufs in ref]
    ws = torch.zeros(max(plan.workspace_bytes(b.index, prec) for b in plan.batches), dtype=torch.uint8,
                     device="cuda")
    for b in plan.batches:
        Pb, G, M, O = ref[b.index]
        B.muon_step(plan, b.index, Pb, G, M, hp, ws, ns_out=O)

    idx = [b.index for b in plan.batches]
    lane_of, need = B.plan_lanes(plan, idx, hp, streams)
    assert sorted(set(lane_of)) == list(range(streams))
    wss = [torch.zeros(n, dtype=torch.uint8, device="cuda") for n in need]
    side = [torch.cuda.Stream() for _ in range(streams - 1)]
    B.muon_step_batches(plan, idx, mine, hp, wss, [None] + [s.cuda_stream for s in side])
    torch.cuda.synchronize()
    for b in plan.batches:
        for k, name in enumerate(["param", "grad", "momentum", "O"]):
            assert torch.equal(mine[b.index][k], ref[b.index][k]), (streams, prec, b.index, name)
        Wp, Mp, O = (H.to_host(mine[b.index][k]) for k in (0, 2, 3))
        arr = host[b.index]
        for q in range(b.count):
            P.check_matrix(arr["param"][q], arr["grad"][q], arr["momentum"][q], Wp[q], Mp[q], O[q], hp,
                           f"streams {streams} {prec} batch {b.index} ({b.M}x{b.N}) matrix {q}")


def test_step_batches_orders_after_and_before_caller_stream():
    """Work enqueued on the caller's stream before the call is seen by every
    lane, and work enqueued after it sees every lane's results."""
    import torch
    plan = B.Plan(SHAPES, max_batch_elems=CAP)
    hp = B.HParams()
    base = _filled(plan, torch.bfloat16, 4)
    ref = [tuple(t.clone() for t in bufs) for bufs in base]
    mine = [tuple(torch.empty_like(t) for t in bufs) for bufs in base]
    ws = torch.zeros(max(plan.workspace_bytes(b.index, "bf16") for b in plan.batches), dtype=torch.uint8,
                     device="cuda")
    for b in plan.batches:
        P, G, M, O = ref[b.index]
        B.muon_step(plan, b.index, P, G, M, hp, ws, ns_out=O)
    idx = [b.index for b in plan.batches]
    lane_of, need = B.plan_lanes(plan, idx, hp, 2)
    wss = [torch.zeros(n, dtype=torch.uint8, device="cuda") for n in need]
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    # inputs written on the caller's stream right before the call, after a
    # long unrelated product, so a lane that did not wait would read garbage
    junk = torch.randn(4096, 4096, device="cuda")
    for _ in range(4):
        junk = junk @ junk.mul_(1e-2)
    for i, bufs in enumerate(base):
        for k in range(4):
            mine[i][k].copy_(bufs[k])
    B.muon_step_batches(plan, idx, mine, hp, wss, [None, side.cuda_stream])
    # read back on the caller's stream without synchronising first
    copies = [tuple(t.clone() for t in bufs) for bufs in mine]
    cur.synchronize()
    for b in plan.batches:
        for k in range(4):
            assert torch.equal(copies[b.index][k], ref[b.index][k]), (b.index, k)


@pytest.mark.parametrize("streams", [1, 2])
def test_prepared_step_matches_calls(streams):
    """PreparedStep (arguments marshalled once) runs the same launches as the
    plain calls: two steps each, bitwise equal results."""
    import torch
    plan = B.Plan(SHAPES, max_batch_elems=CAP)
    hp = B.HParams()
    ref = _filled(plan, torch.bfloat16, 8)
    mine = [tuple(t.clone() for t in bufs) for bufs in ref]
    idx = [b.index for b in plan.batches]
    lane_of, need = B.plan_lanes(plan, idx, hp, streams)
    side = [torch.cuda.Stream() for _ in range(streams - 1)]
    sts = [None] + [s.cuda_stream for s in side]
    ws_ref = [torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None for n in need]
    ws_mine = [torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None for n in need]
    if streams == 1:
        calls = [B.PreparedStep(plan, b, mine[b], hp, ws_mine[0]) for b in idx]
    else:
        calls = [B.PreparedStep(plan, idx, mine, hp, ws_mine, sts)]
    for _ in range(2):
        if streams == 1:
            for b in idx:
                P, G, M, O = ref[b]
                B.muon_step(plan, b, P, G, M, hp, ws_ref[0], ns_out=O)
        else:
            B.muon_step_batches(plan, idx, ref, hp, ws_ref, sts)
        for c in calls:
            c()
    torch.cuda.synchronize()
    for b in idx:
        for k in range(4):
            assert torch.equal(mine[b][k], ref[b][k]), (streams, b, k)


def test_moe_workload_two_streams_bitwise():
    """The MoE expert workload at full size (the 32 + 32 [2048, 7168] expert
    batches and the [32, 24, 10240] experts) on two streams, as the benchmark
    runs it: bitwise the parameters and momentum of muon_step on each batch
    in turn (whose results the full-size parity tests check against the
    oracle)."""
    import torch
    from matrix_optimizer_amd import workloads as WL
    from tests import harness as H
    wl = WL.WORKLOADS["moe_experts"]
    plan = B.Plan([p.shape for p in wl.params])
    assert [(b.count, b.M, b.N) for b in plan.batches] == [(32, 2048, 7168), (32, 2048, 7168), (32, 24, 10240)]
    hp = H.c_hparams(wl.hp)
    gen = torch.Generator(device="cuda").manual_seed(29)
    ref = []
    for b in plan.batches:
        shp = (b.count, b.M, b.N)
        ref.append((torch.randn(shp, device="cuda", generator=gen).mul_(0.02).to(torch.bfloat16),
                    torch.randn(shp, device="cuda", generator=gen).mul_(1e-3).to(torch.bfloat16),
                    torch.randn(shp, device="cuda", generator=gen).mul_(1e-3)))
    mine = [tuple(t.clone() for t in x) for x in ref]
    ws = torch.empty(max(plan.workspace_bytes(b.index, hp.precision) for b in plan.batches), dtype=torch.uint8,
                     device="cuda")
    for b in plan.batches:
        P, G, M = ref[b.index]
        B.muon_step(plan, b.index, P, G, M, hp, ws)
    idx = [b.index for b in plan.batches]
    lane_of, need = B.plan_lanes(plan, idx, hp, 2)
    assert lane_of == [0, 1, 0]   # equal expert batches; the skinny one goes to the first of two equal lanes
    wss = [torch.empty(n, dtype=torch.uint8, device="cuda") for n in need]
    side = torch.cuda.Stream()
    B.muon_step_batches(plan, idx, mine, hp, wss, [None, side.cuda_stream])
    torch.cuda.synchronize()
    for b in plan.batches:
        assert torch.equal(mine[b.index][0], ref[b.index][0]), (b.index, "param")
        assert torch.equal(mine[b.index][2], ref[b.index][2]), (b.index, "momentum")


def test_step_batches_failure_part_way_joins_lanes():
    """A launch that fails part-way through a two-stream step (forced from the
    host with muon_debug_fail_dispatch: lane 1's second batch is refused)
    returns MUON_ERR_HIP after joining every forked lane into the caller's
    stream: work enqueued there afterwards sees lane 1's first batch
    complete, and the same failure under graph capture still lets the
    capture end cleanly."""
    import torch
    plan = B.Plan(SHAPES, max_batch_elems=CAP)
    hp = B.HParams()
    idx = [b.index for b in plan.batches]
    lane_of, need = B.plan_lanes(plan, idx, hp, 2)
    lane1 = [i for i in range(len(idx)) if lane_of[i] == 1]
    lane0 = [i for i in range(len(idx)) if lane_of[i] == 0]
    assert len(lane1) >= 2
    wss = [torch.zeros(n, dtype=torch.uint8, device="cuda") for n in need]
    side = torch.cuda.Stream()
    ref = _filled(plan, torch.bfloat16, 31)
    mine = [tuple(t.clone() for t in bufs) for bufs in ref]
    ws = torch.zeros(max(need), dtype=torch.uint8, device="cuda")
    for b in plan.batches:   # the per-batch results
        Pb, G, M, O = ref[b.index]
        B.muon_step(plan, b.index, Pb, G, M, hp, ws, ns_out=O)
    torch.cuda.synchronize()
    try:
        # lane 0's batches dispatch first, then lane 1's: fail lane 1's second
        B.muon_debug_fail_dispatch(len(lane0) + 1)
        with pytest.raises(B.MuonError) as ei:
            B.muon_step_batches(plan, idx, mine, hp, wss, [None, side.cuda_stream])
        assert ei.value.status == B.MUON_ERR_HIP
        # read back on the caller's stream, without synchronising first: every
        # lane-0 batch and exactly one lane-1 batch (its first) are complete
        got = [tuple(t.clone() for t in mine[i]) for i in range(len(idx))]
        torch.cuda.current_stream().synchronize()
        done = [all(torch.equal(got[i][k], ref[i][k]) for k in (0, 2, 3)) for i in range(len(idx))]
        assert all(done[i] for i in lane0)
        assert sum(done[i] for i in lane1) == 1
        # the same failure while capturing: the capture must still end cleanly
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        B.muon_debug_fail_dispatch(len(lane0) + 1)
        with pytest.raises(B.MuonError):
            with torch.cuda.stream(cap):
                with torch.cuda.graph(graph, stream=cap):
                    B.muon_step_batches(plan, idx, mine, hp, wss, [None, side.cuda_stream])
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        del graph
    finally:
        B.muon_debug_fail_dispatch(-1)
    # the library and the streams still work: a full step matches the per-batch calls
    ref2 = _filled(plan, torch.bfloat16, 32)
    mine2 = [tuple(t.clone() for t in bufs) for bufs in ref2]
    for b in plan.batches:
        Pb, G, M, O = ref2[b.index]
        B.muon_step(plan, b.index, Pb, G, M, hp, ws, ns_out=O)
    B.muon_step_batches(plan, idx, mine2, hp, wss, [None, side.cuda_stream])
    torch.cuda.synchronize()
    for b in plan.batches:
        for k in range(4):
            assert torch.equal(mine2[b.index][k], ref2[b.index][k]), (b.index, k)
