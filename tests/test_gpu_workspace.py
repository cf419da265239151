"""The workspace holds no state between calls: whatever its bytes are before
a step, the step's results are the same.

Each case runs one step three times from the same inputs: on a workspace
filled with 0xFF bytes (NaN in fp32 and bf16, and the largest value in the
products' tile counters), again on the workspace the first call left behind,
and on a zeroed workspace.  W', M' and O must be finite and bitwise equal
across the three.  A kernel that read a workspace byte (a tile of an
intermediate product, a counter, a partial sum) before this step wrote it
would fail: a skipped tile leaves NaN or the previous call's values.

The batch of 10 [2048, 2048] matrices gives 360 Gram and poly tiles and
640 apply tiles, more than one tile per workgroup, so the 256 x 256
products' dynamic tile order runs several rounds and takes tiles from other
XCDs' ranges; the other cases cover 256 x 256 tiles in both orientations
and in every bf16 precision, 128 x 128 tiles and the skinny path in both
Newton-Schulz forms.
"""
import pytest

from matrix_optimizer_amd import binding as B

pytestmark = pytest.mark.gpu

CASES = [
    ("tiled_256_rounds", [(10, 2048, 2048)], 0, "bf16"),
    ("tiled_256_wide_x32", [(512, 1280)] * 3, 0, "bf16_x32"),
    ("tiled_256_tall_x32c", [(1280, 512)] * 3, 0, "bf16_x32c"),
    ("tiled_128_x32c", [(300, 700)] * 2, 0, "bf16_x32c"),
    ("tiled_256_tall", [(1280, 512)] * 3, 0, "bf16"),
    ("tiled_128", [(300, 700)] * 2, 0, "bf16"),
    ("skinny_fused", [(24, 3000)] * 5, 0, "bf16"),
    ("skinny_stepwise", [(24, 3000)] * 5, 2, "bf16"),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


@pytest.mark.parametrize("name,shapes,kernel,prec", CASES, ids=[c[0] for c in CASES])
def test_results_do_not_depend_on_workspace_contents(name, shapes, kernel, prec):
    import torch
    plan = B.Plan(shapes, skinny_kernel=kernel)
    hp = B.HParams(precision=prec)
    gen = torch.Generator(device="cuda").manual_seed(600 + [c[0] for c in CASES].index(name))
    for b in plan.batches:
        shp = (b.count, b.M, b.N)
        W0 = torch.randn(shp, device="cuda", generator=gen).mul_(0.02).to(torch.bfloat16)
        G0 = torch.randn(shp, device="cuda", generator=gen).to(torch.bfloat16)
        M0 = torch.randn(shp, device="cuda", generator=gen).mul_(0.1)
        ws = torch.empty(plan.workspace_bytes(b.index, prec), dtype=torch.uint8, device="cuda")
        runs = []
        for fill in (0xFF, None, 0x00):   # None: what the previous call left
            if fill is not None:
                ws.fill_(fill)
            W, M = W0.clone(), M0.clone()
            O = torch.empty(shp, dtype=torch.float32, device="cuda")
            B.muon_step(plan, b.index, W, G0, M, hp, ws, ns_out=O)
            torch.cuda.synchronize()
            runs.append((W, M, O))
        for t in runs[0]:
            assert torch.isfinite(t.float()).all(), (name, b.index)
        for other in runs[1:]:
            for k, (x, y) in enumerate(zip(runs[0], other)):
                assert torch.equal(x, y), (name, b.index, ("W", "M", "O")[k])
