"""C ABI on the CPU: the library loads, exports every symbol muon.h declares,
its planner agrees with the plain bucketing rules entry by entry, and every
argument error is caught before anything is launched.  No call here reaches a
kernel launch."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from matrix_optimizer_amd import binding as B
from matrix_optimizer_amd import workloads as WL
from oracle import plan_oracle as PO

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "muon.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = _header_functions()
    assert "muon_step" in names and "muon_plan_create" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.EXPORTED)
    assert B.muon_abi_version() == 8


def _cmp_plans(shapes, cap=0, order=0):
    got = B.Plan(shapes, cap, order).batches
    ref = PO.plan(shapes, cap if cap else PO.DEFAULT_CAP, order)
    assert len(got) == len(ref)
    for g, r in zip(got, ref):
        assert (g.M, g.N, g.count, g.transposed) == (r.M, r.N, r.count, r.transposed)
        assert g.segments == [(s.param_index, s.first_matrix, s.num_matrices, s.elem_offset) for s in r.segments]


@pytest.mark.parametrize("name", sorted(WL.WORKLOADS))
def test_plan_matches_rules_on_workloads(name):
    _cmp_plans([p.shape for p in WL.WORKLOADS[name].params])


@pytest.mark.parametrize("seed", range(20))
def test_plan_matches_rules_random(seed):
    rng = np.random.default_rng(seed)
    dims = [1, 2, 3, 5, 8]
    shapes = []
    for _ in range(rng.integers(1, 25)):
        k = rng.integers(0, 3)
        if k == 0:
            shapes.append((int(rng.choice(dims)), int(rng.choice(dims))))
        elif k == 1:
            shapes.append((int(rng.choice(dims)), 1, int(rng.choice(dims))))
        else:
            shapes.append((int(rng.integers(1, 6)), int(rng.choice(dims)), int(rng.choice(dims))))
    cap = int(rng.choice([0, 1, 7, 30, 100]))
    _cmp_plans(shapes, cap, int(rng.integers(0, 2)))


def _plan_status(shapes, cap=0, order=0, skinny_kernel=0):
    arr = (B.muon_shape * max(1, len(shapes)))()
    for i, s in enumerate(shapes):
        arr[i].ndim = len(s)
        for d in range(min(3, len(s))):
            arr[i].dims[d] = s[d]
    opt = B.muon_plan_options(cap, order, skinny_kernel)
    h = C.c_void_p()
    st = B.lib().muon_plan_create(arr, len(shapes), C.byref(opt), C.byref(h))
    if st == 0:
        B.lib().muon_plan_destroy(h)
    return st


def test_plan_errors():
    assert _plan_status([(5,)]) == B.MUON_ERR_UNSUPPORTED
    assert _plan_status([(2, 3, 4, 5)]) == B.MUON_ERR_UNSUPPORTED
    assert _plan_status([(0, 4)]) == B.MUON_ERR_INVALID_ARG
    assert _plan_status([(3, -1, 2)]) == B.MUON_ERR_INVALID_ARG
    assert _plan_status([]) == B.MUON_ERR_INVALID_ARG
    assert _plan_status([(2, 2)], cap=-1) == B.MUON_ERR_INVALID_ARG
    assert _plan_status([(2, 2)], order=2) == B.MUON_ERR_INVALID_ARG
    assert _plan_status([(2, 2)], skinny_kernel=4) == B.MUON_ERR_INVALID_ARG
    assert _plan_status([(2, 2)], skinny_kernel=3) == B.MUON_OK
    assert _plan_status([(2, 2)], skinny_kernel=-1) == B.MUON_ERR_INVALID_ARG
    assert _plan_status([(1 << 20, 1 << 20)]) == B.MUON_ERR_UNSUPPORTED   # above 2^31 elements
    # the limit is on the matrix padded to 256 x 256 tiles: exactly 2^31 padded elements pass, in
    # either orientation and as an expert tensor, one more column (padded to 256 more) does not
    assert _plan_status([(32768, 65536)]) == B.MUON_OK
    assert _plan_status([(65536, 32768)]) == B.MUON_OK
    assert _plan_status([(3, 32768, 65536)]) == B.MUON_OK
    assert _plan_status([(32768, 65537)]) == B.MUON_ERR_UNSUPPORTED
    assert _plan_status([(32513, 65536)]) == B.MUON_OK             # rows pad up to 32768
    assert _plan_status([(32769, 65536)]) == B.MUON_ERR_UNSUPPORTED
    assert _plan_status([(1 << 40, 1 << 40)]) == B.MUON_ERR_INVALID_ARG   # int64 overflow
    assert _plan_status([(1 << 62, 4, 1 << 30)]) == B.MUON_ERR_INVALID_ARG


def test_batch_paths():
    # short side <= 32: Gram-space skinny kernels by default; option 2 forces step by step
    p = B.Plan([(24, 10240)] * 74 + [(300, 200)])
    paths = {(b.M, b.N): b.path for b in p.batches}
    assert paths[(300, 200)] == 0 and paths[(24, 10240)] == 1
    assert sorted(b.path for b in B.Plan([(24, 10240)] * 4 + [(64, 64)], skinny_kernel=1).batches) == [0, 1]
    assert [b.path for b in B.Plan([(24, 10240)], skinny_kernel=2).batches] == [2]
    assert [b.path for b in B.Plan([(10240, 32)], skinny_kernel=2).batches] == [2]
    assert [b.path for b in B.Plan([(33, 10240)], skinny_kernel=2).batches] == [0]
    assert [b.path for b in B.Plan([(8, 1 << 24)]).batches] == [1]
    for k in (1, 2):
        q = B.Plan([(24, 1000)] * 3, skinny_kernel=k)
        for prec in ("bf16", "bf16_x32", "f32"):
            assert q.workspace_bytes(0, prec) % 256 == 0
    # the step-by-step form keeps a second set of Gram partials
    g, s = B.Plan([(24, 1000)] * 3, skinny_kernel=1), B.Plan([(24, 1000)] * 3, skinny_kernel=2)
    assert s.workspace_bytes(0, "bf16") > g.workspace_bytes(0, "bf16")


def test_workspace_bytes():
    p = B.Plan([(24, 10240)] * 3 + [(300, 200)] * 2)
    for b in p.batches:
        for prec in ("bf16", "bf16_x32", "f32"):
            w = p.workspace_bytes(b.index, prec)
            assert w > 0 and w % 256 == 0
    tiled = [b for b in p.batches if b.M == 300][0]   # short side 200: bf16 placements apply
    assert p.workspace_bytes(tiled.index, "bf16_x32") > p.workspace_bytes(tiled.index, "bf16")
    # the master is two bf16 residue buffers of X (2 x 256 x 384 padded) on
    # the tiled path; the compensated mode needs nothing more, and the
    # skinny path runs it as the master mode, short sides 33..127 as fp32
    xe = 2 * 256 * 384
    assert p.workspace_bytes(tiled.index, "bf16_x32") == p.workspace_bytes(tiled.index, "bf16") + 2 * xe * 2
    assert p.workspace_bytes(tiled.index, "bf16_x32c") == p.workspace_bytes(tiled.index, "bf16_x32")
    sk = [b for b in p.batches if b.M == 24][0]
    assert p.workspace_bytes(sk.index, "bf16_x32c") == p.workspace_bytes(sk.index, "bf16_x32")
    mid = B.Plan([(100, 700)] * 2)
    assert mid.workspace_bytes(0, "bf16_x32c") == mid.workspace_bytes(0, "f32")
    with pytest.raises(B.MuonError):
        p.workspace_bytes(99, "bf16")
    out = C.c_size_t(0)
    assert B.lib().muon_workspace_bytes(p.handle, 0, 4, C.byref(out)) == B.MUON_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# argument validation of muon_step and the stage calls (returns before launch)
# ---------------------------------------------------------------------------
class FakeBuffers:
    """Host buffers standing in for device pointers: validation must reject
    every call below before a launch, and leave the bytes untouched."""

    def __init__(self, plan, batch=0, prec="bf16"):
        b = plan.batches[batch]
        n = b.count * b.M * b.N
        self.raw = {k: np.full(nb + 256, 0x5A, np.uint8) for k, nb in
                    [("param", n * 2), ("grad", n * 2), ("mom", n * 4), ("out", n * 4),
                     ("ws", plan.workspace_bytes(batch, prec))]}

    def ptr(self, k, off=0):
        a = self.raw[k].ctypes.data
        return ((a + 255) & ~255) + off

    def untouched(self):
        return all(np.all(v == 0x5A) for v in self.raw.values())


def _step(plan, fb, hp=None, ws_bytes=None, param=None, grad=None, mom=None, out=None, ws=None, batch=0,
          pdt=B.MUON_BF16, gdt=B.MUON_BF16):
    hp = hp or B.HParams()
    hpc, keep = hp.to_c()
    bufs = B.muon_batch_buffers(param if param is not None else fp(fb, "param"), pdt,
                                grad if grad is not None else fp(fb, "grad"), gdt,
                                mom if mom is not None else fp(fb, "mom"), out)
    wsb = ws_bytes if ws_bytes is not None else plan.workspace_bytes(0, hp.precision)
    return B.lib().muon_step(plan.handle, batch, C.byref(bufs), C.byref(hpc),
                             ws if ws is not None else fb.ptr("ws"), wsb, None)


def fp(fb, k):
    return fb.ptr(k)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.fixture(params=[[(24, 1000)] * 2, [(100, 40)]], ids=["skinny", "tiled"])
def plan_fb(request):
    # Host buffers stand in for device pointers here: on a machine with a GPU a
    # validation regression would launch kernels on them, so run on CPU only.
    if _gpu_visible():
        pytest.skip("fake-pointer validation tests run only where no GPU is visible")
    p = B.Plan(request.param)
    return p, FakeBuffers(p)


def test_step_rejects_bad_hparams(plan_fb):
    p, fb = plan_fb
    bad = [B.HParams(ns_steps=0), B.HParams(ns_steps=65), B.HParams(lr=float("nan")),
           B.HParams(momentum=1.5), B.HParams(momentum=-0.1), B.HParams(weight_decay=float("inf")),
           B.HParams(weight_decay=-1.0), B.HParams(eps=-1e-7), B.HParams(lr=-0.1),
           B.HParams(coeffs=(1.0, 2.0)), B.HParams(coeffs=(1.0, float("nan"), 2.0)),
           B.HParams(ns_steps=5, coeffs=(1.0, 2.0, 3.0) * 2)]
    for h in bad:
        assert _step(p, fb, hp=h) == B.MUON_ERR_INVALID_ARG, h
    hpc, keep = B.HParams().to_c()
    hpc.precision = 4
    bufs = B.muon_batch_buffers(fb.ptr("param"), 1, fb.ptr("grad"), 1, fb.ptr("mom"), None)
    assert B.lib().muon_step(p.handle, 0, C.byref(bufs), C.byref(hpc), fb.ptr("ws"), 1 << 40, None) == 1
    hpc.precision = 0
    hpc.scale = 9
    assert B.lib().muon_step(p.handle, 0, C.byref(bufs), C.byref(hpc), fb.ptr("ws"), 1 << 40, None) == 1
    hpc.scale = 1
    hpc.coeffs = C.cast(None, C.POINTER(C.c_float))
    assert B.lib().muon_step(p.handle, 0, C.byref(bufs), C.byref(hpc), fb.ptr("ws"), 1 << 40, None) == 1
    # the device {lr, wd} pointer must be 4-byte aligned
    hpc, keep = B.HParams().to_c()
    hpc.lr_wd_device = fb.ptr("ws", 2)
    assert B.lib().muon_step(p.handle, 0, C.byref(bufs), C.byref(hpc), fb.ptr("ws"), 1 << 40, None) == 1
    assert fb.untouched()


def test_step_rejects_bad_buffers(plan_fb):
    p, fb = plan_fb
    need = p.workspace_bytes(0, "bf16")
    assert _step(p, fb, ws_bytes=need - 1) == B.MUON_ERR_WORKSPACE_TOO_SMALL
    assert _step(p, fb, param=0) == B.MUON_ERR_INVALID_ARG                    # null
    assert _step(p, fb, mom=0) == B.MUON_ERR_INVALID_ARG
    assert _step(p, fb, ws=0) == B.MUON_ERR_INVALID_ARG
    assert _step(p, fb, grad=fb.ptr("grad", 2)) == B.MUON_ERR_INVALID_ARG     # misaligned
    assert _step(p, fb, ws=fb.ptr("ws", 16)) == B.MUON_ERR_INVALID_ARG        # workspace not 256-aligned
    assert _step(p, fb, grad=fb.ptr("param", 256)) == B.MUON_ERR_INVALID_ARG  # overlaps param
    assert _step(p, fb, out=fb.ptr("mom")) == B.MUON_ERR_INVALID_ARG          # ns_out aliases momentum
    assert _step(p, fb, batch=5) == B.MUON_ERR_INVALID_ARG
    assert _step(p, fb, batch=-1) == B.MUON_ERR_INVALID_ARG
    assert _step(p, fb, pdt=3) == B.MUON_ERR_INVALID_ARG
    hpc, keep = B.HParams().to_c()
    assert B.lib().muon_step(p.handle, 0, None, C.byref(hpc), fb.ptr("ws"), need, None) == 1
    assert B.lib().muon_step(None, 0, None, C.byref(hpc), fb.ptr("ws"), need, None) == 1
    assert fb.untouched()


def test_step_ptrs_rejects_bad_args(plan_fb):
    """muon_step_ptrs: the pointer tables are checked like buffers (non-null,
    16-byte aligned, not overlapping each other or the workspace); what they
    hold is device data the host never reads."""
    p, fb = plan_fb
    L = B.lib()
    need = p.workspace_bytes(0, "bf16")
    hpc, keep = B.HParams().to_c()

    def call(params=None, grads=None, moms=None, outs=None, ws=None, wsb=need, pdt=B.MUON_BF16, batch=0):
        bufs = B.muon_batch_ptrs(params if params is not None else fb.ptr("param"), pdt,
                                 grads if grads is not None else fb.ptr("grad"), B.MUON_BF16,
                                 moms if moms is not None else fb.ptr("mom"), outs)
        return L.muon_step_ptrs(p.handle, batch, C.byref(bufs), C.byref(hpc),
                                ws if ws is not None else fb.ptr("ws"), wsb, None)

    assert call(wsb=need - 1) == B.MUON_ERR_WORKSPACE_TOO_SMALL
    assert call(params=0) == B.MUON_ERR_INVALID_ARG
    assert call(grads=0) == B.MUON_ERR_INVALID_ARG
    assert call(moms=0) == B.MUON_ERR_INVALID_ARG
    assert call(grads=fb.ptr("grad", 8)) == B.MUON_ERR_INVALID_ARG      # table not 16-byte aligned
    assert call(grads=fb.ptr("param")) == B.MUON_ERR_INVALID_ARG        # same table twice
    assert call(outs=fb.ptr("ws")) == B.MUON_ERR_INVALID_ARG            # table inside the workspace
    assert call(pdt=5) == B.MUON_ERR_INVALID_ARG
    assert call(batch=9) == B.MUON_ERR_INVALID_ARG
    assert L.muon_step_ptrs(p.handle, 0, None, C.byref(hpc), fb.ptr("ws"), need, None) == 1
    bad, _ = B.HParams(ns_steps=0).to_c()
    bufs = B.muon_batch_ptrs(fb.ptr("param"), 1, fb.ptr("grad"), 1, fb.ptr("mom"), None)
    assert L.muon_step_ptrs(p.handle, 0, C.byref(bufs), C.byref(bad), fb.ptr("ws"), need, None) == 1
    assert fb.untouched()


def test_stage_calls_reject_bad_args(plan_fb):
    p, fb = plan_fb
    L = B.lib()
    hpc, keep = B.HParams().to_c()
    bad, _ = B.HParams(momentum=2.0).to_c()
    assert L.muon_stage_momentum(p.handle, 0, fb.ptr("grad"), 1, fb.ptr("mom"), fb.ptr("mom"),
                                 C.byref(hpc), None) == 1
    assert L.muon_stage_momentum(p.handle, 0, fb.ptr("grad"), 1, fb.ptr("mom"), fb.ptr("out"),
                                 C.byref(bad), None) == 1
    assert L.muon_stage_ns(p.handle, 0, fb.ptr("mom"), fb.ptr("out"), C.byref(hpc), fb.ptr("ws"), 0, None) == 3
    assert L.muon_stage_ns(p.handle, 0, fb.ptr("mom"), fb.ptr("mom"), C.byref(hpc), fb.ptr("ws"), 1 << 40,
                           None) == 1
    bad_lr, _ = B.HParams(lr=float("inf")).to_c()
    assert L.muon_stage_update(p.handle, 0, fb.ptr("param"), 1, fb.ptr("out"), C.byref(bad_lr), None) == 1
    assert L.muon_stage_update(p.handle, 0, fb.ptr("param"), 1, 0, C.byref(hpc), None) == 1
    assert fb.untouched()


def test_status_strings():
    for s in range(7):
        assert B.status_str(s)
    assert B.status_str(42) == "unknown status"


def test_plan_lanes():
    """muon_plan_lanes: the longest batch first, each onto the least-loaded
    lane; a lane's workspace is the largest of its batches'."""
    p = B.Plan([(2048, 7168)] * 36 + [(2048, 4096)] * 20 + [(24, 10240)] * 32)
    idx = [b.index for b in p.batches]
    assert [(b.count, b.M, b.N) for b in p.batches] == [(36, 2048, 7168), (20, 2048, 4096), (32, 24, 10240)]
    hp = B.HParams()
    ws = [p.workspace_bytes(i, "bf16") for i in idx]
    lanes, need = B.plan_lanes(p, idx, hp, 1)
    assert lanes == [0, 0, 0] and need == [max(ws)]
    lanes, need = B.plan_lanes(p, idx, hp, 2)
    assert lanes == [0, 1, 1] and need == [ws[0], max(ws[1], ws[2])]
    lanes, need = B.plan_lanes(p, idx, hp, 4)
    assert lanes == [0, 1, 2] and need == ws + [0]   # three batches: one lane each, lane 3 empty
    # the order given does not change which batch goes where
    lanes_r, _ = B.plan_lanes(p, idx[::-1], hp, 2)
    assert lanes_r == [1, 1, 0]
    # equal batches alternate lanes in the order given
    q = B.Plan([(256, 512)] * 4, max_batch_elems=256 * 512)
    lanes, need = B.plan_lanes(q, [0, 1, 2, 3], hp, 2)
    assert lanes == [0, 1, 0, 1] and need[0] == need[1] == q.workspace_bytes(0, "bf16")
    L = B.lib()
    hpc, keep = hp.to_c()
    lo = (C.c_int32 * 3)()
    wb = (C.c_size_t * 9)()
    for batches, ns in [([0, 0], 2), ([0, 5], 2), ([0], 0), ([0], 9), ([-1], 1)]:
        arr = (C.c_int32 * len(batches))(*batches)
        assert L.muon_plan_lanes(p.handle, len(batches), arr, C.byref(hpc), ns, lo, wb) == B.MUON_ERR_INVALID_ARG
    arr = (C.c_int32 * 1)(0)
    assert L.muon_plan_lanes(p.handle, 0, arr, C.byref(hpc), 1, lo, wb) == B.MUON_ERR_INVALID_ARG
    assert L.muon_plan_lanes(p.handle, 1, arr, C.byref(hpc), 1, None, wb) == B.MUON_ERR_INVALID_ARG
    bad, _ = B.HParams(ns_steps=0).to_c()
    assert L.muon_plan_lanes(p.handle, 1, arr, C.byref(bad), 1, lo, wb) == B.MUON_ERR_INVALID_ARG


def test_step_batches_rejects_bad_args():
    """muon_step_batches checks every batch's buffers and every used lane's
    workspace, and that all of them are disjoint (lanes run concurrently),
    before anything is enqueued."""
    if _gpu_visible():
        pytest.skip("fake-pointer validation tests run only where no GPU is visible")
    p = B.Plan([(24, 1000)] * 2 + [(100, 40)])
    assert len(p.batches) == 2
    fbs = [FakeBuffers(p, 0), FakeBuffers(p, 1)]
    hp = B.HParams()
    lanes, need = B.plan_lanes(p, [0, 1], hp, 2)
    assert sorted(lanes) == [0, 1]
    ws_of = {lanes[i]: fbs[i].ptr("ws") for i in range(2)}
    L = B.lib()
    hpc, keep = hp.to_c()

    def call(batches=(0, 1), bufs=None, wsp=None, wsb=None, streams=(None, None), hpp=None, n=None):
        bl = list(batches)
        fb = (B.muon_batch_buffers * 2)()
        for i in range(2):
            f = fbs[i]
            fb[i] = B.muon_batch_buffers(f.ptr("param"), 1, f.ptr("grad"), 1, f.ptr("mom"), None)
        if bufs:
            for i, v in bufs.items():
                fb[i] = v
        w = wsp if wsp is not None else [ws_of[0], ws_of[1]]
        wb = wsb if wsb is not None else list(need)
        arr = (C.c_int32 * len(bl))(*bl)
        return L.muon_step_batches(p.handle, len(bl) if n is None else n, arr, fb, C.byref(hpp or hpc),
                                   (C.c_void_p * 2)(*w), (C.c_size_t * 2)(*wb), (C.c_void_p * 2)(*streams),
                                   2)

    assert call(wsb=[need[0] - 1, need[1]]) == B.MUON_ERR_WORKSPACE_TOO_SMALL
    assert call(wsb=[need[0], need[1] - 1]) == B.MUON_ERR_WORKSPACE_TOO_SMALL
    assert call(wsp=[0, ws_of[1]]) == B.MUON_ERR_INVALID_ARG                     # used lane without workspace
    assert call(wsp=[ws_of[0], ws_of[0]]) == B.MUON_ERR_INVALID_ARG              # lanes share a workspace
    assert call(wsp=[ws_of[0] + 16, ws_of[1]]) == B.MUON_ERR_INVALID_ARG         # not 256-byte aligned
    f0, f1 = fbs
    # batch 1's momentum inside batch 0's: both lanes would write it
    assert call(bufs={1: B.muon_batch_buffers(f1.ptr("param"), 1, f1.ptr("grad"), 1, f0.ptr("mom"), None)}) == 1
    # an output inside the other lane's workspace
    assert call(bufs={0: B.muon_batch_buffers(f0.ptr("param"), 1, f0.ptr("grad"), 1, f0.ptr("mom"),
                                              ws_of[lanes[1]])}) == 1
    assert call(bufs={0: B.muon_batch_buffers(f0.ptr("param"), 7, f0.ptr("grad"), 1, f0.ptr("mom"), None)}) == 1
    assert call(batches=(0, 0)) == B.MUON_ERR_INVALID_ARG
    assert call(batches=(0, 2)) == B.MUON_ERR_INVALID_ARG
    assert call(n=0) == B.MUON_ERR_INVALID_ARG
    bad, _ = B.HParams(lr=float("nan")).to_c()
    assert call(hpp=bad) == B.MUON_ERR_INVALID_ARG
    arr = (C.c_int32 * 2)(0, 1)
    fb = (B.muon_batch_buffers * 2)()
    assert L.muon_step_batches(p.handle, 2, arr, fb, C.byref(hpc), None, None, None, 2) == B.MUON_ERR_INVALID_ARG
    assert L.muon_step_batches(p.handle, 2, arr, fb, C.byref(hpc), (C.c_void_p * 9)(), (C.c_size_t * 9)(),
                               (C.c_void_p * 9)(), 9) == B.MUON_ERR_INVALID_ARG
    assert all(f.untouched() for f in fbs)


def test_step_rows_rejects_bad_args(plan_fb):
    """muon_step_rows: the row tables, momentum and workspace are checked like
    buffers (non-null, 16-byte aligned, disjoint); the rows they point at are
    device data the host never reads."""
    p, fb = plan_fb
    L = B.lib()
    need = p.workspace_bytes(0, "bf16")
    hpc, keep = B.HParams().to_c()

    def call(prow=None, grow=None, mom=None, out=None, ws=None, wsb=need, pdt=B.MUON_BF16, batch=0):
        bufs = B.muon_batch_rows(prow if prow is not None else fb.ptr("param"), pdt,
                                 grow if grow is not None else fb.ptr("grad"), B.MUON_BF16,
                                 mom if mom is not None else fb.ptr("mom"), out)
        return L.muon_step_rows(p.handle, batch, C.byref(bufs), C.byref(hpc),
                                ws if ws is not None else fb.ptr("ws"), wsb, None)

    assert call(wsb=need - 1) == B.MUON_ERR_WORKSPACE_TOO_SMALL
    assert call(prow=0) == B.MUON_ERR_INVALID_ARG
    assert call(grow=0) == B.MUON_ERR_INVALID_ARG
    assert call(mom=0) == B.MUON_ERR_INVALID_ARG
    assert call(grow=fb.ptr("grad", 8)) == B.MUON_ERR_INVALID_ARG      # table not 16-byte aligned
    assert call(grow=fb.ptr("param")) == B.MUON_ERR_INVALID_ARG        # same table twice
    assert call(mom=fb.ptr("ws")) == B.MUON_ERR_INVALID_ARG            # momentum inside the workspace
    assert call(out=fb.ptr("mom")) == B.MUON_ERR_INVALID_ARG           # O over the momentum
    assert call(pdt=5) == B.MUON_ERR_INVALID_ARG
    assert call(batch=9) == B.MUON_ERR_INVALID_ARG
    assert L.muon_step_rows(p.handle, 0, None, C.byref(hpc), fb.ptr("ws"), need, None) == 1
    assert fb.untouched()


# ---------------------------------------------------------------------------
# muon_step_noalloc: refusals that happen before the device is touched
# ---------------------------------------------------------------------------
def test_step_noalloc_refuses_before_touching_anything():
    if _gpu_visible():
        pytest.skip("fake-pointer validation tests run only where no GPU is visible")
    big = B.Plan([(4096, 4096)])   # workspace far above the static array
    assert big.workspace_bytes(0, "bf16") > B.NOALLOC_SCRATCH_BYTES
    fb = FakeBuffers(B.Plan([(24, 100)]))
    hpc, keep = B.HParams().to_c()
    bufs = B.muon_batch_buffers(fb.ptr("param"), 1, fb.ptr("grad"), 1, fb.ptr("mom"), None)
    L = B.lib()
    assert L.muon_step_noalloc(big.handle, 0, C.byref(bufs), C.byref(hpc), None) == B.MUON_ERR_WORKSPACE_TOO_SMALL
    small = B.Plan([(24, 100)])
    assert L.muon_step_noalloc(small.handle, 1, C.byref(bufs), C.byref(hpc), None) == B.MUON_ERR_INVALID_ARG
    assert L.muon_step_noalloc(None, 0, C.byref(bufs), C.byref(hpc), None) == B.MUON_ERR_INVALID_ARG
    assert L.muon_step_noalloc(small.handle, 0, None, C.byref(hpc), None) == B.MUON_ERR_INVALID_ARG
    assert L.muon_step_noalloc(small.handle, 0, C.byref(bufs), None, None) == B.MUON_ERR_INVALID_ARG
    hpc.precision = 9
    assert L.muon_step_noalloc(small.handle, 0, C.byref(bufs), C.byref(hpc), None) == B.MUON_ERR_INVALID_ARG
    assert fb.untouched()


# ---------------------------------------------------------------------------
# host-built address tables refuse addresses the kernels cannot take
# ---------------------------------------------------------------------------
def test_row_and_pointer_tables_refuse_misaligned_addresses():
    import torch
    base = torch.zeros(64, 64, dtype=torch.bfloat16)
    assert base.data_ptr() % 16 == 0
    # a column range starting at column 3 of bf16 rows: rows start 6 bytes in
    with pytest.raises(ValueError, match="16-byte"):
        B.row_addresses(base[:, 3:27])
    # starting at column 8 (16 bytes) with a 128-byte row stride is fine
    addr = B.row_addresses(base[:, 8:32])
    assert bool((addr % 16 == 0).all()) and addr.numel() == 64
    # an odd row stride misaligns every other row
    odd = torch.zeros(64 * 33, dtype=torch.bfloat16)[: 64 * 33].view(64, 33)
    with pytest.raises(ValueError, match="16-byte"):
        B.row_addresses(odd[:, 0:24])
    flat = torch.zeros(4096, dtype=torch.float32)
    mats = [flat[i * 256:(i + 1) * 256].view(16, 16) for i in range(3)]
    assert B.pointer_table(mats, device="cpu").numel() == 3
    with pytest.raises(ValueError, match="16-byte"):
        B.pointer_table([flat[1:257].view(16, 16)], device="cpu")
