"""ctypes binding of libmuon's C ABI (include/muon.h).

Argument marshalling only: every step of the optimizer runs in the library's
HIP kernels.  PyTorch supplies device memory and the stream (``data_ptr()``
and ``torch.cuda.current_stream().cuda_stream``).  If the built library is
missing, loading fails with an error; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmuon.so")
_lib = None

# enums (muon.h)
MUON_OK, MUON_ERR_INVALID_ARG, MUON_ERR_UNSUPPORTED, MUON_ERR_WORKSPACE_TOO_SMALL, \
    MUON_ERR_NO_MEMORY, MUON_ERR_HIP, MUON_ERR_INTERNAL = range(7)
MUON_F32, MUON_BF16 = 0, 1
MUON_PREC_BF16, MUON_PREC_BF16_X32, MUON_PREC_F32, MUON_PREC_BF16_X32C = 0, 1, 2, 3
MUON_SCALE_NONE, MUON_SCALE_RMS = 0, 1

PRECISIONS = {"bf16": MUON_PREC_BF16, "bf16_x32": MUON_PREC_BF16_X32, "f32": MUON_PREC_F32,
              "bf16_x32c": MUON_PREC_BF16_X32C}
SCALES = {"none": MUON_SCALE_NONE, "rms": MUON_SCALE_RMS}

EXPORTED = ["muon_abi_version", "muon_status_str", "muon_plan_create", "muon_plan_destroy", "muon_step_ptrs",
            "muon_plan_num_batches", "muon_plan_batch_info", "muon_plan_segments",
            "muon_workspace_bytes", "muon_step", "muon_stage_momentum", "muon_stage_ns",
            "muon_stage_update", "muon_trace_start", "muon_trace_stop", "muon_plan_lanes",
            "muon_step_batches", "muon_step_rows", "muon_ns_schedule", "muon_step_noalloc",
            "muon_debug_fail_dispatch"]

# size of the static device workspace of muon_step_noalloc (MUON_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class muon_shape(C.Structure):
    _fields_ = [("ndim", C.c_int32), ("dims", C.c_int64 * 3)]


class muon_plan_options(C.Structure):
    _fields_ = [("max_batch_elems", C.c_int64), ("order", C.c_int32), ("skinny_kernel", C.c_int32)]


class muon_batch_info(C.Structure):
    _fields_ = [("M", C.c_int64), ("N", C.c_int64), ("count", C.c_int64),
                ("transposed", C.c_int32), ("num_segments", C.c_int32), ("path", C.c_int32),
                ("reserved", C.c_int32)]


class muon_segment(C.Structure):
    _fields_ = [("param_index", C.c_int32), ("reserved", C.c_int32), ("first_matrix", C.c_int64),
                ("num_matrices", C.c_int64), ("elem_offset", C.c_int64)]


class muon_hparams(C.Structure):
    _fields_ = [("lr", C.c_float), ("momentum", C.c_float), ("weight_decay", C.c_float),
                ("eps", C.c_float), ("nesterov", C.c_int32), ("ns_steps", C.c_int32),
                ("coeffs", C.POINTER(C.c_float)), ("num_coeff_sets", C.c_int32),
                ("scale", C.c_int32), ("precision", C.c_int32), ("lr_wd_device", C.c_void_p)]


class muon_batch_buffers(C.Structure):
    _fields_ = [("param", C.c_void_p), ("param_dtype", C.c_int32), ("grad", C.c_void_p),
                ("grad_dtype", C.c_int32), ("momentum", C.c_void_p), ("ns_out", C.c_void_p)]


class muon_batch_ptrs(C.Structure):
    _fields_ = [("params", C.c_void_p), ("param_dtype", C.c_int32), ("grads", C.c_void_p),
                ("grad_dtype", C.c_int32), ("momenta", C.c_void_p), ("ns_out", C.c_void_p)]


class muon_batch_rows(C.Structure):
    _fields_ = [("param_rows", C.c_void_p), ("param_dtype", C.c_int32), ("grad_rows", C.c_void_p),
                ("grad_dtype", C.c_int32), ("momentum", C.c_void_p), ("ns_out", C.c_void_p)]


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libmuon.so (built by matrix_optimizer_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libmuon is not built ({_LIB_PATH} missing); run "
                          "`python -m matrix_optimizer_amd.build` or __graft_entry__.build()")
    L = C.CDLL(_LIB_PATH)
    L.muon_abi_version.restype = C.c_int32
    L.muon_status_str.restype = C.c_char_p
    L.muon_status_str.argtypes = [C.c_int32]
    L.muon_plan_create.restype = C.c_int32
    L.muon_plan_create.argtypes = [C.POINTER(muon_shape), C.c_int32, C.POINTER(muon_plan_options),
                                   C.POINTER(C.c_void_p)]
    L.muon_plan_destroy.restype = None
    L.muon_plan_destroy.argtypes = [C.c_void_p]
    L.muon_plan_num_batches.restype = C.c_int32
    L.muon_plan_num_batches.argtypes = [C.c_void_p]
    L.muon_plan_batch_info.restype = C.c_int32
    L.muon_plan_batch_info.argtypes = [C.c_void_p, C.c_int32, C.POINTER(muon_batch_info)]
    L.muon_plan_segments.restype = C.c_int32
    L.muon_plan_segments.argtypes = [C.c_void_p, C.c_int32, C.POINTER(muon_segment), C.c_int32]
    L.muon_workspace_bytes.restype = C.c_int32
    L.muon_workspace_bytes.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(C.c_size_t)]
    L.muon_step.restype = C.c_int32
    L.muon_step.argtypes = [C.c_void_p, C.c_int32, C.POINTER(muon_batch_buffers), C.POINTER(muon_hparams),
                            C.c_void_p, C.c_size_t, C.c_void_p]
    L.muon_step_noalloc.restype = C.c_int32
    L.muon_step_noalloc.argtypes = [C.c_void_p, C.c_int32, C.POINTER(muon_batch_buffers), C.POINTER(muon_hparams),
                                    C.c_void_p]
    L.muon_step_ptrs.restype = C.c_int32
    L.muon_step_ptrs.argtypes = [C.c_void_p, C.c_int32, C.POINTER(muon_batch_ptrs), C.POINTER(muon_hparams),
                                 C.c_void_p, C.c_size_t, C.c_void_p]
    L.muon_step_rows.restype = C.c_int32
    L.muon_step_rows.argtypes = [C.c_void_p, C.c_int32, C.POINTER(muon_batch_rows), C.POINTER(muon_hparams),
                                 C.c_void_p, C.c_size_t, C.c_void_p]
    L.muon_plan_lanes.restype = C.c_int32
    L.muon_plan_lanes.argtypes = [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(muon_hparams), C.c_int32,
                                  C.POINTER(C.c_int32), C.POINTER(C.c_size_t)]
    L.muon_step_batches.restype = C.c_int32
    L.muon_step_batches.argtypes = [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(muon_batch_buffers),
                                    C.POINTER(muon_hparams), C.POINTER(C.c_void_p), C.POINTER(C.c_size_t),
                                    C.POINTER(C.c_void_p), C.c_int32]
    L.muon_stage_momentum.restype = C.c_int32
    L.muon_stage_momentum.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                      C.POINTER(muon_hparams), C.c_void_p]
    L.muon_stage_ns.restype = C.c_int32
    L.muon_stage_ns.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.POINTER(muon_hparams),
                                C.c_void_p, C.c_size_t, C.c_void_p]
    L.muon_stage_update.restype = C.c_int32
    L.muon_stage_update.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p,
                                    C.POINTER(muon_hparams), C.c_void_p]
    L.muon_ns_schedule.restype = C.c_int32
    L.muon_ns_schedule.argtypes = [C.c_int32, C.c_double, C.c_double, C.c_double, C.POINTER(C.c_float),
                                   C.POINTER(C.c_double)]
    L.muon_debug_fail_dispatch.restype = None
    L.muon_debug_fail_dispatch.argtypes = [C.c_int32]
    L.muon_trace_start.restype = C.c_int32
    L.muon_trace_start.argtypes = [C.c_int32]
    L.muon_trace_stop.restype = C.c_int32
    L.muon_trace_stop.argtypes = [C.POINTER(C.c_float), C.POINTER(C.c_char_p), C.c_int32]
    _lib = L
    return L


def status_str(s: int) -> str:
    try:
        return lib().muon_status_str(s).decode()
    except ImportError:
        return str(s)


def _check(status: int, where: str):
    if status != MUON_OK:
        raise MuonError(status, where)


def muon_abi_version() -> int:
    return lib().muon_abi_version()


def ns_schedule(steps: int, lower: float = 1e-3, safety: float = 1.0, cushion: float = 0.0):
    """Per-step Newton-Schulz coefficients (muon_ns_schedule): returns (coeffs,
    bounds), coeffs a tuple of 3*steps floats for HParams(ns_steps=steps,
    coeffs=coeffs), bounds a list of (lo, hi) singular-value intervals after
    each step."""
    co = (C.c_float * (3 * steps))()
    bo = (C.c_double * (2 * steps))()
    _check(lib().muon_ns_schedule(int(steps), float(lower), float(safety), float(cushion), co, bo),
           "muon_ns_schedule")
    return tuple(float(v) for v in co), [(bo[2 * k], bo[2 * k + 1]) for k in range(steps)]


@dataclass
class BatchInfo:
    index: int
    M: int
    N: int
    count: int
    transposed: bool
    segments: List[Tuple[int, int, int, int]]   # (param_index, first_matrix, num_matrices, elem_offset)
    path: int = 0                               # 0 tiled, 1 skinny Gram space, 2 skinny step by step

    @property
    def elems(self) -> int:
        return self.count * self.M * self.N


class Plan:
    """muon_plan_create / muon_plan_* on a list of parameter shapes."""

    def __init__(self, shapes: Sequence[Sequence[int]], max_batch_elems: int = 0, order: int = 0,
                 skinny_kernel: int = 0):
        L = lib()
        arr = (muon_shape * len(shapes))()
        for i, s in enumerate(shapes):
            arr[i].ndim = len(s)
            for d in range(min(len(s), 3)):
                arr[i].dims[d] = int(s[d])
        opt = muon_plan_options(int(max_batch_elems), int(order), int(skinny_kernel))
        h = C.c_void_p()
        _check(L.muon_plan_create(arr, len(shapes), C.byref(opt), C.byref(h)), "muon_plan_create")
        self._h = h
        self.shapes = [tuple(int(x) for x in s) for s in shapes]
        self.batches: List[BatchInfo] = []
        for b in range(L.muon_plan_num_batches(h)):
            info = muon_batch_info()
            _check(L.muon_plan_batch_info(h, b, C.byref(info)), "muon_plan_batch_info")
            segs = (muon_segment * max(1, info.num_segments))()
            _check(L.muon_plan_segments(h, b, segs, info.num_segments), "muon_plan_segments")
            self.batches.append(BatchInfo(b, info.M, info.N, info.count, bool(info.transposed),
                                          [(s.param_index, s.first_matrix, s.num_matrices, s.elem_offset)
                                           for s in segs[:info.num_segments]], info.path))

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.muon_plan_destroy(h)
            self._h = None

    def workspace_bytes(self, batch: int, precision: str = "bf16") -> int:
        out = C.c_size_t()
        _check(lib().muon_workspace_bytes(self._h, batch, PRECISIONS[precision], C.byref(out)),
               "muon_workspace_bytes")
        return out.value


@dataclass
class HParams:
    lr: float = 0.02
    momentum: float = 0.95
    weight_decay: float = 0.1
    eps: float = 1e-7
    nesterov: bool = True
    ns_steps: int = 5
    coeffs: Tuple[float, ...] = (3.4445, -4.7750, 2.0315)
    scale: str = "rms"
    precision: str = "bf16"
    lr_wd: object = None   # optional device float32 tensor [lr, weight_decay], read when the kernels run

    def to_c(self):
        """(struct, keep-alive coefficient array)."""
        arr = (C.c_float * len(self.coeffs))(*self.coeffs)
        hp = muon_hparams(self.lr, self.momentum, self.weight_decay, self.eps, int(bool(self.nesterov)),
                          int(self.ns_steps), C.cast(arr, C.POINTER(C.c_float)), len(self.coeffs) // 3,
                          SCALES[self.scale], PRECISIONS[self.precision],
                          None if self.lr_wd is None else self.lr_wd.data_ptr())
        return hp, arr


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    if t.dtype == torch.float32:
        return MUON_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream)


def muon_step(plan: Plan, batch: int, param, grad, momentum, hp: HParams, workspace,
              ns_out=None, stream=None) -> None:
    """One full step on one batch (muon_step).  Tensors are device tensors;
    param/grad bf16 or fp32, momentum fp32, workspace a uint8 tensor."""
    hpc, keep = hp.to_c()
    bufs = muon_batch_buffers(_ptr(param), _dtype_code(param), _ptr(grad), _dtype_code(grad),
                              _ptr(momentum), _ptr(ns_out))
    st = lib().muon_step(plan.handle, batch, C.byref(bufs), C.byref(hpc), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "muon_step")


def muon_step_noalloc(plan: Plan, batch: int, param, grad, momentum, hp: HParams, ns_out=None,
                      stream=None) -> None:
    """muon_step with the library's static device workspace (muon_step_noalloc):
    no workspace argument, nothing allocated.  Raises MuonError (workspace too
    small) for a batch needing more than NOALLOC_SCRATCH_BYTES.  Calls that
    overlap on one device share that workspace and race."""
    hpc, keep = hp.to_c()
    bufs = muon_batch_buffers(_ptr(param), _dtype_code(param), _ptr(grad), _dtype_code(grad),
                              _ptr(momentum), _ptr(ns_out))
    _check(lib().muon_step_noalloc(plan.handle, batch, C.byref(bufs), C.byref(hpc), _stream(stream)),
           "muon_step_noalloc")


class PreparedStep:
    """muon_step (one batch) or muon_step_batches (several, on several streams)
    with every argument marshalled once: each call is then one foreign call,
    for loops that repeat the same step on the same buffers.  Addresses,
    hyperparameters and streams are fixed at construction (the stream that is
    current then, if none is given); values behind hp.lr_wd may change
    between calls.  Keeps the tensors alive."""

    def __init__(self, plan: Plan, batches, bufs, hp: HParams, workspaces, streams=None):
        self._hpc, self._keep = hp.to_c()
        self._refs = (plan, bufs, workspaces, hp.lr_wd)
        L = lib()
        if isinstance(batches, int):   # one batch: muon_step
            param, grad, mom = bufs[0], bufs[1], bufs[2]
            out = bufs[3] if len(bufs) > 3 else None
            self._bufs = muon_batch_buffers(_ptr(param), _dtype_code(param), _ptr(grad), _dtype_code(grad),
                                            _ptr(mom), _ptr(out))
            ws = workspaces
            self._fn, self._where = L.muon_step, "muon_step"
            self._args = (plan.handle, batches, C.byref(self._bufs), C.byref(self._hpc), _ptr(ws),
                          ws.numel() * ws.element_size(), _stream(streams))
            return
        n, ns = len(batches), len(streams)
        if len(bufs) != n or len(workspaces) != ns:
            raise ValueError("PreparedStep: one buffer set per batch and one workspace per stream")
        self._arr = (C.c_int32 * n)(*batches)
        self._fb = (muon_batch_buffers * n)()
        for i, t in enumerate(bufs):
            out = t[3] if len(t) > 3 else None
            self._fb[i] = muon_batch_buffers(_ptr(t[0]), _dtype_code(t[0]), _ptr(t[1]), _dtype_code(t[1]),
                                             _ptr(t[2]), _ptr(out))
        self._wp = (C.c_void_p * ns)(*[_ptr(w) for w in workspaces])
        self._wb = (C.c_size_t * ns)(*[0 if w is None else w.numel() * w.element_size() for w in workspaces])
        self._sp = (C.c_void_p * ns)(*[_stream(s) if i == 0 else int(s) for i, s in enumerate(streams)])
        self._fn, self._where = L.muon_step_batches, "muon_step_batches"
        self._args = (plan.handle, n, self._arr, self._fb, C.byref(self._hpc), self._wp, self._wb, self._sp, ns)

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != MUON_OK:
            raise MuonError(st, self._where)


def _check_aligned(addrs, what: str) -> None:
    """The kernels move 16-byte runs: every address must be 16-byte aligned."""
    bad = [a for a in addrs if a % 16]
    if bad:
        raise ValueError(f"{what}: {len(bad)} address(es) not 16-byte aligned (first {bad[0]:#x}); "
                         "the kernels issue 16-byte loads and stores there")


def pointer_table(tensors, device="cuda"):
    """Device array (int64 tensor) of the data pointers of `tensors`, one per
    matrix, for muon_step_ptrs.  Every pointer must be 16-byte aligned
    (ValueError otherwise).  Keep it alive until the step has run."""
    import torch
    ptrs = [t.data_ptr() for t in tensors]
    _check_aligned(ptrs, "pointer_table")
    return torch.tensor(ptrs, dtype=torch.int64, device=device)


def muon_step_ptrs(plan: Plan, batch: int, params, grads, momenta, hp: HParams, workspace,
                   ns_out=None, stream=None, param_dtype=None, grad_dtype=None) -> None:
    """muon_step on per-matrix tensors (muon_step_ptrs): params, grads,
    momenta (and optionally ns_out) are sequences of `count` [M, N] device
    tensors, matrix i of the batch each, or device pointer tables made with
    pointer_table (then param_dtype / grad_dtype, "bf16" or "f32", say what
    they point at).  Nothing is packed or copied."""
    import torch

    def is_table(x):
        return isinstance(x, torch.Tensor) and x.dtype == torch.int64 and x.dim() == 1

    def table(x):
        if x is None:
            return None
        return x if is_table(x) else pointer_table(x)

    def dtype_of(x, given, what):
        if not is_table(x):
            return _dtype_code(x[0])
        if given not in ("bf16", "f32"):
            raise ValueError(f"{what} must be 'bf16' or 'f32' with a pointer table")
        return MUON_BF16 if given == "bf16" else MUON_F32

    tp, tg, tm, tn = table(params), table(grads), table(momenta), table(ns_out)
    if stream is not None:   # tables made here stay allocated until that stream has run the step
        ext = torch.cuda.ExternalStream(int(stream))
        for t in (tp, tg, tm, tn):
            if t is not None:
                t.record_stream(ext)
    pdt = dtype_of(params, param_dtype, "param_dtype")
    gdt = dtype_of(grads, grad_dtype, "grad_dtype")
    hpc, keep = hp.to_c()
    bufs = muon_batch_ptrs(_ptr(tp), pdt, _ptr(tg), gdt, _ptr(tm), _ptr(tn))
    st = lib().muon_step_ptrs(plan.handle, batch, C.byref(bufs), C.byref(hpc), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "muon_step_ptrs")


def row_addresses(t):
    """Start address of every row of t (an int64 CPU tensor, leading indices in
    row-major order).  t may be any strided view whose last dimension is
    contiguous: a slice of rows, a range of columns, every k-th row, or one
    part of an interleaved layout such as W.view(heads, 3, d, H)[:, 0].  Every
    row must start at a 16-byte aligned address (for a column range of bf16
    rows: a first column that is a multiple of 8, and a row stride that keeps
    it so); ValueError otherwise."""
    import torch
    if t.dim() < 2 or (t.stride(-1) != 1 and t.shape[-1] > 1):
        raise ValueError("row_addresses: rows must be contiguous (stride 1 along the last dimension)")
    lead = tuple(t.shape[:-1])
    addr = torch.full(lead, t.data_ptr(), dtype=torch.int64)
    for d, (size, stride) in enumerate(zip(lead, t.stride()[:-1])):
        shape = [1] * len(lead)
        shape[d] = size
        addr = addr + (torch.arange(size, dtype=torch.int64) * (stride * t.element_size())).view(shape)
    addr = addr.reshape(-1)
    if bool((addr % 16 != 0).any()):
        _check_aligned(addr.tolist(), "row_addresses")
    return addr


def row_table(views, device="cuda"):
    """Device row table for muon_step_rows: the rows of each logical matrix
    view in `views`, matrix after matrix (batch order).  Each view's rows,
    flattened over its leading dimensions, are the M stored rows of one
    [M, N] matrix."""
    import torch
    return torch.cat([row_addresses(v) for v in views]).to(device)


def muon_step_rows(plan: Plan, batch: int, param_rows, grad_rows, momentum, hp: HParams, workspace,
                   param_dtype, grad_dtype, ns_out=None, stream=None) -> None:
    """muon_step on row-level views (muon_step_rows): param_rows / grad_rows are
    row tables (row_table) of the logical matrices, param_dtype / grad_dtype
    ("bf16" or "f32") the type of the rows; momentum (and ns_out) contiguous
    [count, M, N] fp32.  The tables must stay alive until the step has run."""
    dt = {"bf16": MUON_BF16, "f32": MUON_F32}
    if param_dtype not in dt or grad_dtype not in dt:
        raise ValueError("param_dtype and grad_dtype must be 'bf16' or 'f32'")
    if stream is not None:
        import torch
        ext = torch.cuda.ExternalStream(int(stream))
        param_rows.record_stream(ext)
        grad_rows.record_stream(ext)
    hpc, keep = hp.to_c()
    bufs = muon_batch_rows(_ptr(param_rows), dt[param_dtype], _ptr(grad_rows), dt[grad_dtype], _ptr(momentum),
                           _ptr(ns_out))
    st = lib().muon_step_rows(plan.handle, batch, C.byref(bufs), C.byref(hpc), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "muon_step_rows")


def plan_lanes(plan: Plan, batches, hp: HParams, nstreams: int):
    """(lane of each batch, workspace bytes of each lane) for muon_step_batches
    over `nstreams` streams (muon_plan_lanes)."""
    n = len(batches)
    arr = (C.c_int32 * n)(*batches)
    lane_of = (C.c_int32 * n)()
    wsb = (C.c_size_t * max(int(nstreams), 1))()
    hpc, keep = hp.to_c()
    _check(lib().muon_plan_lanes(plan.handle, n, arr, C.byref(hpc), int(nstreams), lane_of, wsb), "muon_plan_lanes")
    return list(lane_of), list(wsb)[:int(nstreams)]


def muon_step_batches(plan: Plan, batches, bufs, hp: HParams, workspaces, streams) -> None:
    """One step over several batches on several streams (muon_step_batches).
    bufs[i] = (param, grad, momentum[, ns_out]) of batch batches[i];
    workspaces[l] (uint8 tensor, or None for a lane with no batch) and
    streams[l] (hipStream_t handle as an int; None in place 0 = the current
    stream) per lane."""
    n, ns = len(batches), len(streams)
    if len(bufs) != n or len(workspaces) != ns:
        raise ValueError("muon_step_batches: one buffer set per batch and one workspace per stream")
    arr = (C.c_int32 * n)(*batches)
    fb = (muon_batch_buffers * n)()
    for i, t in enumerate(bufs):
        param, grad, mom = t[0], t[1], t[2]
        out = t[3] if len(t) > 3 else None
        fb[i] = muon_batch_buffers(_ptr(param), _dtype_code(param), _ptr(grad), _dtype_code(grad), _ptr(mom), _ptr(out))
    wp = (C.c_void_p * ns)(*[_ptr(w) for w in workspaces])
    wb = (C.c_size_t * ns)(*[0 if w is None else w.numel() * w.element_size() for w in workspaces])
    sp = (C.c_void_p * ns)(*[_stream(s) if i == 0 else int(s) for i, s in enumerate(streams)])
    hpc, keep = hp.to_c()
    _check(lib().muon_step_batches(plan.handle, n, arr, fb, C.byref(hpc), wp, wb, sp, ns), "muon_step_batches")


def muon_stage_momentum(plan: Plan, batch: int, grad, momentum, u_out, hp: HParams, stream=None) -> None:
    hpc, keep = hp.to_c()
    _check(lib().muon_stage_momentum(plan.handle, batch, _ptr(grad), _dtype_code(grad), _ptr(momentum),
                                     _ptr(u_out), C.byref(hpc), _stream(stream)), "muon_stage_momentum")


def muon_stage_ns(plan: Plan, batch: int, u_in, o_out, hp: HParams, workspace, stream=None) -> None:
    hpc, keep = hp.to_c()
    _check(lib().muon_stage_ns(plan.handle, batch, _ptr(u_in), _ptr(o_out), C.byref(hpc), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)), "muon_stage_ns")


def muon_stage_update(plan: Plan, batch: int, param, o_in, hp: HParams, stream=None) -> None:
    hpc, keep = hp.to_c()
    _check(lib().muon_stage_update(plan.handle, batch, _ptr(param), _dtype_code(param), _ptr(o_in),
                                   C.byref(hpc), _stream(stream)), "muon_stage_update")


def muon_debug_fail_dispatch(n: int) -> None:
    """Failure injection for tests of the error paths: the (n + 1)-th batch
    dispatch from now returns MUON_ERR_HIP without launching anything (then
    the injection is off); n < 0 turns it off."""
    lib().muon_debug_fail_dispatch(int(n))


def muon_trace_start(max_launches: int) -> None:
    _check(lib().muon_trace_start(int(max_launches)), "muon_trace_start")


def muon_trace_stop() -> List[Tuple[str, float]]:
    """(kernel name, milliseconds) of every traced launch, in launch order."""
    L = lib()
    cap = 1 << 16
    ms = (C.c_float * cap)()
    names = (C.c_char_p * cap)()
    n = L.muon_trace_stop(ms, names, cap)
    if n < 0:
        raise RuntimeError("muon_trace_stop: tracing was not started")
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]


class BatchedMuon:
    """All batches of a plan with per-batch contiguous [count, M, N] buffers
    (parameters of a batch are views into its buffer, as in HyperParallel-FSDP
    §6.6's merged tensor).  streams = 1: the batches run in plan order on the
    caller's stream with one workspace sized for the largest batch; streams > 1:
    muon_step_batches spreads them over the caller's stream and streams - 1
    side streams (default priority), one workspace per lane."""

    def __init__(self, shapes, dtype, hp: HParams, device="cuda", max_batch_elems=0, order=0, skinny_kernel=0,
                 streams=1):
        import torch
        self.plan = Plan(shapes, max_batch_elems, order, skinny_kernel)
        self.hp = hp
        self.dtype = dtype
        self.device = device
        self.params, self.grads, self.moms = [], [], []
        for b in self.plan.batches:
            shp = (b.count, b.M, b.N)
            self.params.append(torch.empty(shp, dtype=dtype, device=device))
            self.grads.append(torch.empty(shp, dtype=dtype, device=device))
            self.moms.append(torch.zeros(shp, dtype=torch.float32, device=device))
        self.nstreams = max(1, min(int(streams), len(self.plan.batches)))
        if self.nstreams == 1:
            ws = max(self.plan.workspace_bytes(b.index, hp.precision) for b in self.plan.batches)
            self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
        else:
            idx = [b.index for b in self.plan.batches]
            self.lane_of, need = plan_lanes(self.plan, idx, hp, self.nstreams)
            self.workspaces = [torch.empty(max(w, 256), dtype=torch.uint8, device=device) if w else None
                               for w in need]
            self.side_streams = [torch.cuda.Stream(device=device) for _ in range(self.nstreams - 1)]

    def step(self, ns_outs=None, stream=None):
        if self.nstreams == 1:
            for b in self.plan.batches:
                muon_step(self.plan, b.index, self.params[b.index], self.grads[b.index], self.moms[b.index],
                          self.hp, self.workspace, None if ns_outs is None else ns_outs[b.index], stream)
            return
        bufs = [(self.params[b.index], self.grads[b.index], self.moms[b.index],
                 None if ns_outs is None else ns_outs[b.index]) for b in self.plan.batches]
        muon_step_batches(self.plan, [b.index for b in self.plan.batches], bufs, self.hp, self.workspaces,
                          [stream] + [s.cuda_stream for s in self.side_streams])

    def capture_graph(self, ns_outs=None):
        """Record one step (every batch) into a HIP graph (torch.cuda.CUDAGraph)
        and return it; graph.replay() then runs a step on the same buffers
        (and writes O into ns_outs, one [count, M, N] fp32 tensor per batch,
        if given).  With hp.lr_wd set, the learning rate and decay written
        into that device tensor before a replay are the ones the replay uses."""
        import torch
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                self.step(ns_outs)
        torch.cuda.current_stream().wait_stream(side)
        return graph
