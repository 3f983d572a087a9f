"""ctypes binding of libmuon_hip.so (include/muon.h).

Argument marshalling only: every step of the Muon update runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
If the library has not been built the first call raises
``MuonLibraryMissing``; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuon_hip.so")

MUON_F32 = 0
MUON_BF16 = 1

STATUS = {
    0: "MUON_OK",
    1: "MUON_ERR_INVALID_ARG",
    2: "MUON_ERR_SHAPE",
    3: "MUON_ERR_DTYPE",
    4: "MUON_ERR_PLAN_MISMATCH",
    5: "MUON_ERR_WORKSPACE",
    6: "MUON_ERR_HIP",
    7: "MUON_ERR_ALIGNMENT",
    8: "MUON_ERR_TIMEOUT",
}

EXPORTS = ["muon_plan_create", "muon_plan_destroy", "muon_plan_workspace_bytes",
           "muon_plan_num_groups", "muon_plan_group_info", "muon_step", "muon_ns",
           "muon_plan_num_matrices", "muon_plan_assign", "muon_shard_update", "muon_adamw_step",
           "muon_workspace_status", "muon_set_wait_limit", "muon_set_side_stream", "muon_poll_timeout",
           "muon_step_noalloc",
           "muon_kernel_timing", "muon_kernel_timing_read",
           "muon_status_str", "muon_last_error_detail", "muon_version"]


class MuonLibraryMissing(RuntimeError):
    pass


class MuonError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        self.detail = detail
        super().__init__(f"{self.name}: {detail}")


class MuonShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raise MuonLibraryMissing if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MuonLibraryMissing(
            f"{path} not found: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, sz, i32, i64, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    P = ctypes.POINTER
    lib.muon_plan_create.argtypes = [P(MuonShape), i32, i32, i32, i32, P(vp)]
    lib.muon_plan_create.restype = i32
    lib.muon_plan_destroy.argtypes = [vp]
    lib.muon_plan_destroy.restype = None
    lib.muon_plan_workspace_bytes.argtypes = [vp, P(sz)]
    lib.muon_plan_workspace_bytes.restype = i32
    lib.muon_plan_num_groups.argtypes = [vp, P(i32)]
    lib.muon_plan_num_groups.restype = i32
    lib.muon_plan_group_info.argtypes = [vp, i32, P(i64), P(i64), P(i64), P(i64), P(i64)]
    lib.muon_plan_group_info.restype = i32
    lib.muon_step.argtypes = [vp, P(vp), P(vp), P(vp), P(MuonShape), i32, f32, f32, i32, f32,
                              f32, f32, f32, i32, f32, vp, sz, vp]
    lib.muon_step.restype = i32
    lib.muon_step_noalloc.argtypes = [vp, P(vp), P(vp), P(vp), P(MuonShape), i32, f32, f32, i32, f32,
                                      f32, f32, f32, i32, f32, vp]
    lib.muon_step_noalloc.restype = i32
    lib.muon_ns.argtypes = [vp, P(vp), P(vp), P(MuonShape), i32, f32, f32, f32, i32, vp, sz, vp]
    lib.muon_ns.restype = i32
    lib.muon_plan_num_matrices.argtypes = [vp, P(i64)]
    lib.muon_plan_num_matrices.restype = i32
    lib.muon_plan_assign.argtypes = [vp, i32, P(i32), i64, P(ctypes.c_double)]
    lib.muon_plan_assign.restype = i32
    lib.muon_shard_update.argtypes = [vp, i32, vp, i64, i64, f32, f32, f32, vp]
    lib.muon_shard_update.restype = i32
    lib.muon_adamw_step.argtypes = [P(vp), P(vp), P(vp), P(vp), P(i64), i32, i32, f32, f32, f32, f32, f32, i64, vp]
    lib.muon_adamw_step.restype = i32
    lib.muon_workspace_status.argtypes = [vp, vp, sz, vp, P(i32)]
    lib.muon_workspace_status.restype = i32
    lib.muon_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.muon_set_wait_limit.restype = None
    lib.muon_set_side_stream.argtypes = [i32]
    lib.muon_set_side_stream.restype = None
    lib.muon_poll_timeout.argtypes = [P(i32)]
    lib.muon_poll_timeout.restype = i32
    lib.muon_kernel_timing.argtypes = [i32]
    lib.muon_kernel_timing.restype = i32
    lib.muon_kernel_timing_read.argtypes = [P(ctypes.c_double), P(i64), P(ctypes.c_double), P(ctypes.c_double)]
    lib.muon_kernel_timing_read.restype = i32
    lib.muon_status_str.argtypes = [i32]
    lib.muon_status_str.restype = ctypes.c_char_p
    lib.muon_last_error_detail.argtypes = []
    lib.muon_last_error_detail.restype = ctypes.c_char_p
    lib.muon_version.argtypes = []
    lib.muon_version.restype = i32
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        detail = load_library().muon_last_error_detail().decode()
        raise MuonError(status, detail)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return MUON_F32
    if dt == torch.bfloat16:
        return MUON_BF16
    raise MuonError(3, f"unsupported dtype {dt}")


def _as_shape(s: Sequence[int]) -> Tuple[int, int, int]:
    s = tuple(int(x) for x in s)
    if len(s) == 2:
        return (1, s[0], s[1])
    if len(s) == 3:
        return s
    raise MuonError(2, f"parameters must be 2-D or 3-D, got shape {s}")


def _ptrs(tensors: Sequence[torch.Tensor]):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


class MuonPlan:
    """Grouping plan for a fixed list of parameter shapes (muon_plan_create)."""

    def __init__(self, shapes: Sequence[Sequence[int]], dtype: torch.dtype = torch.bfloat16):
        lib = load_library()
        self.shapes = [_as_shape(s) for s in shapes]
        self.orig_shapes = [tuple(int(x) for x in s) for s in shapes]
        self.dtype = dtype
        n = len(self.shapes)
        self._cshapes = (MuonShape * max(n, 1))(*[MuonShape(*s) for s in self.shapes])
        h = ctypes.c_void_p()
        code = _dtype_code(dtype)
        _check(lib.muon_plan_create(self._cshapes, n, code, code, MUON_F32, ctypes.byref(h)))
        self._h = h
        b = ctypes.c_size_t()
        _check(lib.muon_plan_workspace_bytes(self._h, ctypes.byref(b)))
        self.workspace_bytes = int(b.value)

    @classmethod
    def for_params(cls, params: Sequence[torch.Tensor]) -> "MuonPlan":
        dts = {p.dtype for p in params}
        if len(dts) != 1:
            raise MuonError(3, "all parameters of one plan share a dtype")
        return cls([tuple(p.shape) for p in params], dts.pop())

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.muon_plan_destroy(h)
            self._h = None

    def groups(self) -> List[dict]:
        lib = load_library()
        n = ctypes.c_int32()
        _check(lib.muon_plan_num_groups(self._h, ctypes.byref(n)))
        out = []
        for g in range(n.value):
            v = [ctypes.c_int64() for _ in range(5)]
            _check(lib.muon_plan_group_info(self._h, g, *[ctypes.byref(x) for x in v]))
            out.append(dict(m=v[0].value, n=v[1].value, count=v[2].value,
                            n_transposed=v[3].value, n_chunks=v[4].value))
        return out

    def num_matrices(self) -> int:
        """Matrices of the plan: 1 per 2-D parameter, E per expert slab."""
        n = ctypes.c_int64()
        _check(load_library().muon_plan_num_matrices(self._h, ctypes.byref(n)))
        return int(n.value)

    def matrices(self) -> List[Tuple[int, int]]:
        """(parameter index, slice index) of every matrix, in plan order."""
        out = []
        for i, (b, _, _) in enumerate(self.shapes):
            out.extend((i, e) for e in range(b))
        return out

    def assign(self, n_ranks: int) -> Tuple[List[int], List[float]]:
        """Greedy whole-matrix split over n_ranks (muon_plan_assign): the
        owner rank of every matrix and each rank's total NS cost."""
        nm = self.num_matrices()
        owner = (ctypes.c_int32 * max(nm, 1))()
        cost = (ctypes.c_double * max(int(n_ranks), 1))()
        _check(load_library().muon_plan_assign(self._h, int(n_ranks), owner, nm, cost))
        return [int(owner[j]) for j in range(nm)], [float(cost[r]) for r in range(int(n_ranks))]

    def workspace_timed_out(self, workspace: torch.Tensor, stream=None) -> bool:
        """Synchronise the stream and report (and clear) the skinny path's
        timeout flag in `workspace` (muon_workspace_status)."""
        flag = ctypes.c_int32()
        _check(load_library().muon_workspace_status(self._h, ctypes.c_void_p(workspace.data_ptr()),
                                                    workspace.numel(), ctypes.c_void_p(self._stream(stream)),
                                                    ctypes.byref(flag)))
        return bool(flag.value)

    def rank_views(self, tensors: Sequence[torch.Tensor], owner: Sequence[int], rank: int) -> List[torch.Tensor]:
        """The matrices that `owner` (from assign) gives to `rank`, as 2-D
        views of `tensors` (a parameter, or one slice of an expert slab), in
        plan order.  A plan built over their shapes steps exactly those
        matrices in place."""
        mats = self.matrices()
        if len(owner) != len(mats):
            raise MuonError(1, f"owner has {len(owner)} entries for {len(mats)} matrices")
        out = []
        for (i, e), o in zip(mats, owner):
            if o == rank:
                t = tensors[i]
                out.append(t[e] if t.dim() == 3 else t)
        return out

    def new_workspace(self, device="cuda") -> torch.Tensor:
        """Zero-filled workspace of the plan's size (a torch uint8 tensor)."""
        return torch.zeros(self.workspace_bytes, dtype=torch.uint8, device=device)

    def _check_tensors(self, ts: Sequence[torch.Tensor], dtype: torch.dtype, what: str):
        if len(ts) != len(self.shapes):
            raise MuonError(4, f"{what}: {len(ts)} tensors for a plan of {len(self.shapes)}")
        for i, t in enumerate(ts):
            if t.dtype != dtype:
                raise MuonError(3, f"{what}[{i}] has dtype {t.dtype}, expected {dtype}")
            if not t.is_contiguous():
                raise MuonError(1, f"{what}[{i}] is not contiguous")
            if not t.is_cuda:
                raise MuonError(1, f"{what}[{i}] is not a device tensor")
            if _as_shape(t.shape) != self.shapes[i]:
                raise MuonError(4, f"{what}[{i}] has shape {tuple(t.shape)}")

    @staticmethod
    def _stream(stream) -> int:
        s = stream if stream is not None else torch.cuda.current_stream()
        return int(s.cuda_stream)

    def step(self, params, grads, moms, *, lr: float, mu: float = 0.95, nesterov: bool = True,
             wd: float = 0.0, coeffs=(3.4445, -4.7750, 2.0315), ns_steps: int = 5,
             scale: float = 1.0, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
        """One Muon step (muon_step), enqueued on `stream` (default: current)."""
        lib = load_library()
        self._check_tensors(params, self.dtype, "params")
        self._check_tensors(grads, self.dtype, "grads")
        self._check_tensors(moms, torch.float32, "moms")
        if workspace is None:
            workspace = self._default_ws(params[0].device)
        a, b, c = (float(x) for x in coeffs)
        _check(lib.muon_step(self._h, _ptrs(params), _ptrs(grads), _ptrs(moms), self._cshapes,
                             len(self.shapes), float(lr), float(mu), int(bool(nesterov)), float(wd),
                             a, b, c, int(ns_steps), float(scale), ctypes.c_void_p(workspace.data_ptr()),
                             workspace.numel(), ctypes.c_void_p(self._stream(stream))))

    def step_noalloc(self, params, grads, moms, *, lr: float, mu: float = 0.95, nesterov: bool = True,
                     wd: float = 0.0, coeffs=(3.4445, -4.7750, 2.0315), ns_steps: int = 5,
                     scale: float = 1.0, stream=None) -> None:
        """One Muon step without a workspace (muon_step_noalloc): the library's
        64 MiB static device array serves as workspace, shared by every such
        call on the device.  For plans whose workspace fits in it."""
        lib = load_library()
        self._check_tensors(params, self.dtype, "params")
        self._check_tensors(grads, self.dtype, "grads")
        self._check_tensors(moms, torch.float32, "moms")
        a, b, c = (float(x) for x in coeffs)
        _check(lib.muon_step_noalloc(self._h, _ptrs(params), _ptrs(grads), _ptrs(moms), self._cshapes,
                                     len(self.shapes), float(lr), float(mu), int(bool(nesterov)), float(wd),
                                     a, b, c, int(ns_steps), float(scale), ctypes.c_void_p(self._stream(stream))))

    def ns(self, inputs, outputs, *, coeffs=(3.4445, -4.7750, 2.0315), ns_steps: int = 5,
           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
        """Newton-Schulz alone (muon_ns): outputs (fp32) = NS(inputs)."""
        lib = load_library()
        self._check_tensors(inputs, self.dtype, "inputs")
        self._check_tensors(outputs, torch.float32, "outputs")
        if workspace is None:
            workspace = self._default_ws(inputs[0].device)
        a, b, c = (float(x) for x in coeffs)
        _check(lib.muon_ns(self._h, _ptrs(inputs), _ptrs(outputs), self._cshapes, len(self.shapes),
                           a, b, c, int(ns_steps), ctypes.c_void_p(workspace.data_ptr()),
                           workspace.numel(), ctypes.c_void_p(self._stream(stream))))

    def bind(self, params, grads, moms, *, workspace: Optional[torch.Tensor] = None) -> "BoundStep":
        """Validate the tensors once and keep their pointer arrays, so that
        repeated steps over the same tensors cost one C call each."""
        self._check_tensors(params, self.dtype, "params")
        self._check_tensors(grads, self.dtype, "grads")
        self._check_tensors(moms, torch.float32, "moms")
        if workspace is None:
            workspace = self._default_ws(params[0].device)
        return BoundStep(self, params, grads, moms, workspace)

    def bind_ns(self, inputs, outputs, *, workspace: Optional[torch.Tensor] = None) -> "BoundNS":
        """Validate NS inputs and fp32 outputs once (see bind)."""
        self._check_tensors(inputs, self.dtype, "inputs")
        self._check_tensors(outputs, torch.float32, "outputs")
        if workspace is None:
            workspace = self._default_ws(inputs[0].device)
        return BoundNS(self, inputs, outputs, workspace)

    def _default_ws(self, device) -> torch.Tensor:
        ws = getattr(self, "_ws", None)
        if ws is None or ws.device != device:
            ws = self.new_workspace(device)
            self._ws = ws
        return ws


class BoundStep:
    """muon_step over a fixed set of tensors (see MuonPlan.bind).  The tensors
    are kept alive by this object; their storage must not be reallocated."""

    def __init__(self, plan: MuonPlan, params, grads, moms, workspace: torch.Tensor):
        self.plan = plan
        self._keep = (list(params), list(grads), list(moms), workspace)
        self._p, self._g, self._m = _ptrs(params), _ptrs(grads), _ptrs(moms)
        self._ws = ctypes.c_void_p(workspace.data_ptr())
        self._ws_bytes = workspace.numel()
        self._lib = load_library()

    def step(self, *, lr: float, mu: float = 0.95, nesterov: bool = True, wd: float = 0.0,
             coeffs=(3.4445, -4.7750, 2.0315), ns_steps: int = 5, scale: float = 1.0, stream=None) -> None:
        a, b, c = coeffs
        _check(self._lib.muon_step(self.plan._h, self._p, self._g, self._m, self.plan._cshapes,
                                   len(self.plan.shapes), lr, mu, 1 if nesterov else 0, wd, a, b, c,
                                   ns_steps, scale, self._ws, self._ws_bytes,
                                   ctypes.c_void_p(MuonPlan._stream(stream))))


def shard_update(w_shard: torch.Tensor, o_full: torch.Tensor, offset: int, *, lr: float, wd: float = 0.0,
                 scale: float = 1.0, stream=None) -> None:
    """One rank's flat shard of a parameter takes the decoupled update from
    the full O (muon_shard_update): w_shard = W.flatten()[offset:offset+len]."""
    lib = load_library()
    if not (w_shard.is_cuda and o_full.is_cuda):
        raise MuonError(1, "w_shard and o_full must be device tensors")
    if not (w_shard.is_contiguous() and o_full.is_contiguous()):
        raise MuonError(1, "w_shard and o_full must be contiguous")
    if o_full.dtype != torch.float32:
        raise MuonError(3, "o_full must be float32")
    if offset < 0 or offset + w_shard.numel() > o_full.numel():
        raise MuonError(1, f"shard [{offset}, {offset + w_shard.numel()}) is outside O of {o_full.numel()} elements")
    _check(lib.muon_shard_update(ctypes.c_void_p(w_shard.data_ptr()), _dtype_code(w_shard.dtype),
                                 ctypes.c_void_p(o_full.data_ptr()), int(offset), w_shard.numel(), float(lr),
                                 float(wd), float(scale), ctypes.c_void_p(MuonPlan._stream(stream))))


class AdamWGroup:
    """A fixed list of 1-D parameters with their gradients and fp32 moment
    buffers for muon_adamw_step.  The tensors are validated once and their
    pointer arrays kept, so each step() is one C call; their storage must not
    be reallocated while the group is in use."""

    def __init__(self, params, grads, exp_avgs, exp_avg_sqs):
        n = len(params)
        if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == n):
            raise MuonError(1, "params, grads, exp_avgs and exp_avg_sqs must have the same length")
        self.dtype = params[0].dtype if n else torch.float32
        for i in range(n):
            p, g, m, v = params[i], grads[i], exp_avgs[i], exp_avg_sqs[i]
            if p.dtype != self.dtype or g.dtype != self.dtype:
                raise MuonError(3, f"tensor {i}: params and grads must all be {self.dtype}")
            if m.dtype != torch.float32 or v.dtype != torch.float32:
                raise MuonError(3, f"tensor {i}: moment buffers must be float32")
            if not (p.numel() == g.numel() == m.numel() == v.numel()):
                raise MuonError(2, f"tensor {i}: element counts differ")
            if not all(t.is_cuda and t.is_contiguous() for t in (p, g, m, v)):
                raise MuonError(1, f"tensor {i}: tensors must be contiguous device tensors")
        self.n = n
        self._keep = (list(params), list(grads), list(exp_avgs), list(exp_avg_sqs))
        self._p, self._g, self._m, self._v = _ptrs(params), _ptrs(grads), _ptrs(exp_avgs), _ptrs(exp_avg_sqs)
        self._numels = (ctypes.c_int64 * max(n, 1))(*[t.numel() for t in params])
        self._dt = _dtype_code(self.dtype)
        self._lib = load_library()

    def step(self, *, lr: float, betas=(0.9, 0.999), eps: float = 1e-8, wd: float = 0.0, step: int,
             stream=None) -> None:
        b1, b2 = betas
        _check(self._lib.muon_adamw_step(self._p, self._g, self._m, self._v, self._numels, self.n, self._dt,
                                         lr, b1, b2, eps, wd, step, ctypes.c_void_p(MuonPlan._stream(stream))))


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, *, lr: float, betas=(0.9, 0.999), eps: float = 1e-8,
               wd: float = 0.0, step: int, stream=None) -> None:
    """AdamW on a list of 1-D parameters in one call (muon_adamw_step).
    params/grads share a dtype (bf16 or fp32); the moment buffers are fp32."""
    AdamWGroup(params, grads, exp_avgs, exp_avg_sqs).step(lr=lr, betas=betas, eps=eps, wd=wd, step=step,
                                                          stream=stream)


def poll_timeout() -> bool:
    """True if a skinny-path launch on the current device that has completed
    by now timed out since the last check (muon_poll_timeout); clears the
    report.  No synchronisation: synchronise first to cover every launch."""
    flag = ctypes.c_int32()
    _check(load_library().muon_poll_timeout(ctypes.byref(flag)))
    return bool(flag.value)


def kernel_timing(enable: bool) -> None:
    """Start or stop event timing of the MFMA path's apply launches
    (muon_kernel_timing); for benchmarks."""
    _check(load_library().muon_kernel_timing(1 if enable else 0))


def kernel_timing_read() -> dict:
    """Summed duration (ms), count, algorithmic and executed flops of the
    applies timed since the last read (muon_kernel_timing_read)."""
    ms, n, alg, ex = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
    _check(load_library().muon_kernel_timing_read(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(alg),
                                                  ctypes.byref(ex)))
    return dict(ms=ms.value, launches=int(n.value), alg_flops=alg.value, exec_flops=ex.value)


def set_wait_limit(polls: int) -> None:
    """Polls before a waiting workgroup of the skinny kernel gives up
    (muon_set_wait_limit; 0 restores the default)."""
    load_library().muon_set_wait_limit(int(polls))


def set_side_stream(enable: bool) -> None:
    """Whether small MFMA groups may run their R chain on the plan's side
    stream (muon_set_side_stream; on by default, never changes a result)."""
    load_library().muon_set_side_stream(1 if enable else 0)


class BoundNS:
    """muon_ns over a fixed set of tensors (see MuonPlan.bind_ns)."""

    def __init__(self, plan: MuonPlan, inputs, outputs, workspace: torch.Tensor):
        self.plan = plan
        self._keep = (list(inputs), list(outputs), workspace)
        self._i, self._o = _ptrs(inputs), _ptrs(outputs)
        self._ws = ctypes.c_void_p(workspace.data_ptr())
        self._ws_bytes = workspace.numel()
        self._lib = load_library()

    def ns(self, *, coeffs=(3.4445, -4.7750, 2.0315), ns_steps: int = 5, stream=None) -> None:
        a, b, c = coeffs
        _check(self._lib.muon_ns(self.plan._h, self._i, self._o, self.plan._cshapes, len(self.plan.shapes),
                                 a, b, c, ns_steps, self._ws, self._ws_bytes,
                                 ctypes.c_void_p(MuonPlan._stream(stream))))
