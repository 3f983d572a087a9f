"""muon_step_noalloc, called through the C ABI: bit-identical to muon_step
with a workspace on the same inputs, on two calls in a row (the second on a
smaller parameter set than the first, so it runs on what the first left in
the shared scratch array), and it rejects a plan whose workspace exceeds the
array before touching anything."""
from __future__ import annotations

import ctypes

import pytest
import torch

from newton_schulz_05_amd import binding as B
from newton_schulz_05_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCRATCH_BYTES = 64 << 20


def _plan(shapes):
    lib = B.load_library()
    cs = [B.MuonShape(*B._as_shape(s)) for s in shapes]
    arr = (B.MuonShape * len(cs))(*cs)
    h = ctypes.c_void_p()
    assert lib.muon_plan_create(arr, len(cs), B.MUON_BF16, B.MUON_BF16, B.MUON_F32, ctypes.byref(h)) == 0
    nb = ctypes.c_size_t()
    assert lib.muon_plan_workspace_bytes(h, ctypes.byref(nb)) == 0
    return lib, h, arr, int(nb.value)


def _hyper(lr=0.02):
    return (lr, 0.95, 1, 0.1, 3.4445, -4.7750, 2.0315, 5, 1.0)


def _run(shapes, number, steps=2):
    """Both entry points on copies of the same seeded inputs, `steps`
    consecutive steps with fresh gradients; returns (W, M) of each."""
    lib, h, arr, wsb = _plan(shapes)
    assert wsb <= SCRATCH_BYTES
    wl = WL.custom(shapes, number=number)
    p0 = WL.make_params(wl, DEV, "cpu")
    grads = [WL.make_grads(wl, s, DEV, "cpu") for s in range(steps)]
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for variant in ("workspace", "noalloc"):
        ps = [p.clone() for p in p0]
        ms = [torch.zeros(p.shape, dtype=torch.float32, device=DEV) for p in p0]
        for s in range(steps):
            args = (h, B._ptrs(ps), B._ptrs(grads[s]), B._ptrs(ms), arr, len(shapes)) + _hyper()
            if variant == "workspace":
                rc = lib.muon_step(*args, ctypes.c_void_p(ws.data_ptr()), wsb, st)
            else:
                rc = lib.muon_step_noalloc(*args, st)
            assert rc == 0, lib.muon_last_error_detail().decode()
        torch.cuda.synchronize()
        out.append((ps, ms))
    lib.muon_plan_destroy(h)
    return out


def test_noalloc_matches_workspace_step_on_two_calls():
    big = [(24, 10240)] * 20 + [(96, 640)] * 3 + [(640, 96)]
    small = [(24, 3000)] * 4 + [(64, 200)]
    for shapes, number in ((big, 81), (small, 82)):
        (pw, mw), (pn, mn) = _run(shapes, number)
        for i in range(len(shapes)):
            assert torch.equal(pw[i], pn[i]), f"W[{i}] of {shapes[i]} differs"
            assert torch.equal(mw[i], mn[i]), f"M[{i}] of {shapes[i]} differs"


def test_noalloc_rejects_a_plan_beyond_the_scratch_array():
    shapes = [(1536, 2048)] * 8
    lib, h, arr, wsb = _plan(shapes)
    assert wsb > SCRATCH_BYTES
    ptrs = (ctypes.c_void_p * 8)(*([0x10000] * 8))  # never dereferenced: rejected first
    rc = lib.muon_step_noalloc(h, ptrs, ptrs, ptrs, arr, 8, *_hyper(), None)
    assert rc == 5  # MUON_ERR_WORKSPACE
    assert "scratch" in lib.muon_last_error_detail().decode()
    lib.muon_plan_destroy(h)
