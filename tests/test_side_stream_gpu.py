"""The side stream of small MFMA groups changes when launches run, never a
bit: steps and Newton-Schulz alone with it (the default) and without it
(muon_set_side_stream(0)) must agree bit for bit.  The shapes take the
overlap, each group's m x m launches holding fewer tiles than the device has
compute units: the precise chain in a group of 4 steps (512 x 1024, the MoE
experts' 1536 x 2048 stored tall), the whole recipe in one group of 5 steps
(300 x 700) and the lean recipe's bf16 chain (4096 x 4096, one matrix)."""
from __future__ import annotations

import pytest
import torch

from newton_schulz_05_amd import MuonPlan
from newton_schulz_05_amd import binding as B
from newton_schulz_05_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda"

SHAPES = [(512, 1024)] * 4 + [(300, 700)] * 3 + [(2048, 1536)] * 2 + [(4096, 4096)]


def _steps(plan, wl, side: bool, steps: int = 3):
    B.set_side_stream(side)
    try:
        ws = plan.new_workspace(DEV)
        params = WL.make_params(wl, DEV, "cpu")
        moms = WL.make_moms(wl, DEV)
        for s in range(steps):
            plan.step(params, WL.make_grads(wl, s, DEV, "cpu"), moms, **wl.hyper(), workspace=ws)
        outs = [torch.empty(p.shape, dtype=torch.float32, device=DEV) for p in params]
        plan.ns(WL.make_grads(wl, 7, DEV, "cpu"), outs, workspace=ws)
        torch.cuda.synchronize()
        assert not plan.workspace_timed_out(ws)
        return params, moms, outs
    finally:
        B.set_side_stream(True)


def test_side_stream_is_bitwise_neutral():
    wl = WL.custom(SHAPES, g_std=1e-2, number=85)
    plan = MuonPlan(wl.shapes, wl.dtype)
    with_side = _steps(plan, wl, True)
    without = _steps(plan, wl, False)
    again = _steps(plan, wl, True)  # the side stream made by the first run, used again
    for name, a, b, c in zip(("W", "M", "O"), with_side, without, again):
        for i, s in enumerate(SHAPES):
            assert torch.equal(a[i], b[i]), f"{name}[{i}] of {s} differs without the side stream"
            assert torch.equal(a[i], c[i]), f"{name}[{i}] of {s} differs between runs with it"


def test_plan_destroyed_right_after_its_steps():
    """Steps whose R launches went to the side stream, then the plan is
    destroyed before anything is synchronised: the results must be those of
    the same steps without the side stream (the destructor waits for the
    side stream before it releases the stream and its events)."""
    import gc
    shapes = [(512, 1024)] * 4 + [(300, 700)] * 2
    wl = WL.custom(shapes, g_std=1e-2, number=86)
    ref = _steps(MuonPlan(wl.shapes, wl.dtype), wl, False)
    plan = MuonPlan(wl.shapes, wl.dtype)
    ws = plan.new_workspace(DEV)
    params = WL.make_params(wl, DEV, "cpu")
    moms = WL.make_moms(wl, DEV)
    grads = [WL.make_grads(wl, s, DEV, "cpu") for s in range(3)]
    torch.cuda.synchronize()
    for s in range(3):
        plan.step(params, grads[s], moms, **wl.hyper(), workspace=ws)
    del plan
    gc.collect()
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        assert torch.equal(params[i], ref[0][i]), f"W[{i}] of {s} differs"
        assert torch.equal(moms[i], ref[1][i]), f"M[{i}] of {s} differs"
