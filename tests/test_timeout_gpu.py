"""The skinny path's bounded waits: a forced timeout (a wait limit of one
poll, set from the host) is reported by muon_workspace_status, the kernel
still completes, and after the default limit is restored the flag clears and
results are correct again.  No kernel faults or hangs: every wait is bounded
and the grid drains."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from newton_schulz_05_amd import MuonPlan
from newton_schulz_05_amd import binding as B
from newton_schulz_05_amd import workloads as WL
from oracle import muon_ref as ref
from tests.helpers import check_o, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_forced_timeout_is_reported_and_clears():
    wl = WL.WORKLOADS["c2"]
    plan = MuonPlan(wl.shapes, wl.dtype)
    ws = plan.new_workspace(DEV)
    moms = WL.make_moms(wl, DEV)
    grads = WL.make_grads(wl, 0, DEV, DEV)
    params = [torch.zeros(s, dtype=wl.dtype, device=DEV) for s in wl.shapes]
    assert not plan.workspace_timed_out(ws)
    try:
        B.set_wait_limit(1)
        seen = False
        for _ in range(10):  # 740 workgroups: some always wait longer than one poll
            plan.step(params, grads, moms, **wl.hyper(), workspace=ws)
            if plan.workspace_timed_out(ws):
                seen = True
                break
        assert seen, "a one-poll wait limit never timed out"
    finally:
        B.set_wait_limit(0)
    assert not plan.workspace_timed_out(ws), "the flag was not cleared"
    # a clean step afterwards: O read back through W = 0, wd = 0, lr = -1
    for p in params:
        p.zero_()
    for m in moms:
        m.zero_()
    kw = dict(wl.hyper())
    kw.update(lr=-1.0, wd=0.0)
    plan.step(params, grads, moms, **kw, workspace=ws)
    assert not plan.workspace_timed_out(ws)
    a, b, c = wl.coeffs
    for i in (0, 37, 73):
        o_ref = ref.newton_schulz((1.0 + wl.mu) * host64(grads[i]), a, b, c, wl.ns_steps)
        check_o(host64(params[i]), o_ref, True, f"O[{i}] after the timeout test")
