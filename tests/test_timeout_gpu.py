"""The skinny path's bounded waits: a forced timeout (a wait limit of one
poll, set from the host) is reported by muon_workspace_status and by the
status of the next call, the workgroups that gave up leave W unwritten, the
kernel still completes, and after the default limit is restored the flags
clear and results are correct again.  No kernel faults or hangs: every wait
is bounded and the grid drains."""
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


def _slabs_written_or_untouched(params, slab_w):
    """Each workgroup owns one column slab of one matrix and either writes
    all of it or (after a timed-out wait) none of it.  W starts at zero and
    the step writes O (lr = -1, wd = 0), so an untouched slab is all zero.
    Returns the number of untouched slabs."""
    untouched = 0
    for p in params:
        for c0 in range(0, p.shape[1], slab_w):
            blk = p[:, c0:c0 + slab_w]
            nz = int(torch.count_nonzero(blk))
            assert nz == 0 or nz >= 0.99 * blk.numel(), f"slab at column {c0} partly written ({nz}/{blk.numel()})"
            untouched += nz == 0
    return untouched


def test_forced_timeout_is_reported_and_clears():
    wl = WL.WORKLOADS["c2"]
    plan = MuonPlan(wl.shapes, wl.dtype)
    ws = plan.new_workspace(DEV)
    moms = WL.make_moms(wl, DEV)
    grads = WL.make_grads(wl, 0, DEV, DEV)
    params = [torch.zeros(s, dtype=wl.dtype, device=DEV) for s in wl.shapes]
    kw = dict(wl.hyper())
    kw.update(lr=-1.0, wd=0.0)
    plan.step(params, grads, moms, **kw, workspace=ws)  # a clean call first
    torch.cuda.synchronize()
    assert not plan.workspace_timed_out(ws)
    assert not B.poll_timeout()
    try:
        B.set_wait_limit(1)
        seen = False
        for _ in range(10):  # 740 workgroups: some always wait longer than one poll
            for p in params:
                p.zero_()
            plan.step(params, grads, moms, **kw, workspace=ws)
            if plan.workspace_timed_out(ws):
                seen = True
                break
        assert seen, "a one-poll wait limit never timed out"
    finally:
        B.set_wait_limit(0)
    assert not plan.workspace_timed_out(ws), "the workspace flag was not cleared"
    # the workgroups that gave up left their slabs of W unwritten
    assert _slabs_written_or_untouched(params, 1024) >= 1
    # the next call reports the timeout through its status and enqueues nothing
    w_before = [p.clone() for p in params]
    m_before = [m.clone() for m in moms]
    with pytest.raises(B.MuonError) as ei:
        plan.step(params, grads, moms, **kw, workspace=ws)
    assert ei.value.status == 8
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(params, w_before))
    assert all(torch.equal(a, b) for a, b in zip(moms, m_before))
    assert not B.poll_timeout(), "the host-visible report was not cleared"
    # a clean step afterwards: O read back through W = 0, wd = 0, lr = -1
    for p in params:
        p.zero_()
    for m in moms:
        m.zero_()
    plan.step(params, grads, moms, **kw, workspace=ws)
    assert not plan.workspace_timed_out(ws)
    assert not B.poll_timeout()
    a, b, c = wl.coeffs
    for i in (0, 37, 73):
        o_ref = ref.newton_schulz((1.0 + wl.mu) * host64(grads[i]), a, b, c, wl.ns_steps)
        check_o(host64(params[i]), o_ref, True, f"O[{i}] after the timeout test")
