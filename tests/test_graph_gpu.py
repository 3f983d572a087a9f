"""muon_step recorded into a HIP graph (through torch.cuda.graph) and
replayed: every replay must give bit for bit what the same step gives eagerly.
The skinny launches of a recorded step number themselves from a counter in
the workspace (a one-thread kernel advances it before each), so replays never
reuse an exchange tag.  Between replays the program runs its own eager steps
on the same workspace and synchronises, and each replay is checked."""
from __future__ import annotations

import pytest
import torch

from newton_schulz_05_amd import MuonPlan
from newton_schulz_05_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("shapes", [
    [(24, 3000)] * 6 + [(96, 640), (640, 96)],
    [(24, 10240)] * 74,
], ids=["skinny_and_mfma", "skinny_74x24x10240"])
def test_graph_replays_match_eager_steps(shapes):
    wl = WL.custom(shapes, g_std=1e-2, number=81)
    plan = MuonPlan(wl.shapes, wl.dtype)
    ws = plan.new_workspace(DEV)
    p_eager = WL.make_params(wl, DEV, "cpu")
    p_graph = [p.clone() for p in p_eager]
    m_eager = WL.make_moms(wl, DEV)
    m_graph = WL.make_moms(wl, DEV)
    gsets = [WL.make_grads(wl, s, DEV, "cpu") for s in range(3)]
    gbuf = [g.clone() for g in gsets[0]]          # the graph reads gradients from here
    hyper = wl.hyper()
    bound = plan.bind(p_graph, gbuf, m_graph, workspace=ws)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            bound.step(**hyper, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # recording ran nothing
    assert all(torch.equal(a, b) for a, b in zip(p_graph, p_eager))

    for s in range(3):
        for dst, src in zip(gbuf, gsets[s]):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        plan.step(p_eager, gsets[s], m_eager, **hyper, workspace=ws)   # eager, same workspace
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(p_graph[i], p_eager[i]), f"replay {s}: W[{i}] differs from the eager step"
            assert torch.equal(m_graph[i], m_eager[i]), f"replay {s}: M[{i}] differs from the eager step"
    assert not plan.workspace_timed_out(ws)
