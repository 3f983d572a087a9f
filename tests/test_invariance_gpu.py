"""Bitwise invariances of the HIP path: results depend on nothing but the
matrix itself.  Batching (RFC item 3) and expert slicing (RFC item 2) must
not change a single bit of any matrix's momentum, weight or O."""
from __future__ import annotations

import pytest
import torch

from newton_schulz_05_amd import MuonPlan
from newton_schulz_05_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _step(shapes, params, grads, dtype, steps=2):
    plan = MuonPlan(shapes, dtype)
    moms = [torch.zeros(p.shape, dtype=torch.float32, device=DEV) for p in params]
    for s in range(steps):
        plan.step(params, grads[s], moms, lr=0.02, wd=0.1)
    torch.cuda.synchronize()
    return params, moms


def _draw(shapes, dtype, seed):
    wl = WL.custom(shapes, dtype=dtype, number=seed)
    return WL.make_params(wl, DEV, "cpu"), [WL.make_grads(wl, s, DEV, "cpu") for s in range(2)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shapes", [
    [(24, 3000)] * 5,
    [(100, 300)] * 3 + [(300, 100)] * 2,
    [(130, 260)] * 4,
], ids=["skinny", "mfma_mixed_orientation", "mfma_ragged"])
def test_grouped_equals_alone(shapes, dtype):
    params, grads = _draw(shapes, dtype, 71)
    pa = [p.clone() for p in params]
    pg, mg = _step(shapes, pa, grads, dtype)
    for i, s in enumerate(shapes):
        p1 = [params[i].clone()]
        g1 = [[grads[0][i]], [grads[1][i]]]
        p1, m1 = _step([s], p1, g1, dtype)
        assert torch.equal(p1[0], pg[i]), f"W[{i}] differs when computed alone"
        assert torch.equal(m1[0], mg[i]), f"M[{i}] differs when computed alone"


def test_batch_position_and_order():
    shapes = [(48, 512)] * 4
    params, grads = _draw(shapes, torch.bfloat16, 72)
    pa, _ = _step(shapes, [p.clone() for p in params], grads, torch.bfloat16)
    perm = [2, 0, 3, 1]
    pb, _ = _step(shapes, [params[i].clone() for i in perm],
                  [[g[i] for i in perm] for g in grads], torch.bfloat16)
    for k, i in enumerate(perm):
        assert torch.equal(pb[k], pa[i])


def test_expert_slices_independent():
    """Perturbing expert j's gradient leaves every other expert bit-identical."""
    for shape in [(6, 48, 40), (4, 24, 1000)]:
        params, grads = _draw([shape], torch.bfloat16, 73)
        pa, ma = _step([shape], [params[0].clone()], grads, torch.bfloat16)
        g2 = [[g[0].clone()] for g in grads]
        g2[0][0][2].mul_(30.0)
        g2[1][0][2, 0, 0] = 5.0
        pb, mb = _step([shape], [params[0].clone()], g2, torch.bfloat16)
        others = [e for e in range(shape[0]) if e != 2]
        assert torch.equal(pa[0][others], pb[0][others])
        assert torch.equal(ma[0][others], mb[0][others])
        assert not torch.equal(pa[0][2], pb[0][2])


def test_slab_equals_separate_matrices():
    shape = (5, 64, 96)
    params, grads = _draw([shape], torch.bfloat16, 74)
    pa, ma = _step([shape], [params[0].clone()], grads, torch.bfloat16)
    sep = [tuple(shape[1:])] * shape[0]
    pb, mb = _step(sep, [params[0][e].clone() for e in range(shape[0])],
                   [[g[0][e] for e in range(shape[0])] for g in grads], torch.bfloat16)
    for e in range(shape[0]):
        assert torch.equal(pa[0][e], pb[e]) and torch.equal(ma[0][e], mb[e])


def test_run_to_run_deterministic():
    wl = WL.WORKLOADS["c3"]
    outs = []
    for _ in range(2):
        params = WL.make_params(wl, DEV, "cpu")
        moms = WL.make_moms(wl, DEV)
        plan = MuonPlan(wl.shapes, wl.dtype)
        for s in range(2):
            plan.step(params, WL.make_grads(wl, s, DEV, "cpu"), moms, **wl.hyper())
        torch.cuda.synchronize()
        outs.append([p.clone() for p in params] + [m.clone() for m in moms])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_checkpoint_resume_bitwise():
    """k steps, save W and M, one more step == the uninterrupted run."""
    wl = WL.custom([(24, 2000), (96, 160)], number=75)
    plan = MuonPlan(wl.shapes, wl.dtype)
    params = WL.make_params(wl, DEV, "cpu")
    moms = WL.make_moms(wl, DEV)
    for s in range(2):
        plan.step(params, WL.make_grads(wl, s, DEV, "cpu"), moms, **wl.hyper())
    saved = ([p.cpu().clone() for p in params], [m.cpu().clone() for m in moms])
    plan.step(params, WL.make_grads(wl, 2, DEV, "cpu"), moms, **wl.hyper())
    torch.cuda.synchronize()
    plan2 = MuonPlan(wl.shapes, wl.dtype)
    p2 = [p.to(DEV) for p in saved[0]]
    m2 = [m.to(DEV) for m in saved[1]]
    plan2.step(p2, WL.make_grads(wl, 2, DEV, "cpu"), m2, **wl.hyper())
    torch.cuda.synchronize()
    for a, b in zip(params + moms, p2 + m2):
        assert torch.equal(a, b)


def test_gemm_tile_choice_is_bitwise_neutral():
    """Eight [2048, 2304] matrices run with 256 x 256 GEMM tiles, one alone
    with 128 x 128 tiles (too few tiles to fill the chip at 256); per 16-wide
    k slice both kernels take each output's MFMA products in the same order,
    so the results must agree bit for bit.  The last matrix is tall."""
    shapes = [(2048, 2304)] * 7 + [(2304, 2048)]
    params, grads = _draw(shapes, torch.bfloat16, 75)
    pg, mg = _step(shapes, [p.clone() for p in params], grads, torch.bfloat16)
    for i in (0, 7):
        p1, m1 = _step([shapes[i]], [params[i].clone()], [[grads[0][i]], [grads[1][i]]], torch.bfloat16)
        assert torch.equal(p1[0], pg[i]), f"W[{i}] differs between the 128 and 256 tile kernels"
        assert torch.equal(m1[0], mg[i])


def test_bound_ns_equals_ns():
    shapes = [(24, 3000)] * 3 + [(96, 640)]
    wl = WL.custom(shapes, number=76)
    ins = WL.make_grads(wl, 0, DEV, "cpu")
    plan = MuonPlan(shapes, torch.bfloat16)
    o1 = [torch.empty(s, dtype=torch.float32, device=DEV) for s in shapes]
    o2 = [torch.empty(s, dtype=torch.float32, device=DEV) for s in shapes]
    plan.ns(ins, o1)
    plan.bind_ns(ins, o2).ns()
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(o1, o2))


def test_ranks_stepping_their_assigned_matrices_reproduce_the_full_step():
    """The de-duplicated split on one device: each of 3 simulated ranks steps
    only the matrices muon_plan_assign gives it (its own plan over 2-D views,
    expert slices included); together they must reproduce the single
    full-set step bit for bit."""
    shapes = [(4, 96, 160), (24, 3000), (24, 3000), (200, 96), (96, 200), (2, 24, 1000)]
    params, grads = _draw(shapes, torch.bfloat16, 77)
    full_p, full_m = _step(shapes, [p.clone() for p in params], grads, torch.bfloat16)
    plan = MuonPlan(shapes, torch.bfloat16)
    owner, _ = plan.assign(3)
    p_split = [p.clone() for p in params]
    m_split = [torch.zeros(p.shape, dtype=torch.float32, device=DEV) for p in params]
    for r in range(3):
        pv = plan.rank_views(p_split, owner, r)
        if not pv:
            continue
        mv = plan.rank_views(m_split, owner, r)
        sub = MuonPlan([tuple(v.shape) for v in pv], torch.bfloat16)
        for s in range(2):
            gv = plan.rank_views(grads[s], owner, r)
            sub.step(pv, gv, mv, lr=0.02, wd=0.1)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(p_split[i], full_p[i]), f"W[{i}]"
        assert torch.equal(m_split[i], full_m[i]), f"M[{i}]"


@pytest.mark.parametrize("shapes", [[(2048, 1536)] * 8, [(1536, 2048)] * 5, [(4096, 8192)] * 2],
                         ids=["gram_poly_split", "apply_split", "symmetric_256_split"])
def test_partial_round_at_smaller_tile_is_bitwise_neutral(shapes):
    """A grid whose last round is partial runs that round at half the tile
    size: eight transposed [2048, 1536] experts have 624 symmetric 128-tiles
    (Gram, poly) against 512 co-resident slots, five [1536, 2048] have 960
    apply tiles, and two [4096, 8192] (256-tiles, grouped NS steps) have 272
    symmetric 256-tiles against 256 slots for the Gram and every m x m
    product.  Each matrix stepped alone (no split; 128-tiles for a single
    [4096, 8192]) must give the same bits."""
    params, grads = _draw(shapes, torch.bfloat16, 78)
    pg, mg = _step(shapes, [p.clone() for p in params], grads, torch.bfloat16)
    for i in (0, len(shapes) - 1):
        p1, m1 = _step([shapes[i]], [params[i].clone()], [[grads[0][i]], [grads[1][i]]], torch.bfloat16)
        assert torch.equal(p1[0], pg[i]), f"W[{i}] differs between the split and single-matrix grids"
        assert torch.equal(m1[0], mg[i])


def test_padding_of_the_group_is_bitwise_neutral():
    """Nine [2000, 2900] matrices (the last stored tall) take 256-tiles and
    are padded to [2048, 3072]; one alone takes 128-tiles and [2048, 2944].
    The momentum kernel's sum-of-squares slots and their summation order
    follow the matrix's own 64 x 64 tiles, not the padded grid, so every bit
    of W and M must agree."""
    shapes = [(2000, 2900)] * 8 + [(2900, 2000)]
    params, grads = _draw(shapes, torch.bfloat16, 79)
    pg, mg = _step(shapes, [p.clone() for p in params], grads, torch.bfloat16)
    for i in (0, 4, 8):
        p1, m1 = _step([shapes[i]], [params[i].clone()], [[grads[0][i]], [grads[1][i]]], torch.bfloat16)
        assert torch.equal(p1[0], pg[i]), f"W[{i}] differs between the grouped (256-tile) and alone (128-tile) runs"
        assert torch.equal(m1[0], mg[i])


@pytest.mark.parametrize("shapes,picks,chunks", [
    ([(24, 1024)] * 170, (0, 56, 57, 113, 114, 169), 3),
    ([(64, 200)] * 90, (0, 44, 45, 89), 2),
], ids=["skinny_3_chunks", "mfma_2_chunks"])
def test_chunking_is_bitwise_neutral(shapes, picks, chunks):
    """A group larger than one launch's descriptor table is split into
    chunks; every matrix must come out as it does stepped alone, whichever
    chunk (first, last, either side of a boundary) holds it."""
    plan = MuonPlan(shapes, torch.bfloat16)
    assert plan.groups()[0]["n_chunks"] == chunks
    params, grads = _draw(shapes, torch.bfloat16, 80)
    pg, mg = _step(shapes, [p.clone() for p in params], grads, torch.bfloat16)
    for i in picks:
        p1, m1 = _step([shapes[i]], [params[i].clone()], [[grads[0][i]], [grads[1][i]]], torch.bfloat16)
        assert torch.equal(p1[0], pg[i]), f"W[{i}] differs between the chunked group and alone"
        assert torch.equal(m1[0], mg[i])
