"""Whole-matrix work split over ranks (muon_plan_assign): the greedy,
load-balancing assignment of items 1(3) and 4 of the HyperParallel FSDP Muon
optimizer RFC.  Host only; no GPU.

Pins that do not restate the implementation: the owners partition the
matrices; each rank's reported cost is the sum of its matrices' costs; on
tiny instances the largest load stays within Graham's bound for
largest-first greedy, (4/3 - 1/(3R)) times the optimum found by brute force;
equal matrices go round-robin; the mixed transformer set splits exactly
evenly over 8 ranks; two processes compute the same split."""
from __future__ import annotations

import itertools
import os
import random
import socket

import pytest
import torch

from newton_schulz_05_amd import MuonError, MuonPlan
from newton_schulz_05_amd import workloads as WL


def ns_cost(shape):
    m, n = min(shape[-2:]), max(shape[-2:])
    return 3.0 * m * m * n + float(m) ** 3


def matrix_costs(shapes):
    out = []
    for s in shapes:
        b = s[0] if len(s) == 3 else 1
        out += [ns_cost(s)] * b
    return out


def test_partition_and_reported_costs():
    shapes = [(4096, 4096)] * 3 + [(14336, 4096), (4096, 14336), (6, 64, 48), (24, 10240)]
    plan = MuonPlan(shapes)
    assert plan.num_matrices() == 3 + 2 + 6 + 1
    assert plan.matrices()[5:11] == [(5, e) for e in range(6)]
    owner, cost = plan.assign(3)
    c = matrix_costs(shapes)
    assert len(owner) == len(c) and set(owner) <= {0, 1, 2}
    for r in range(3):
        tot = sum(ci for ci, o in zip(c, owner) if o == r)
        assert abs(tot - cost[r]) <= 1e-12 * max(tot, 1.0)


def test_one_rank_and_more_ranks_than_matrices():
    plan = MuonPlan([(64, 128), (32, 32), (128, 512)])
    owner, cost = plan.assign(1)
    assert owner == [0, 0, 0]
    owner, cost = plan.assign(5)
    # heaviest first, each to the emptiest rank (lowest on ties)
    assert owner == [1, 2, 0]
    assert cost[3] == 0.0 and cost[4] == 0.0


def test_equal_matrices_round_robin_in_plan_order():
    plan = MuonPlan([(48, 512)] * 7)
    owner, _ = plan.assign(3)
    assert owner == [0, 1, 2, 0, 1, 2, 0]


@pytest.mark.parametrize("seed", range(6))
def test_makespan_within_lpt_bound_of_optimum(seed):
    rng = random.Random(seed)
    shapes = [(rng.choice([16, 32, 48, 64, 96]), rng.choice([64, 128, 256, 512])) for _ in range(rng.randint(4, 8))]
    c = matrix_costs(shapes)
    for R in (2, 3):
        owner, cost = MuonPlan(shapes).assign(R)
        best = min(max(sum(ci for ci, a in zip(c, asg) if a == r) for r in range(R))
                   for asg in itertools.product(range(R), repeat=len(c)))
        assert max(cost) >= best * (1 - 1e-12)
        assert max(cost) <= (4.0 / 3.0 - 1.0 / (3 * R)) * best * (1 + 1e-12)


def test_mixed_transformer_set_splits_evenly():
    wl = WL.WORKLOADS["c4"]
    owner, cost = MuonPlan(wl.shapes).assign(8)
    assert max(cost) == min(cost)
    assert [owner.count(r) for r in range(8)] == [28] * 8


def test_bad_arguments():
    plan = MuonPlan([(64, 128)])
    with pytest.raises(MuonError):
        plan.assign(0)
    from newton_schulz_05_amd import binding as B
    import ctypes
    owner = (ctypes.c_int32 * 4)()
    assert B.load_library().muon_plan_assign(plan._h, 2, owner, 3, None) == 1  # n_owner != matrices


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _rank_main(rank, world, port, out_dir):
    import torch.distributed as dist
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    try:
        wl = WL.WORKLOADS["c4"]
        owner, _ = MuonPlan(wl.shapes).assign(world)
        mine = torch.tensor([j for j, o in enumerate(owner) if o == rank], dtype=torch.int64)
        own_t = torch.tensor(owner, dtype=torch.int32)
        all_own = [torch.empty_like(own_t) for _ in range(world)]
        dist.all_gather(all_own, own_t)
        sizes = [torch.zeros(1, dtype=torch.int64) for _ in range(world)]
        dist.all_gather(sizes, torch.tensor([mine.numel()], dtype=torch.int64))
        ok = all(torch.equal(a, own_t) for a in all_own) and int(sum(s.item() for s in sizes)) == len(owner)
        with open(os.path.join(out_dir, f"rank{rank}"), "w") as f:
            f.write("ok" if ok else "mismatch")
    finally:
        dist.destroy_process_group()


def test_two_gloo_ranks_compute_the_same_split(tmp_path):
    import torch.multiprocessing as mp
    mp.spawn(_rank_main, args=(2, _free_port(), str(tmp_path)), nprocs=2, join=True)
    for r in range(2):
        assert (tmp_path / f"rank{r}").read_text() == "ok"


def test_rank_views_cover_each_matrix_once():
    shapes = [(64, 128), (3, 32, 48), (100, 40)]
    plan = MuonPlan(shapes)
    ts = [torch.zeros(s) for s in shapes]
    owner, _ = plan.assign(2)
    views = [plan.rank_views(ts, owner, r) for r in range(2)]
    assert sum(len(v) for v in views) == plan.num_matrices()
    for v in views[0] + views[1]:
        v.add_(1.0)
    assert all(bool((t == 1.0).all()) for t in ts)
