"""CPU checks of the work counts bench.py reports.

`executed_flops` mirrors the library's NS schedule for the bf16 path (which
steps take the split A^2, which steps are grouped); on the two [8192, 28672]
matrices its figure matched the bf16 MFMA operation counters of a rocprofv3
run launch by launch.  Here it is pinned to closed forms written out by hand
for that workload and for the schedule's other branches."""
from __future__ import annotations

import pytest
import torch

import bench
from newton_schulz_05_amd import workloads as WL


def _wl(shapes, ns_steps=5, dtype=torch.bfloat16):
    return WL.custom(shapes, dtype=dtype, ns_steps=ns_steps)


def test_algorithmic_count_is_3m2n_plus_m3_per_step():
    m, n = 24, 10240
    assert bench.alg_flops(WL.WORKLOADS["c2"]) == 74 * 5 * (3 * m * m * n + m ** 3)
    assert bench.alg_flops(_wl([(300, 100)], ns_steps=2)) == 2 * (3 * 100 ** 2 * 300 + 100 ** 3)


def test_executed_count_grouped_steps_on_the_large_pair():
    # lean recipe (m >= 4096), 5 steps as a group of 4 and a single step.
    # Group: Gram m^2 n, A^2 in steps 0-2 as one product and in step 3 as
    # three, T, A' and R for steps 1-3, apply with X_0's lo plane 2 x 2 m^2 n.
    # Last step: Gram, split A^2, apply.
    m, n = 8192, 28672
    group = m * m * n + (1 + 1 + 1 + 3) * m ** 3 + 3 * 3 * m ** 3 + 2 * 2 * m * m * n
    single = 3 * m * m * n + 3 * m ** 3
    assert bench.executed_flops(WL.WORKLOADS["c5"]) == 2 * (group + single)


@pytest.mark.parametrize("ns_steps,groups", [(1, [1]), (2, [2]), (3, [2, 1]), (4, [3, 1]),
                                             (6, [4, 2]), (7, [4, 2, 1])])
def test_executed_count_group_lengths(ns_steps, groups):
    # precise recipe (512 <= m < 4096): first Gram with X_0's lo plane (3
    # products), chain products split (3 each), applies with R's lo plane and,
    # in the first group, X_0's; below m = 1536 A^2 is a single product in
    # steps 0-1 only
    m, n = 600, 1300
    split = [k >= min(2, ns_steps - 2) for k in range(ns_steps)]
    want, k = 0, 0
    for g in groups:
        gram = (3 if k == 0 else 1) * m * m * n
        apply = (3 if k == 0 else 2) * 2 * m * m * n
        want += gram + sum((3 if split[k + j] else 1) * m ** 3 for j in range(g)) + 9 * (g - 1) * m ** 3 + apply
        k += g
    assert bench.executed_flops(_wl([(m, n)], ns_steps)) == want


@pytest.mark.parametrize("ns_steps,rprod", [(5, 1), (6, 3)])
def test_executed_count_precise_r_single_from_1024(ns_steps, rprod):
    # precise recipe at m = 1536 (the experts): T and A' split, R a single
    # product up to 5 steps (three beyond); 5 steps as 4 + 1, 6 as 4 + 2
    m, n = 1536, 2048
    split = [k >= min(3, ns_steps - 2) for k in range(ns_steps)]
    groups = [4, 1] if ns_steps == 5 else [4, 2]
    want, k = 0, 0
    for g in groups:
        gram = (3 if k == 0 else 1) * m * m * n
        apply = (3 if k == 0 else 2) * 2 * m * m * n
        want += gram + sum((3 if split[k + j] else 1) * m ** 3 for j in range(g)) + (6 + rprod) * (g - 1) * m ** 3 + apply
        k += g
    assert bench.executed_flops(_wl([(n, m)], ns_steps)) == want


def test_executed_count_whole_group_below_512():
    # m < 512: all 5 steps in one group, split A^2 everywhere, split chain,
    # first Gram and the one apply with both lo planes
    m, n = 300, 700
    want = 3 * m * m * n + 5 * 3 * m ** 3 + 9 * 4 * m ** 3 + 3 * 2 * m * m * n
    assert bench.executed_flops(_wl([(n, m)])) == want
