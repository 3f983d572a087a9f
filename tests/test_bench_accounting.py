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
    # 5 steps as a group of 4 and a single step.  Group: Gram m^2 n, A^2 in
    # steps 0-2 as one product and in step 3 as three, T, A' and R for steps
    # 1-3, apply 2 m^2 n.  Last step: Gram, split A^2, apply.
    m, n = 8192, 28672
    group = 3 * m * m * n + (1 + 1 + 1 + 3) * m ** 3 + 3 * 3 * m ** 3
    single = 3 * m * m * n + 3 * m ** 3
    assert bench.executed_flops(WL.WORKLOADS["c5"]) == 2 * (group + single)
    assert abs(bench.executed_flops(WL.WORKLOADS["c5"]) / 1e12 - 42.881) < 1e-3


@pytest.mark.parametrize("ns_steps,groups", [(1, [1]), (2, [2]), (3, [2, 1]), (4, [3, 1]),
                                             (6, [4, 2]), (7, [4, 2, 1])])
def test_executed_count_group_lengths(ns_steps, groups):
    m, n = 600, 1300  # grouped: m >= 512, n >= 2 m
    split = [k >= min(3, ns_steps - 2) for k in range(ns_steps)]
    want, k = 0, 0
    for g in groups:
        want += 3 * m * m * n + sum((3 if split[k + j] else 1) * m ** 3 for j in range(g)) + 3 * (g - 1) * m ** 3
        k += g
    assert bench.executed_flops(_wl([(m, n)], ns_steps)) == want


def test_executed_count_single_steps():
    # square (not grouped, single-product A^2 in steps 0-2) and m < 512 (split
    # in every step)
    m = 512
    want = 5 * 3 * m ** 3 + (1 + 1 + 1 + 3 + 3) * m ** 3
    assert bench.executed_flops(_wl([(m, m)])) == want
    m, n = 300, 700
    assert bench.executed_flops(_wl([(n, m)])) == 5 * (3 * m * m * n + 3 * m ** 3)
