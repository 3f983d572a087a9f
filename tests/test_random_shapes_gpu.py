"""Seeded random parameter sets against the fp64 oracle (two steps, the
step's own O, and muon_ns).  Each set mixes shapes that exercise different
kernels and edge cases: skinny (m <= 32; KS 6 and 8), MFMA groups with both
GEMM tiles, single and grouped NS steps at m >= 512, tall members, expert
slabs and ragged sizes.  The shapes come from
a fixed seed, so every run checks the same sets."""
from __future__ import annotations

import random

import pytest
import torch

from newton_schulz_05_amd import workloads as WL
from tests.test_parity_gpu import ns_and_compare, run_and_compare

pytestmark = pytest.mark.gpu


def _random_set(seed):
    rng = random.Random(seed)
    shapes = []
    for _ in range(rng.randint(2, 5)):
        kind = rng.choice(["skinny", "skinny", "mfma", "mfma", "slab"])
        if kind == "skinny":
            m, n = rng.randint(1, 32), rng.randint(33, 4000)
        elif kind == "mfma":
            m, n = rng.randint(33, 400), rng.randint(33, 1200)
        else:
            e, m, n = rng.randint(2, 5), rng.randint(8, 120), rng.randint(16, 300)
            shapes.append((e, m, n) if rng.random() < 0.5 else (e, n, m))
            continue
        shapes.append((m, n) if rng.random() < 0.6 else (n, m))
    return shapes


def _random_large_set(seed):
    """m in [512, 1100] and n in [m, 3m]: grouped steps (4 + 1) of the precise
    recipe, with the single-product A^2 of the first steps (two below
    m = 1536)."""
    rng = random.Random(seed)
    shapes = []
    for _ in range(rng.randint(1, 3)):
        m = rng.randint(512, 1100)
        n = rng.randint(m, 3 * m)
        shapes.append((m, n) if rng.random() < 0.6 else (n, m))
    return shapes


@pytest.mark.parametrize("seed", range(6))
def test_random_bf16_sets(seed):
    shapes = _random_set(seed)
    print(f"[random] seed {seed}: {shapes}", flush=True)
    wl = WL.custom(shapes, dtype=torch.bfloat16, g_std=1e-2, number=200 + seed)
    run_and_compare(wl, steps=2)
    ns_and_compare(wl)


@pytest.mark.parametrize("seed", range(3))
def test_random_large_bf16_sets(seed):
    shapes = _random_large_set(400 + seed)
    print(f"[random] large seed {seed}: {shapes}", flush=True)
    wl = WL.custom(shapes, dtype=torch.bfloat16, g_std=1e-3, number=400 + seed)
    run_and_compare(wl, steps=2)
    ns_and_compare(wl)


@pytest.mark.parametrize("seed", range(2))
def test_random_f32_sets(seed):
    shapes = _random_set(100 + seed)
    print(f"[random] f32 seed {seed}: {shapes}", flush=True)
    wl = WL.custom(shapes, dtype=torch.float32, g_std=1.0, number=300 + seed)
    run_and_compare(wl, steps=2)
    ns_and_compare(wl)


def test_large_group_uses_both_tiles():
    """A group big enough for 256-wide GEMM tiles next to a small one on
    128-wide tiles, in one step."""
    shapes = [(2048, 2304)] * 8 + [(300, 700)] * 2
    print(f"[random] tiles: {shapes}", flush=True)
    wl = WL.custom(shapes, dtype=torch.bfloat16, g_std=1e-2, number=310)
    run_and_compare(wl, steps=1)
