"""Seeded synthetic workloads (shapes, value laws, hyper-parameters).

This module only draws inputs; it holds none of the Muon arithmetic.  Tests
and the benchmark hand the same tensors to the HIP path and (as float64 host
copies) to the CPU oracle, so neither side re-implements the other's RNG.

The shapes follow the pages: 74 parameters of [24, 10240] batched as one
[74, 24, 10240] tensor and a [32, 24, 10240] slab (HyperParallel FSDP Muon
optimizer RFC, item 3), one rank's share of an expert slab [E/shard, M, N]
(item 2), plus a dense transformer set and two large FFN matrices.
Weights ~ N(0, 1); gradients ~ N(0, std^2) with the stated std; momenta
start at zero.  Seeds: W of parameter i is drawn with 1000*k + i (k = the
workload number), the gradients of step s with 1000*k + i + 100003*(s + 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

QUINTIC = (3.4445, -4.7750, 2.0315)


@dataclass(frozen=True)
class Workload:
    key: str
    number: int
    name: str
    shapes: Tuple[Tuple[int, ...], ...]
    dtype: torch.dtype
    g_std: float
    w_std: float = 1.0
    lr: float = 0.02
    mu: float = 0.95
    nesterov: bool = True
    wd: float = 0.1
    coeffs: Tuple[float, float, float] = QUINTIC
    ns_steps: int = 5
    scale: float = 1.0

    def hyper(self) -> dict:
        return dict(lr=self.lr, mu=self.mu, nesterov=self.nesterov, wd=self.wd,
                    coeffs=self.coeffs, ns_steps=self.ns_steps, scale=self.scale)

    def n_matrices(self) -> int:
        return sum(s[0] if len(s) == 3 else 1 for s in self.shapes)

    def n_elements(self) -> int:
        tot = 0
        for s in self.shapes:
            e = 1
            for d in s:
                e *= d
            tot += e
        return tot


def _c4_shapes():
    layer = [(4096, 4096)] * 4 + [(14336, 4096)] * 2 + [(4096, 14336)]
    return tuple(layer * 32)


WORKLOADS = {
    "c1": Workload("c1", 1, "tiny_fp32_4x64x128", ((64, 128),) * 4, torch.float32, g_std=1.0),
    "c2": Workload("c2", 2, "skinny_74x24x10240", ((24, 10240),) * 74, torch.bfloat16, g_std=1e-2),
    "c3": Workload("c3", 3, "moe_slab_8x2048x1536_plus_32x24x10240",
                   ((8, 2048, 1536), (32, 24, 10240)), torch.bfloat16, g_std=1e-3),
    "c4": Workload("c4", 4, "mixed_32_layers_4096_14336", _c4_shapes(), torch.bfloat16, g_std=1e-3),
    "c5": Workload("c5", 5, "large_2x8192x28672", ((8192, 28672),) * 2, torch.bfloat16, g_std=1e-3),
}


def custom(shapes: Sequence[Sequence[int]], dtype=torch.bfloat16, g_std=1e-2, number=90, **kw) -> Workload:
    """A workload with arbitrary shapes (tests of ragged and edge cases)."""
    return Workload("custom", number, "custom", tuple(tuple(s) for s in shapes), dtype, g_std=g_std, **kw)


def _randn(shape, seed: int, std: float, dtype: torch.dtype, device, gen_device) -> torch.Tensor:
    gd = torch.device(gen_device if gen_device is not None else device)
    g = torch.Generator(device=gd)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=gd, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype=dtype).to(device)


def make_params(wl: Workload, device, gen_device=None) -> List[torch.Tensor]:
    return [_randn(s, 1000 * wl.number + i, wl.w_std, wl.dtype, device, gen_device)
            for i, s in enumerate(wl.shapes)]


def make_grads(wl: Workload, step: int, device, gen_device=None) -> List[torch.Tensor]:
    return [_randn(s, 1000 * wl.number + i + 100003 * (step + 1), wl.g_std, wl.dtype, device, gen_device)
            for i, s in enumerate(wl.shapes)]


def make_moms(wl: Workload, device) -> List[torch.Tensor]:
    return [torch.zeros(tuple(s), dtype=torch.float32, device=device) for s in wl.shapes]


def numpy_normal(shape, seed: int, std: float, dtype: torch.dtype) -> torch.Tensor:
    """Host-side draw with NumPy's PCG64 generator (integer arithmetic, so the
    values are the same on every machine), rounded to `dtype`.  Used where a
    stored expected value must be reproduced on another host."""
    import numpy as np

    rng = np.random.Generator(np.random.PCG64(int(seed)))
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(dtype)


def spectral(rows: int, cols: int, kind: str, seed: int, peak: float = 0.05,
             dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """A seeded [rows, cols] matrix with a prescribed singular-value
    spectrum, drawn on the host with NumPy's PCG64 generator and rounded to
    `dtype`, scaled so that its largest entry is `peak`.  With m = min and
    n = max of the dimensions:
      'logD'  : Q1 diag(s) Q2^T with s_i = 10^(-D i / (m - 1)), i = 0 .. m-1
                (singular values log-spaced over [10^-D, 1]), Q1 [m, m] and
                Q2 [n, m] orthonormal from QR of Gaussian matrices;
      'rankK' : the product of Gaussian [m, r] and [r, n] matrices with
                r = max(1, m // K) (rank m / K before the rounding to dtype).
    Stands in for a momentum whose spectrum spreads over decades."""
    import numpy as np

    m, n = min(rows, cols), max(rows, cols)
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    if kind.startswith("log"):
        d = float(kind[3:])
        q1, _ = np.linalg.qr(rng.standard_normal((m, m)))
        q2, _ = np.linalg.qr(rng.standard_normal((n, m)))
        z = (q1 * np.logspace(-d, 0.0, m)) @ q2.T
    elif kind.startswith("rank"):
        r = max(1, m // int(kind[4:]))
        z = rng.standard_normal((m, r)) @ rng.standard_normal((r, n))
    else:
        raise ValueError(f"unknown spectrum kind {kind!r}")
    z *= peak / np.max(np.abs(z))
    if rows > cols:
        z = z.T
    return torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)).to(dtype)
