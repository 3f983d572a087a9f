"""GPU parity of muon_adamw_step (AdamW on a list of 1-D parameters) with
the fp64 oracle (oracle/adamw_ref.py), over three steps, on ragged sizes that
straddle the per-workgroup chunk and more tensors than one launch takes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from newton_schulz_05_amd import adamw_step
from newton_schulz_05_amd import workloads as WL
from oracle import adamw_ref as A
from tests.helpers import host64, ulp_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"
HP = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)


def _bound_moment(ref_prev, g, ref_new, b):
    # one fp32 FMA of b*x + (1-b)*y plus the rounding of (1-b)*y, chained over steps
    return 2.0 ** -22 * (np.abs(b * ref_prev) + np.abs(g) + np.abs(ref_new)) + 1e-30


def _run(sizes, dtype, seed, steps=3):
    ps = [WL.numpy_normal((n,), seed + i, 1.0, dtype).to(DEV) for i, n in enumerate(sizes)]
    ms = [torch.zeros(n, dtype=torch.float32, device=DEV) for n in sizes]
    vs = [torch.zeros(n, dtype=torch.float32, device=DEV) for n in sizes]
    ref = [(host64(p), np.zeros(n), np.zeros(n)) for p, n in zip(ps, sizes)]
    errs = {"p": 0.0, "m": 0.0, "v": 0.0}
    for t in range(1, steps + 1):
        gs = [WL.numpy_normal((n,), 7919 * t + seed + i, 0.01, dtype).to(DEV) for i, n in enumerate(sizes)]
        adamw_step(ps, gs, ms, vs, lr=HP["lr"], betas=(HP["b1"], HP["b2"]), eps=HP["eps"], wd=HP["wd"], step=t)
        torch.cuda.synchronize()
        for i, n in enumerate(sizes):
            p_prev, m_prev, v_prev = ref[i]
            g = host64(gs[i])
            p_ref, m_ref, v_ref = A.adamw_step(p_prev, g, m_prev, v_prev, HP["lr"], HP["b1"], HP["b2"],
                                               HP["eps"], HP["wd"], t)
            mg, vg, pg = host64(ms[i]), host64(vs[i]), host64(ps[i])
            assert np.all(np.isfinite(pg))
            # moments: fp32 rounding only (checked against a bound that accumulates over steps)
            mb = _bound_moment(m_prev, (1 - HP["b1"]) * g, m_ref, HP["b1"]) * t
            vb = _bound_moment(v_prev, (1 - HP["b2"]) * g * g, v_ref, HP["b2"]) * t
            errs["m"] = max(errs["m"], float(np.max(np.abs(mg - m_ref) / mb)) if n else 0.0)
            errs["v"] = max(errs["v"], float(np.max(np.abs(vg - v_ref) / vb)) if n else 0.0)
            # parameter: one rounding to the storage type plus fp32 arithmetic on the step
            step_mag = HP["lr"] * np.abs(m_ref / (1 - HP["b1"] ** t)) / (np.sqrt(v_ref / (1 - HP["b2"] ** t)) + HP["eps"])
            if dtype == torch.bfloat16:
                pb = ulp_bf16(p_ref) + 1e-5 * step_mag + 1e-30
            else:
                pb = 4e-7 * np.abs(p_ref) + 1e-5 * step_mag + 1e-30
            errs["p"] = max(errs["p"], float(np.max(np.abs(pg - p_ref) / pb)) if n else 0.0)
            # continue the oracle from the GPU state (rounded p), so errors do not compound
            ref[i] = (pg, mg, vg)
    return errs


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_ragged_sizes_match_oracle(dtype):
    sizes = [1, 2047, 2048, 2049, 4096, 0, 100003, 33]
    errs = _run(sizes, dtype, 900)
    assert errs["m"] <= 1.0 and errs["v"] <= 1.0 and errs["p"] <= 1.0, errs


def test_more_tensors_than_one_launch():
    sizes = [4096] * 65 + [17] * 5   # the 1-D gains of a 32-layer model plus a few biases
    errs = _run(sizes, torch.bfloat16, 1200, steps=2)
    assert errs["m"] <= 1.0 and errs["v"] <= 1.0 and errs["p"] <= 1.0, errs


def test_zero_gradient_only_decays():
    p = torch.linspace(-1, 1, 5000, device=DEV)
    p0 = p.clone()
    g = torch.zeros_like(p)
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    adamw_step([p], [g], [m], [v], lr=1e-2, wd=0.5, step=1)
    torch.cuda.synchronize()
    assert torch.equal(m, torch.zeros_like(m)) and torch.equal(v, torch.zeros_like(v))
    assert torch.allclose(p, p0 * (1 - 1e-2 * 0.5), rtol=1e-7, atol=0)


def test_vector_and_element_paths_agree():
    """Whole chunks of 16-byte aligned tensors take the vector path; the
    same data viewed two elements in (4-byte but not 8-byte aligned) take
    the element path: the bits must agree."""
    n = 3 * 2048 + 5
    base = WL.numpy_normal((n + 2,), 1300, 1.0, torch.bfloat16).to(DEV)
    g = WL.numpy_normal((n + 2,), 1301, 0.01, torch.bfloat16).to(DEV)
    sl = slice(2, 2 + n)
    p1, m1, v1 = base.clone(), torch.zeros(n + 2, device=DEV), torch.zeros(n + 2, device=DEV)
    p0, m0, v0 = base[sl].clone(), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    g0 = g[sl].clone()
    for t in (1, 2):
        adamw_step([p1[sl]], [g[sl]], [m1[sl]], [v1[sl]], lr=1e-3, betas=(0.9, 0.95), wd=0.1, step=t)
        adamw_step([p0], [g0], [m0], [v0], lr=1e-3, betas=(0.9, 0.95), wd=0.1, step=t)
    torch.cuda.synchronize()
    assert torch.equal(p0, p1[sl]) and torch.equal(m0, m1[sl]) and torch.equal(v0, v1[sl])
    assert not torch.equal(p0, base[sl])
