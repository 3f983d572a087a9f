"""GPU parity at the full sizes of the large workloads, in the launch
configuration bench.py times.

* mixed transformer set (32 layers of 4 x [4096, 4096], 2 x [14336, 4096],
  [4096, 14336]; 224 matrices, 7.8 G parameters): one muon_step over the whole
  set.  The oracle recomputes three sampled matrices whole (one of each shape,
  including a tall one that runs transposed).
* two [8192, 28672] matrices: muon_ns and muon_step on the whole pair, checked
  at stored sample positions against the fp64 oracle's output, written by
  tests/golden/make_large_golden.py from the same PCG64 inputs.
The step's O is read back with W = 0, wd = 0, lr = -1 (so W becomes O rounded
to bf16); the momentum after one step from zero is exactly G.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from newton_schulz_05_amd import MuonPlan
from newton_schulz_05_amd import workloads as WL
from oracle import muon_ref as ref
from tests.helpers import BF16_O_MAXABS, BF16_O_RELF, check_o, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "c5_ns_samples.npz")


def _say(msg):
    print(f"[large] {msg}", flush=True)


@pytest.mark.timeout(600)
def test_mixed_transformer_full_size_sampled():
    wl = WL.WORKLOADS["c4"]
    _say(f"{wl.name}: drawing {wl.n_elements() / 1e9:.2f} G parameters on the GPU")
    plan = MuonPlan(wl.shapes, wl.dtype)
    params = [torch.zeros(s, dtype=wl.dtype, device=DEV) for s in wl.shapes]
    moms = WL.make_moms(wl, DEV)
    grads = WL.make_grads(wl, 0, DEV, DEV)
    ws = plan.new_workspace(DEV)
    kw = dict(wl.hyper())
    kw.update(lr=-1.0, wd=0.0)
    plan.step(params, grads, moms, **kw, workspace=ws)
    torch.cuda.synchronize()
    _say("step done; checking momenta and three sampled matrices")
    for i in range(len(params)):
        assert torch.equal(moms[i], grads[i].float()), f"M[{i}] != G after one step from zero"
    a, b, c = wl.coeffs
    for i in (0, 4 + 7 * 31, 6 + 7 * 16):  # first attention matrix, a tall up-projection, a down-projection
        u = (1.0 + wl.mu) * host64(grads[i])  # Nesterov look-ahead from zero momentum
        o_ref = ref.newton_schulz(u, a, b, c, wl.ns_steps)
        r, ma = check_o(host64(params[i]), o_ref, True, f"step O[{i}] {tuple(wl.shapes[i])}")
        _say(f"matrix {i} {tuple(wl.shapes[i])}: relF {r:.3e} maxabs {ma:.3e}")


def _golden():
    if not os.path.exists(GOLDEN):
        pytest.skip("tests/golden/c5_ns_samples.npz not generated")
    return np.load(GOLDEN, allow_pickle=False)


def _check_samples(outs, gold, what):
    for k in range(len(outs)):
        o = outs[k]
        rows = torch.from_numpy(gold["rows"][k]).to(DEV)
        cols = torch.from_numpy(gold["cols"][k]).to(DEV)
        got = o[rows, cols].double().cpu().numpy()
        exp = gold["vals"][k]
        relf = np.linalg.norm(got - exp) / np.linalg.norm(exp)
        ma = float(np.max(np.abs(got - exp)))
        nrm = float(torch.linalg.vector_norm(o.double()))
        _say(f"{what}[{k}]: sampled relF {relf:.3e} maxabs {ma:.3e}; ||O|| {nrm:.5f} vs {gold['norms'][k]:.5f}")
        assert relf <= BF16_O_RELF and ma <= BF16_O_MAXABS
        assert abs(nrm - gold["norms"][k]) <= BF16_O_RELF * gold["norms"][k]


@pytest.mark.timeout(600)
def test_large_matrices_ns_against_stored_oracle():
    gold = _golden()
    shape = tuple(int(x) for x in gold["shape"])
    _say(f"drawing 2 x {shape} with PCG64")
    ins = [WL.numpy_normal(shape, int(sd), float(gold["std"]), torch.bfloat16).to(DEV) for sd in gold["seeds"]]
    plan = MuonPlan([shape] * len(ins), torch.bfloat16)
    outs = [torch.empty(shape, dtype=torch.float32, device=DEV) for _ in ins]
    plan.ns(ins, outs, coeffs=WL.QUINTIC, ns_steps=5)
    torch.cuda.synchronize()
    _check_samples(outs, gold, "ns O")


@pytest.mark.timeout(600)
def test_large_matrices_step_against_stored_oracle():
    """The step's NS input is U = G + mu * (mu * 0 + G) = (1 + mu) G, and NS is
    scale invariant, so the stored NS(G) is also the step's O (up to eps)."""
    gold = _golden()
    shape = tuple(int(x) for x in gold["shape"])
    grads = [WL.numpy_normal(shape, int(sd), float(gold["std"]), torch.bfloat16).to(DEV) for sd in gold["seeds"]]
    plan = MuonPlan([shape] * len(grads), torch.bfloat16)
    params = [torch.zeros(shape, dtype=torch.bfloat16, device=DEV) for _ in grads]
    moms = [torch.zeros(shape, dtype=torch.float32, device=DEV) for _ in grads]
    plan.step(params, grads, moms, lr=-1.0, mu=0.95, nesterov=True, wd=0.0, coeffs=WL.QUINTIC, ns_steps=5)
    torch.cuda.synchronize()
    for m, g in zip(moms, grads):
        assert torch.equal(m, g.float())
    _check_samples(params, gold, "step O")
