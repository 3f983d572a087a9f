"""GPU parity of muon_shard_update, the per-rank slice update after NS of a
gathered momentum (item 1(1) of the HyperParallel FSDP Muon optimizer RFC),
against the oracle's decoupled update (its item 6) on the same slice."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from newton_schulz_05_amd import MuonPlan, shard_update
from newton_schulz_05_amd import workloads as WL
from oracle import muon_ref as ref
from tests.helpers import check_w, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _draw(shape, dtype, seed):
    w = WL.numpy_normal(shape, seed, 1.0, dtype).to(DEV)
    o = WL.numpy_normal(shape, seed + 1, 0.05, torch.float32).to(DEV)
    return w, o


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_ragged_shards_match_oracle(dtype):
    shape = (300, 701)
    w, o = _draw(shape, dtype, 501)
    w_ref = ref.decoupled_update(host64(w), host64(o), 0.02, 0.1, 1.5)
    flat = w.view(-1)
    cuts = [0, 1, 4097, 100000, 150001, flat.numel()]
    for a, b in zip(cuts[:-1], cuts[1:]):
        shard_update(flat[a:b], o, a, lr=0.02, wd=0.1, scale=1.5)
    torch.cuda.synchronize()
    check_w(host64(w), w_ref, dtype == torch.bfloat16, 0.02, 1.5)


def test_shards_equal_one_whole_update():
    w, o = _draw((257, 1000), torch.bfloat16, 502)
    w1 = w.clone()
    shard_update(w1.view(-1), o, 0, lr=0.02, wd=0.1)
    w2 = w.clone()
    f = w2.view(-1)
    step = 12345
    for a in range(0, f.numel(), step):
        shard_update(f[a:a + step], o, a, lr=0.02, wd=0.1)
    torch.cuda.synchronize()
    assert torch.equal(w1, w2)


def test_sharded_flow_on_one_gpu():
    """The AllGather design end to end on one device: full momentum -> NS of
    U (muon_ns) -> each of 4 'ranks' updates its flat quarter of W.  Checked
    against the oracle's step on the same matrix."""
    shape = (96, 640)
    wl = WL.custom([shape], g_std=1e-2, number=77)
    w = WL.make_params(wl, DEV, "cpu")[0]
    g = WL.make_grads(wl, 0, DEV, "cpu")[0]
    m = torch.zeros(shape, dtype=torch.float32, device=DEV)
    hp = ref.MuonHyper(lr=0.02, mu=0.95, nesterov=True, wd=0.1, a=3.4445, b=-4.7750, c=2.0315,
                       ns_steps=5, scale=1.0)
    w_ref, _, _ = ref.muon_step_matrix(host64(w), host64(g), np.zeros(shape), hp)
    # momentum from zero: M = G, U = G + mu M = (1 + mu) G (elementwise, per shard in the real flow)
    u = (g.float() * (1.0 + hp.mu)).to(torch.bfloat16)
    plan = MuonPlan([shape], torch.bfloat16)
    o = torch.empty(shape, dtype=torch.float32, device=DEV)
    plan.ns([u], [o], coeffs=(hp.a, hp.b, hp.c), ns_steps=hp.ns_steps)
    flat = w.view(-1)
    q = flat.numel() // 4
    for r in range(4):
        a, b = r * q, (flat.numel() if r == 3 else (r + 1) * q)
        shard_update(flat[a:b], o, a, lr=hp.lr, wd=hp.wd, scale=hp.scale)
    torch.cuda.synchronize()
    check_w(host64(w), w_ref, True, hp.lr, hp.scale)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_vector_and_element_paths_agree(dtype):
    """A 16-byte aligned shard takes the vector path, an odd offset the
    element path; both must give the same bits."""
    w, o = _draw((64, 1000), dtype, 503)
    flat = w.view(-1)
    a = w.clone().view(-1)
    shard_update(a[8:8 + 40000], o, 8, lr=0.02, wd=0.1)          # aligned shard, aligned O
    b = w.clone().view(-1)
    for lo, hi in ((8, 9), (9, 40008)):                             # element path (odd start)
        shard_update(b[lo:hi], o, lo, lr=0.02, wd=0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, flat)
