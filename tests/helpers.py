"""Shared test helpers: host copies, oracle runs and the comparison bars."""
from __future__ import annotations

import numpy as np
import torch

from oracle import muon_ref as ref

# bars for the bf16 path (O) and the fp32 path
BF16_O_RELF = 1e-2
BF16_O_MAXABS = 3e-2
F32_O_RELF = 1e-4


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def hyper(wl, **over) -> ref.MuonHyper:
    a, b, c = wl.coeffs
    kw = dict(lr=wl.lr, mu=wl.mu, nesterov=wl.nesterov, wd=wl.wd, a=a, b=b, c=c,
              ns_steps=wl.ns_steps, scale=wl.scale)
    kw.update(over)
    return ref.MuonHyper(**kw)


def relf(x: np.ndarray, ref_: np.ndarray) -> float:
    d = float(np.linalg.norm((x - ref_).ravel()))
    n = float(np.linalg.norm(ref_.ravel()))
    return d / n if n > 0 else d


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, bf16: bool, what: str = "O"):
    r = relf(o_gpu, o_ref)
    ma = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite values"
    if bf16:
        assert r <= BF16_O_RELF and ma <= BF16_O_MAXABS, f"{what}: relF {r:.3e} maxabs {ma:.3e}"
    else:
        assert r <= F32_O_RELF, f"{what}: relF {r:.3e}"
    return r, ma


def momentum_bound(b_prev: np.ndarray, m_prev_ref: np.ndarray, m_ref: np.ndarray,
                   g: np.ndarray, mu: float) -> np.ndarray:
    """Elementwise error bound of the fp32 momentum chain M <- fma(mu, M, G).

    b_k = mu*b_{k-1} + 2^-23*(|mu*M_{k-1}| + |G| + |M_k|) + |mu32 - mu|*|M_{k-1}|:
    the previous error scaled by mu, one rounding of the fused multiply-add
    (with a factor 2 of slack), and the representation error of mu in fp32.
    """
    mu32 = float(np.float32(mu))
    return (abs(mu) * b_prev + 2.0 ** -23 * (np.abs(mu * m_prev_ref) + np.abs(g) + np.abs(m_ref))
            + abs(mu32 - mu) * np.abs(m_prev_ref))


def check_m(m_gpu: np.ndarray, m_ref: np.ndarray, bound: np.ndarray, what: str = "M"):
    err = np.abs(m_gpu - m_ref)
    bad = err > bound + 1e-38
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the fp32 bound (worst " \
                          f"{float(np.max(err - bound)):.3e} over)"


def check_w(w_gpu: np.ndarray, w_ref: np.ndarray, bf16: bool, lr: float, scale: float, what: str = "W"):
    err = np.abs(w_gpu - w_ref)
    if bf16:
        bound = ulp_bf16(w_ref) + abs(lr * scale) * BF16_O_MAXABS
    else:
        bound = 1e-6 * (1.0 + np.abs(w_ref))
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert worst <= 1.0, f"{what}: error reaches {worst:.2f}x the bound"
