"""Pins of the AdamW oracle (oracle/adamw_ref.py), CPU only.

* Library routine: torch.optim.AdamW (float64, CPU, single-tensor path) over
  several steps agrees to rounding.  Its denominator is sqrt(v)/sqrt(1-b2^t)
  + eps, algebraically the oracle's sqrt(v_hat) + eps.
* Closed form: a constant gradient from zero moments gives m_hat = g and
  v_hat = g^2 at every step, so each step is p <- p(1 - lr wd) - lr g/(|g| + eps).
* Mutants of the closed-form check: dropping either bias correction, or
  coupling the decay into the gradient (L2 style), is caught.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import adamw_ref as A


def test_matches_torch_adamw_float64():
    rng = np.random.default_rng(3)
    p0 = rng.standard_normal(257)
    grads = [rng.standard_normal(257) * 0.1 for _ in range(5)]
    lr, b1, b2, eps, wd = 1e-2, 0.9, 0.95, 1e-8, 0.1
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    p, m, v = p0.copy(), np.zeros(257), np.zeros(257)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = A.adamw_step(p, g, m, v, lr, b1, b2, eps, wd, t)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=0, atol=1e-14)
    st = opt.state[tp]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-14, atol=1e-18)


def _closed_form(p0, g, lr, wd, eps, steps):
    p = p0.copy()
    for _ in range(steps):
        p = p * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    return p


def _run(step_fn, p0, g, steps, lr=1e-2, b1=0.9, b2=0.999, eps=1e-8, wd=0.05):
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for t in range(1, steps + 1):
        p, m, v = step_fn(p, g, m, v, lr, b1, b2, eps, wd, t)
    return p


def test_constant_gradient_closed_form():
    p0 = np.linspace(-2, 2, 11)
    g = np.array([1e-3, -2.0, 0.5, 3.0, -1e-2, 7.0, -0.25, 0.125, 1.0, -1.0, 4.0])
    got = _run(A.adamw_step, p0, g, 7)
    np.testing.assert_allclose(got, _closed_form(p0, g, 1e-2, 0.05, 1e-8, 7), rtol=0, atol=1e-13)


def _no_bc1(p, g, m, v, lr, b1, b2, eps, wd, t):
    p = p * (1 - lr * wd); m = b1 * m + (1 - b1) * g; v = b2 * v + (1 - b2) * g * g
    return p - lr * m / (np.sqrt(v / (1 - b2 ** t)) + eps), m, v


def _no_bc2(p, g, m, v, lr, b1, b2, eps, wd, t):
    p = p * (1 - lr * wd); m = b1 * m + (1 - b1) * g; v = b2 * v + (1 - b2) * g * g
    return p - lr * (m / (1 - b1 ** t)) / (np.sqrt(v) + eps), m, v


def _coupled_decay(p, g, m, v, lr, b1, b2, eps, wd, t):
    g = g + wd * p
    m = b1 * m + (1 - b1) * g; v = b2 * v + (1 - b2) * g * g
    return p - lr * (m / (1 - b1 ** t)) / (np.sqrt(v / (1 - b2 ** t)) + eps), m, v


@pytest.mark.parametrize("mutant", [_no_bc1, _no_bc2, _coupled_decay])
def test_closed_form_catches_mutants(mutant):
    p0 = np.linspace(-2, 2, 11)
    g = np.array([1e-3, -2.0, 0.5, 3.0, -1e-2, 7.0, -0.25, 0.125, 1.0, -1.0, 4.0])
    got = _run(mutant, p0, g, 7)
    assert np.max(np.abs(got - _closed_form(p0, g, 1e-2, 0.05, 1e-8, 7))) > 1e-6
