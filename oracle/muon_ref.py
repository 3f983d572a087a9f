"""Plain fp64 CPU oracle for one Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and this module imports
nothing from the product path: the two share no code.

What it computes follows the HyperParallel FSDP Muon optimizer performance RFC
(mindspore-ai/hyper-parallel):

* item 1(1): Newton-Schulz (NS) orthogonalisation is applied to the gradient
  momentum M_t and needs each matrix whole;
* item 2: for an expert slab [E, M, N] the NS iteration only involves the last
  two dimensions, so the E slices are independent of each other;
* item 3: matrices that share their trailing [M, N] shape are batched as one
  [B, M, N] tensor (batching is an execution choice; it does not change the
  result, so this oracle simply loops over matrices);
* item 6: an AdamW-style decoupled weight decay term is added to the update.

The RFC gives no formula for any of these steps.  Where it is silent this
module takes the plainest reading (each is listed with its reason in the
repository's design notes):

* momentum  M <- mu*M + G  (no dampening);
* Nesterov  U = G + mu*M_new, otherwise U = M_new;
* NS input  X0 = U / (||U||_F + eps), eps = 1e-7 added to the norm;
* one quintic NS step  A = X X^T,  X <- a X + (b A + c A^2) X,  repeated
  ns_steps times with one (a, b, c) for every step;
* tall matrices (M > N) run on U^T and the result is transposed back; in exact
  arithmetic the orientation does not change the result;
* decoupled update  W <- W - lr*(scale*O + wd*W), with W taken before the
  update.

Everything is float64.  bf16 and fp32 inputs upcast exactly.  No blocking,
fusion or reordering beyond the steps above: each NS step is three library
matrix products in the order written.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

EPS = 1e-7


@dataclass(frozen=True)
class MuonHyper:
    """Hyper-parameters of one step (all scalars)."""

    lr: float = 0.02
    mu: float = 0.95
    nesterov: bool = True
    wd: float = 0.1
    a: float = 3.4445
    b: float = -4.7750
    c: float = 2.0315
    ns_steps: int = 5
    scale: float = 1.0
    eps: float = EPS


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def momentum_update(m: np.ndarray, g: np.ndarray, mu: float) -> np.ndarray:
    """Gradient momentum M_t (RFC item 1(1)): M <- mu*M + G."""
    return mu * _f64(m) + _f64(g)


def ns_input(g: np.ndarray, m_new: np.ndarray, mu: float, nesterov: bool) -> np.ndarray:
    """Matrix handed to NS: the Nesterov look-ahead G + mu*M_new, or M_new."""
    g = _f64(g)
    m_new = _f64(m_new)
    return g + mu * m_new if nesterov else m_new.copy()


def frobenius_normalise(x: np.ndarray, eps: float = EPS) -> np.ndarray:
    """X / (||X||_F + eps): puts every singular value at or below 1."""
    x = _f64(x)
    return x / (np.sqrt(np.sum(x * x)) + eps)


def ns_quintic_step(x: np.ndarray, a: float, b: float, c: float) -> np.ndarray:
    """One NS step on a wide (rows <= cols) matrix: A = X X^T; X <- aX + (bA + cA^2)X."""
    gram = x @ x.T
    poly = b * gram + c * (gram @ gram)
    return a * x + poly @ x


def newton_schulz(u: np.ndarray, a: float, b: float, c: float, steps: int,
                  eps: float = EPS) -> np.ndarray:
    """NS orthogonalisation of one 2-D matrix (RFC item 1(1)).

    Tall inputs are transposed to wide first and the result transposed back.
    Returns a float64 array of u's shape.
    """
    u = _f64(u)
    if u.ndim != 2:
        raise ValueError("newton_schulz expects a 2-D matrix")
    tall = u.shape[0] > u.shape[1]
    x = u.T if tall else u
    x = frobenius_normalise(x, eps)
    for _ in range(steps):
        x = ns_quintic_step(x, a, b, c)
    return x.T.copy() if tall else x


def decoupled_update(w: np.ndarray, o: np.ndarray, lr: float, wd: float,
                     scale: float) -> np.ndarray:
    """AdamW-style decoupled decay plus the Muon update (RFC item 6).

    W_new = W - lr*(scale*O + wd*W), using W from before the update.
    """
    w = _f64(w)
    return w - lr * (scale * _f64(o) + wd * w)


def muon_step_matrix(w, g, m, hp: MuonHyper) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One Muon step on one 2-D parameter.  Returns (W_new, M_new, O)."""
    m_new = momentum_update(m, g, hp.mu)
    u = ns_input(g, m_new, hp.mu, hp.nesterov)
    o = newton_schulz(u, hp.a, hp.b, hp.c, hp.ns_steps, hp.eps)
    w_new = decoupled_update(w, o, hp.lr, hp.wd, hp.scale)
    return w_new, m_new, o


def muon_step(params: Sequence[np.ndarray], grads: Sequence[np.ndarray],
              moms: Sequence[np.ndarray], hp: MuonHyper
              ) -> Tuple[List[np.ndarray], List[np.ndarray], List[np.ndarray]]:
    """One Muon step over a list of parameters.

    A parameter of shape [M, N] is one matrix; a parameter of shape [E, M, N]
    (an expert slab) is E independent matrices (RFC item 2).  Returns lists of
    float64 arrays (W_new, M_new, O) with the parameters' shapes.
    """
    w_out, m_out, o_out = [], [], []
    for w, g, m in zip(params, grads, moms):
        w = _f64(w)
        g = _f64(g)
        m = _f64(m)
        if w.ndim == 2:
            wn, mn, o = muon_step_matrix(w, g, m, hp)
        elif w.ndim == 3:
            parts = [muon_step_matrix(w[e], g[e], m[e], hp) for e in range(w.shape[0])]
            wn = np.stack([p[0] for p in parts])
            mn = np.stack([p[1] for p in parts])
            o = np.stack([p[2] for p in parts])
        else:
            raise ValueError("Muon parameters are 2-D matrices or 3-D slabs")
        w_out.append(wn)
        m_out.append(mn)
        o_out.append(o)
    return w_out, m_out, o_out


def ns_batch(inputs: Sequence[np.ndarray], a: float, b: float, c: float, steps: int,
             eps: float = EPS) -> List[np.ndarray]:
    """NS alone on a list of 2-D matrices or 3-D slabs (slices independent)."""
    out = []
    for u in inputs:
        u = _f64(u)
        if u.ndim == 2:
            out.append(newton_schulz(u, a, b, c, steps, eps))
        elif u.ndim == 3:
            out.append(np.stack([newton_schulz(u[e], a, b, c, steps, eps)
                                 for e in range(u.shape[0])]))
        else:
            raise ValueError("NS inputs are 2-D matrices or 3-D slabs")
    return out
