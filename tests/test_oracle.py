"""Pins for the fp64 oracle, checked against mathematics it does not share code with.

The pages print no worked numerical example for Newton-Schulz (NS), so the
oracle is pinned to what the mathematics fixes:

* P1  cubic coefficients (1.5, -0.5, 0) converge to the polar factor U V^T
      of a brute-force SVD (tiny inputs);
* P2  for any (a, b, c) NS acts on singular values only:
      O = U_s diag(phi^k(sigma / (||sigma||_2 + eps))) V_s^T with
      phi(s) = a s + b s^3 + c s^5 (SVD built here, not in the oracle);
* P3  a 1 x n (or n x 1) matrix: x_k = phi^k(r) / r * x0 with r = ||x0|| / (||x0|| + eps);
* P4  transposition invariance, and the tall orientation computed directly;
* P5  orthogonal equivariance  NS(Q X R) = Q NS(X) R;
* P6  scale invariance up to eps;
* P7  elementwise parts against hand-worked numbers;
* P8  expert slices of a slab are independent (RFC item 2).

Each `check_*` takes the callables under test, so the same checks are also run
against planted mistakes (mutants) to show every pin can fail.
"""
import math

import numpy as np
import pytest

from oracle import muon_ref as ref

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


def phi(s, a, b, c):
    return a * s + b * s ** 3 + c * s ** 5


def phi_k(s, abc, k):
    for _ in range(k):
        s = phi(s, *abc)
    return s


def svd_closed_form(u, abc, k, eps=ref.EPS):
    """O = U_s diag(phi^k(sigma / (||sigma|| + eps))) V_s^T from numpy's SVD."""
    us, sig, vt = np.linalg.svd(u, full_matrices=False)
    s0 = sig / (math.sqrt(float(np.sum(sig ** 2))) + eps)
    return (us * phi_k(s0, abc, k)) @ vt


def rand_with_spectrum(rng, m, n, sig):
    q1, _ = np.linalg.qr(rng.standard_normal((m, m)))
    q2, _ = np.linalg.qr(rng.standard_normal((n, n)))
    r = min(m, n)
    d = np.zeros((m, n))
    d[np.arange(r), np.arange(r)] = sig
    return q1 @ d @ q2.T


# ---------------------------------------------------------------- checks ----

def check_polar_cubic(ns):
    rng = np.random.default_rng(11)
    for (m, n) in [(8, 16), (16, 8), (12, 12)]:
        r = min(m, n)
        sig = np.linspace(0.2, 1.0, r)
        u = rand_with_spectrum(rng, m, n, sig)
        us, _, vt = np.linalg.svd(u, full_matrices=False)
        polar = us @ vt
        # ||sigma|| > 1 here, so normalised singular values start >= 0.2/||sigma||;
        # 60 cubic steps are far past convergence for that range.
        o = ns(u, *CUBIC, 60)
        if not np.allclose(o, polar, rtol=0, atol=1e-12):
            return False
    return True


def check_closed_form(ns):
    rng = np.random.default_rng(12)
    cases = [(4, 9, 1.0), (9, 4, 1.0), (7, 7, 1.0), (5, 30, 3e-7), (24, 64, 1e3)]
    for (m, n, mag) in cases:
        u = mag * rng.standard_normal((m, n))
        for k in (0, 1, 2, 5):
            o = ns(u, *QUINTIC, k)
            e = svd_closed_form(u, QUINTIC, k)
            if o.shape != e.shape or not np.allclose(o, e, rtol=0, atol=1e-12):
                return False
    return True


def check_rank_one_row(ns):
    rng = np.random.default_rng(13)
    for shape in [(1, 10), (10, 1), (1, 1)]:
        x0 = rng.standard_normal(shape)
        nrm = float(np.sqrt(np.sum(x0 ** 2)))
        r = nrm / (nrm + ref.EPS)
        for k in (1, 3, 5):
            e = (phi_k(r, QUINTIC, k) / nrm) * x0
            if not np.allclose(ns(x0, *QUINTIC, k), e, rtol=0, atol=1e-13):
                return False
    return True


def check_transpose(ns):
    rng = np.random.default_rng(14)
    for (m, n) in [(6, 17), (17, 6)]:
        u = rng.standard_normal((m, n))
        if not np.allclose(ns(u.T, *QUINTIC, 5), ns(u, *QUINTIC, 5).T, rtol=0, atol=1e-13):
            return False
        # the tall orientation computed directly with an M x M Gram
        x = u / (np.sqrt(np.sum(u * u)) + ref.EPS)
        for _ in range(5):
            g = x @ x.T
            x = QUINTIC[0] * x + (QUINTIC[1] * g + QUINTIC[2] * g @ g) @ x
        if not np.allclose(ns(u, *QUINTIC, 5), x, rtol=0, atol=1e-12):
            return False
    return True


def check_equivariance(ns):
    rng = np.random.default_rng(15)
    m, n = 6, 11
    u = rng.standard_normal((m, n))
    q, _ = np.linalg.qr(rng.standard_normal((m, m)))
    r, _ = np.linalg.qr(rng.standard_normal((n, n)))
    return bool(np.allclose(ns(q @ u @ r, *QUINTIC, 5), q @ ns(u, *QUINTIC, 5) @ r,
                            rtol=0, atol=1e-12))


def check_scale_invariance(ns):
    rng = np.random.default_rng(16)
    u = rng.standard_normal((5, 13))
    base = ns(u, *QUINTIC, 5)
    return bool(np.allclose(ns(1e3 * u, *QUINTIC, 5), base, rtol=0, atol=1e-6)
                and np.allclose(ns(0.25 * u, *QUINTIC, 5), base, rtol=0, atol=1e-6))


def check_elementwise(step):
    """Hand-worked 1x1 and 1x2 steps (numbers derived in the comments)."""
    hp = ref.MuonHyper(lr=0.1, mu=0.5, nesterov=True, wd=0.2, ns_steps=0, scale=2.0)
    # M = [0, 2], G = [1, 0]: M_new = 0.5*[0, 2] + [1, 0] = [1, 1];
    # U = G + 0.5*M_new = [1.5, 0.5]; ||U|| = sqrt(2.5); O = U / (sqrt(2.5) + eps);
    # W = [3, -1]: W_new = W - 0.1*(2*O + 0.2*W) = 0.98*W - 0.2*O.
    w, mm, o = step(np.array([[3.0, -1.0]]), np.array([[1.0, 0.0]]),
                    np.array([[0.0, 2.0]]), hp)
    o_e = np.array([[1.5, 0.5]]) / (math.sqrt(2.5) + ref.EPS)
    w_e = 0.98 * np.array([[3.0, -1.0]]) - 0.2 * o_e
    if not (np.allclose(mm, [[1.0, 1.0]], rtol=0, atol=1e-15)
            and np.allclose(o, o_e, rtol=0, atol=1e-15)
            and np.allclose(w, w_e, rtol=0, atol=1e-15)):
        return False
    # without Nesterov U = M_new: M = [1, 0], G = [3, 4], mu = 0.5 gives M_new = [3.5, 4] = U.
    hp2 = ref.MuonHyper(lr=0.1, mu=0.5, nesterov=False, wd=0.0, ns_steps=0, scale=1.0)
    w, mm, o = step(np.array([[0.0, 0.0]]), np.array([[3.0, 4.0]]), np.array([[1.0, 0.0]]), hp2)
    # M_new = [3.5, 4.0]; ||U|| = sqrt(12.25 + 16) = sqrt(28.25)
    nrm = math.sqrt(28.25) + ref.EPS
    if not (np.allclose(mm, [[3.5, 4.0]], atol=1e-15)
            and np.allclose(o, [[3.5 / nrm, 4.0 / nrm]], atol=1e-15)
            and np.allclose(w, [[-0.1 * 3.5 / nrm, -0.1 * 4.0 / nrm]], atol=1e-15)):
        return False
    # lr = 0 leaves W exactly unchanged
    rng = np.random.default_rng(17)
    w0 = rng.standard_normal((3, 5))
    w, _, _ = step(w0, rng.standard_normal((3, 5)), np.zeros((3, 5)),
                   ref.MuonHyper(lr=0.0))
    if not np.array_equal(w, w0):
        return False
    # mu = 0 without Nesterov: U = G, so O is NS(G)
    g = rng.standard_normal((4, 7))
    _, mm, o = step(np.zeros((4, 7)), g, rng.standard_normal((4, 7)),
                    ref.MuonHyper(mu=0.0, nesterov=False))
    return bool(np.array_equal(mm, g) and np.allclose(o, svd_closed_form(g, QUINTIC, 5),
                                                      rtol=0, atol=1e-12))


def check_slab_independence(step_many):
    rng = np.random.default_rng(18)
    e, m, n = 4, 6, 10
    w = rng.standard_normal((e, m, n))
    g = rng.standard_normal((e, m, n))
    mo = rng.standard_normal((e, m, n))
    hp = ref.MuonHyper()
    w1, m1, o1 = step_many([w], [g], [mo], hp)
    g2 = g.copy()
    g2[2] *= 50.0
    g2[2, 0, 0] += 7.0
    w2, m2, o2 = step_many([w], [g2], [mo], hp)
    others = [0, 1, 3]
    if not (np.array_equal(o1[0][others], o2[0][others])
            and np.array_equal(w1[0][others], w2[0][others])):
        return False
    # each slice equals the matrix computed alone
    for i in range(e):
        wi, mi, oi = step_many([w[i]], [g[i]], [mo[i]], hp)
        if not np.array_equal(oi[0], o1[0][i]) or not np.array_equal(wi[0], w1[0][i]):
            return False
    return True


# ---------------------------------------------------------- pins (oracle) ---

def ns_oracle(u, a, b, c, k):
    return ref.newton_schulz(u, a, b, c, k)


def test_p1_cubic_converges_to_polar_factor():
    assert check_polar_cubic(ns_oracle)


def test_p2_closed_form_any_steps():
    assert check_closed_form(ns_oracle)


def test_p3_rank_one_row():
    assert check_rank_one_row(ns_oracle)


def test_p4_transpose():
    assert check_transpose(ns_oracle)


def test_p5_orthogonal_equivariance():
    assert check_equivariance(ns_oracle)


def test_p6_scale_invariance():
    assert check_scale_invariance(ns_oracle)


def test_p7_elementwise_parts():
    assert check_elementwise(ref.muon_step_matrix)


def test_p8_slab_independence():
    assert check_slab_independence(ref.muon_step)


def test_quintic_scalar_facts():
    """phi(1) and phi'(0) for the quintic, and where phi^5 sends [1e-2, 1]."""
    a, b, c = QUINTIC
    assert abs(phi(1.0, a, b, c) - 0.7010) < 1e-12
    assert a == pytest.approx(3.4445)
    s = np.linspace(1e-2, 1.0, 20001)
    v = phi_k(s, QUINTIC, 5)
    assert 0.68 < v.min() < 0.69 and 1.13 < v.max() < 1.14


def test_ns_batch_matches_per_matrix():
    rng = np.random.default_rng(19)
    us = [rng.standard_normal((3, 4, 9)), rng.standard_normal((9, 4))]
    out = ref.ns_batch(us, *QUINTIC, 5)
    assert np.array_equal(out[0][1], ref.newton_schulz(us[0][1], *QUINTIC, 5))
    assert np.array_equal(out[1], ref.newton_schulz(us[1], *QUINTIC, 5))


# ------------------------------------------------- planted mistakes (CPU) ---

def _mutant_ns(kind):
    def ns(u, a, b, c, k, eps=ref.EPS):
        u = np.asarray(u, dtype=np.float64)
        tall = u.shape[0] > u.shape[1]
        x = u.T if tall else u
        if kind == "no_normalise":
            x = x.copy()
        elif kind == "eps_in_square":
            x = x / np.sqrt(np.sum(x * x) + eps)
        else:
            x = x / (np.sqrt(np.sum(x * x)) + eps)
        for _ in range(k):
            g = x @ x.T
            if kind == "drop_c":
                x = a * x + (b * g) @ x
            elif kind == "sign_b":
                x = a * x + (-b * g + c * g @ g) @ x
            elif kind == "wrong_operand":
                gt = x.T @ x
                x = a * x + (b * gt + c * gt @ gt) @ x
            elif kind == "a_on_poly":
                x = x + (b * g + c * g @ g) @ (a * x)
            else:
                x = a * x + (b * g + c * g @ g) @ x
        if kind == "no_transpose_back":
            return x
        return x.T.copy() if tall else x
    return ns


def _mutant_step(kind):
    def step(w, g, m, hp):
        w = np.asarray(w, np.float64)
        g = np.asarray(g, np.float64)
        m = np.asarray(m, np.float64)
        if kind == "ema_momentum":
            m_new = hp.mu * m + (1 - hp.mu) * g
        else:
            m_new = hp.mu * m + g
        if kind == "nesterov_old_m":
            u = g + hp.mu * m if hp.nesterov else m_new
        else:
            u = g + hp.mu * m_new if hp.nesterov else m_new
        o = ref.newton_schulz(u, hp.a, hp.b, hp.c, hp.ns_steps, hp.eps)
        if kind == "decay_after":
            w1 = w - hp.lr * hp.scale * o
            w_new = w1 - hp.lr * hp.wd * w1
        elif kind == "decay_unscaled":
            w_new = w - hp.lr * hp.scale * o - hp.wd * w
        else:
            w_new = w - hp.lr * (hp.scale * o + hp.wd * w)
        return w_new, m_new, o
    return step


def _mutant_step_many_global_norm(params, grads, moms, hp):
    out_w, out_m, out_o = [], [], []
    for w, g, m in zip(params, grads, moms):
        w = np.asarray(w, np.float64)
        g = np.asarray(g, np.float64)
        m = np.asarray(m, np.float64)
        m_new = hp.mu * m + g
        u = g + hp.mu * m_new
        if u.ndim == 2:
            o = ref.newton_schulz(u, hp.a, hp.b, hp.c, hp.ns_steps)
        else:  # mistake: one norm over the whole slab
            nrm = np.sqrt(np.sum(u * u)) + hp.eps
            o = np.stack([_ns_scaled(u[e] / nrm, hp) for e in range(u.shape[0])])
        out_w.append(w - hp.lr * (hp.scale * o + hp.wd * w))
        out_m.append(m_new)
        out_o.append(o)
    return out_w, out_m, out_o


def _ns_scaled(x, hp):
    for _ in range(hp.ns_steps):
        g = x @ x.T
        x = hp.a * x + (hp.b * g + hp.c * g @ g) @ x
    return x


NS_MUTANTS = ["no_normalise", "eps_in_square", "drop_c", "sign_b", "wrong_operand",
              "a_on_poly", "no_transpose_back"]


@pytest.mark.parametrize("kind", NS_MUTANTS)
def test_pins_catch_ns_mutant(kind):
    ns = _mutant_ns(kind)
    checks = [check_polar_cubic, check_closed_form, check_rank_one_row, check_transpose,
              check_equivariance, check_scale_invariance]
    caught = []
    for chk in checks:
        try:
            caught.append(not chk(ns))
        except (ValueError, IndexError):
            caught.append(True)
    assert any(caught), kind


@pytest.mark.parametrize("kind", ["ema_momentum", "nesterov_old_m", "decay_after",
                                  "decay_unscaled"])
def test_pins_catch_step_mutant(kind):
    assert not check_elementwise(_mutant_step(kind))


def test_pins_catch_slab_global_norm():
    assert not check_slab_independence(_mutant_step_many_global_norm)
