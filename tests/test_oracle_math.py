"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests retypes the oracle's own formula: each compares it with an
independent route (an SVD closed form, a scalar recursion, a library polar
decomposition, an invariance, a literal evaluation of the page's equation, or a
closed form of the momentum / update recurrences).  Each is chosen so that a
plausible slip in the oracle (a dropped or sign-flipped term, a wrong operand
order or transpose, a misplaced eps, a wrong step order) fails at least one.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import (decay_update, momentum_update, muon_step, newton_schulz,
                    newton_schulz_batched, validate_ndim)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
Q5 = (3.4445, -4.7750, 2.0315)   # quintic coefficients (a, b, c)
CUBIC = (1.5, -0.5, 0.0)
EPS = 1e-7


def p_scalar(s, a, b, c):
    return a * s + b * s ** 3 + c * s ** 5


def ns_by_svd(G, a, b, c, steps, eps):
    """Closed form: NS acts on each singular value through the scalar polynomial."""
    U, S, Vt = np.linalg.svd(np.asarray(G, dtype=np.float64), full_matrices=False)
    s = S / (np.sqrt(np.sum(S ** 2)) + eps)
    for _ in range(steps):
        s = p_scalar(s, a, b, c)
    return (U * s[None, :]) @ Vt


def rel(x, y):
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


def haar_q(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))[None, :]


@pytest.mark.parametrize("shape", [(4, 4), (7, 13), (13, 7), (64, 32), (32, 64), (1, 9), (9, 1)])
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_ns_matches_svd_closed_form(shape, steps):
    rng = np.random.default_rng([7, shape[0], shape[1], steps])
    G = rng.standard_normal(shape)
    O = newton_schulz(G, *Q5, steps, EPS)
    assert rel(O, ns_by_svd(G, *Q5, steps, EPS)) < 1e-12


def test_ns_batched_matches_svd_per_slice():
    rng = np.random.default_rng(11)
    G = rng.standard_normal((3, 8, 16))
    O = newton_schulz_batched(G, *Q5, 5, EPS)
    for i in range(3):
        assert rel(O[i], ns_by_svd(G[i], *Q5, 5, EPS)) < 1e-12
    # the norm is per slice: scaling one slice leaves the others unchanged
    G2 = G.copy()
    G2[1] *= 1e3
    O2 = newton_schulz_batched(G2, *Q5, 5, EPS)
    assert rel(O2[0], O[0]) < 1e-14 and rel(O2[2], O[2]) < 1e-14


def literal_page_form(G, a, b, c, steps, eps):
    """The architecture page's NS equation evaluated literally, with XᵀX, no orientation."""
    X = np.asarray(G, dtype=np.float64)
    X = X / (np.sqrt(np.sum(X * X)) + eps)
    for _ in range(steps):
        XtX = X.T @ X
        X = a * X + b * (X @ X.T @ X) + c * (X @ XtX @ XtX)
    return X


@pytest.mark.parametrize("shape", [(6, 10), (10, 6), (8, 8)])
def test_ns_equals_literal_page_equation(shape):
    rng = np.random.default_rng([3, *shape])
    G = rng.standard_normal(shape)
    assert rel(newton_schulz(G, *Q5, 5, EPS), literal_page_form(G, *Q5, 5, EPS)) < 1e-12


def test_cubic_leaves_orthonormal_rows_fixed():
    rng = np.random.default_rng(5)
    Q = haar_q(rng, 24)[:10, :]            # 10×24 with orthonormal rows
    assert np.allclose(Q @ Q.T, np.eye(10), atol=1e-13)
    for shape_q in (Q, Q.T):               # also the tall (orthonormal columns) form
        out = newton_schulz(shape_q, *CUBIC, 7, EPS, normalize=False)
        assert rel(out, shape_q) < 1e-13


def test_cubic_converges_to_polar_factor():
    rng = np.random.default_rng(6)
    # well-conditioned so that 30 cubic steps converge from σ/‖G‖_F
    U = haar_q(rng, 12)
    V = haar_q(rng, 20)[:, :12]
    G = (U * np.linspace(1.0, 2.0, 12)[None, :]) @ V.T      # 12×20, full rank
    polar_u, _ = scipy.linalg.polar(G.T)                    # G.T = U_p P, U_p 20×12
    O = newton_schulz(G, *CUBIC, 30, EPS)
    assert rel(O, polar_u.T) < 1e-10
    Ot = newton_schulz(G.T, *CUBIC, 30, EPS)               # tall input
    assert rel(Ot, polar_u) < 1e-10


@pytest.mark.parametrize("shape", [(9, 15), (15, 9), (12, 12)])
def test_orthogonal_equivariance(shape):
    rng = np.random.default_rng([8, *shape])
    G = rng.standard_normal(shape)
    Q = haar_q(rng, shape[0])
    R = haar_q(rng, shape[1])
    lhs = newton_schulz(Q @ G @ R, *Q5, 5, EPS)
    rhs = Q @ newton_schulz(G, *Q5, 5, EPS) @ R
    assert rel(lhs, rhs) < 1e-12


def test_transpose_and_scale_equivariance():
    rng = np.random.default_rng(9)
    G = rng.standard_normal((11, 17))
    O = newton_schulz(G, *Q5, 5, EPS)
    assert rel(newton_schulz(G.T, *Q5, 5, EPS), O.T) < 1e-13
    for s in (1e-3, 37.0):
        # the start sG/(s‖G‖ + eps) equals G/(‖G‖ + eps/s): scaling G is scaling eps
        assert rel(newton_schulz(s * G, *Q5, 5, EPS), newton_schulz(G, *Q5, 5, EPS / s)) < 1e-13


def test_rank_one_closed_form_and_golden_sequence():
    """Rank-1 input u vᵀ·s: O = p^k(s/(s+eps)) u vᵀ, with p the scalar quintic."""
    with open(os.path.join(GOLDEN, "quintic_rank1.json")) as f:
        gold = json.load(f)
    rng = np.random.default_rng(10)
    u = rng.standard_normal(6); u /= np.linalg.norm(u)
    v = rng.standard_normal(14); v /= np.linalg.norm(v)
    for s in (1.0, 3.0):
        G = s * np.outer(u, v)
        t = s / (s + EPS)
        for k in range(1, 6):
            t = p_scalar(t, *Q5)
            O = newton_schulz(G, *Q5, k, EPS)
            assert rel(O, t * np.outer(u, v)) < 1e-12
    # the stored scalar sequence p^k(1), k = 1..5 (a + b + c = 0.701 is not 1:
    # the quintic does not fix unit singular values; they oscillate in ~0.7..1.1)
    t = 1.0
    for k, want in enumerate(gold["p_iterates_of_one"], start=1):
        t = p_scalar(t, *Q5)
        assert abs(t - want) < 5e-7, (k, t, want)


def test_eps_sits_on_the_norm():
    """With ‖G‖_F = eps the start is G/(2 eps): singular value 1/2, not 1."""
    u = np.zeros(4); u[0] = 1.0
    v = np.zeros(5); v[2] = 1.0
    G = EPS * np.outer(u, v)
    O = newton_schulz(G, *Q5, 1, EPS)
    assert abs(O[0, 2] - p_scalar(0.5, *Q5)) < 1e-12


def test_zero_input_gives_zero_update_and_pure_decay():
    G = np.zeros((5, 7)); B = np.zeros((5, 7))
    W = np.random.default_rng(12).standard_normal((5, 7))
    B1, O, W1 = muon_step(G, B, W, lr=0.02, mu=0.95, wd=0.01, eps=EPS, a=Q5[0], b=Q5[1],
                          c=Q5[2], steps=5)
    assert np.all(O == 0) and np.all(B1 == 0)
    assert np.array_equal(W1, (1 - 0.02 * 0.01) * W)


def test_momentum_closed_form():
    """From B = 0 with a constant G: B_t = G (1 − μ^t)/(1 − μ)."""
    rng = np.random.default_rng(13)
    G = rng.standard_normal((4, 6))
    B = np.zeros_like(G)
    mu = 0.95
    for t in range(1, 8):
        B = momentum_update(B, G, mu)
        assert rel(B, G * (1 - mu ** t) / (1 - mu)) < 1e-14


def test_update_closed_forms():
    rng = np.random.default_rng(14)
    W = rng.standard_normal((3, 5)); O = rng.standard_normal((3, 5))
    assert rel(decay_update(np.zeros_like(W), O, 0.02, 0.01), -0.02 * O) < 1e-15
    assert rel(decay_update(W, np.zeros_like(O), 0.02, 0.01), 0.9998 * W) < 1e-15
    # decoupled decay is scaled by lr: a Loshchilov-style (1 − wd) would give 0.99
    assert abs(decay_update(np.ones((1, 1)), np.zeros((1, 1)), 0.5, 0.2)[0, 0] - 0.9) < 1e-15


def test_step_order_momentum_then_ns_on_buffer():
    """μB + G is rank 2 with known singular values, so the whole step has a closed form."""
    rng = np.random.default_rng(15)
    Qu = haar_q(rng, 6); Qv = haar_q(rng, 9)
    u1, u2 = Qu[:, 0], Qu[:, 1]
    v1, v2 = Qv[:, 0], Qv[:, 1]
    mu, lr, wd = 0.95, 0.02, 0.01
    B = 2.0 * np.outer(u1, v1)
    G = 0.5 * np.outer(u2, v2)
    W = rng.standard_normal((6, 9))
    B1, O, W1 = muon_step(G, B, W, lr=lr, mu=mu, wd=wd, eps=EPS, a=Q5[0], b=Q5[1], c=Q5[2],
                          steps=5)
    s1, s2 = mu * 2.0, 0.5
    nrm = np.hypot(s1, s2) + EPS
    t1, t2 = s1 / nrm, s2 / nrm
    for _ in range(5):
        t1, t2 = p_scalar(t1, *Q5), p_scalar(t2, *Q5)
    O_want = t1 * np.outer(u1, v1) + t2 * np.outer(u2, v2)
    assert rel(B1, s1 * np.outer(u1, v1) + s2 * np.outer(u2, v2)) < 1e-14
    assert rel(O, O_want) < 1e-12
    assert rel(W1, (1 - lr * wd) * W - lr * O_want) < 1e-12


def test_3d_is_a_loop_over_last_two_dims():
    rng = np.random.default_rng(16)
    G = rng.standard_normal((4, 10, 6))
    B = rng.standard_normal((4, 10, 6))
    W = rng.standard_normal((4, 10, 6))
    hp = dict(lr=0.02, mu=0.95, wd=0.01, eps=EPS, a=Q5[0], b=Q5[1], c=Q5[2], steps=5)
    B1, O, W1 = muon_step(G, B, W, **hp)
    for i in range(4):
        b1, o, w1 = muon_step(G[i], B[i], W[i], **hp)
        assert rel(O[i], o) < 1e-14 and rel(W1[i], w1) < 1e-14 and rel(B1[i], b1) < 1e-14


def test_ndim_rule_from_pages():
    with open(os.path.join(GOLDEN, "ndim_rule.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        if case["accepted"]:
            validate_ndim(case["shape"])
        else:
            with pytest.raises(ValueError):
                validate_ndim(case["shape"])
