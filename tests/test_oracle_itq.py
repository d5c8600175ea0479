"""Pins of the Joint-ITQ oracle (oracle/itq.py) against what the mathematics
fixes: the orthogonal Procrustes step against brute force and local
optimality, exact recovery of a planted rotation, the alternation's
monotone objective, hypercube factors left alone, scale covariance and the
rotation invariance of the factor product.  CPU only."""
import numpy as np
import pytest
from scipy.linalg import expm

import oracle
import synth
from oracle import itq, svid


def _sylvester(n):
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def _rotation(rng, r, eps):
    """exp(eps * A) for a random skew-symmetric A: a rotation near I."""
    a = rng.standard_normal((r, r))
    return expm(eps * (a - a.T))


def test_procrustes_against_brute_force_in_two_dimensions():
    """Every 2x2 orthogonal matrix is a rotation or a reflection by some angle;
    the best <Z, R> over a fine grid of both may not exceed the Procrustes
    step's value, and comes within the grid's quadratic gap of it."""
    rng = np.random.default_rng(41)
    th = np.linspace(0.0, 2 * np.pi, 200001)
    c, s = np.cos(th), np.sin(th)
    for _ in range(5):
        Z = rng.standard_normal((2, 2))
        rot = Z[0, 0] * c - Z[0, 1] * s + Z[1, 0] * s + Z[1, 1] * c
        ref = Z[0, 0] * c + Z[0, 1] * s + Z[1, 0] * s - Z[1, 1] * c
        best = max(rot.max(), ref.max())
        R = itq.procrustes(Z)
        got = float(np.sum(Z * R))
        assert np.allclose(R.T @ R, np.eye(2), atol=1e-14)
        assert got >= best - 1e-12
        assert got <= best + 0.5 * (th[1] - th[0]) ** 2 * np.abs(Z).sum()


def test_procrustes_is_a_local_maximum():
    """No small rotation R exp(eps A) of the Procrustes solution raises <Z, R>."""
    rng = np.random.default_rng(42)
    Z = rng.standard_normal((6, 6))
    R = itq.procrustes(Z)
    base = float(np.sum(Z * R))
    assert np.allclose(R.T @ R, np.eye(6), atol=1e-13)
    for _ in range(200):
        Rq = R @ _rotation(rng, 6, 1e-3)
        assert float(np.sum(Z * Rq)) <= base + 1e-12


@pytest.mark.parametrize("which", ["both", "u_only", "v_only"])
def test_itq_recovers_a_planted_rotation(which):
    """Factors that are orthogonal +-1 columns turned by a rotation Q near I:
    their signs at R = I are those columns, so one step gives R = Q exactly and
    Q = 0 from then on.  With one factor zero the other alone must still give Q
    (both factors enter the Procrustes step)."""
    rng = np.random.default_rng(43)
    r = 8
    Q = _rotation(rng, r, 0.05)
    Bu, Bv = _sylvester(32)[:, :r], _sylvester(64)[:, 1:r + 1]
    Up, Vp = Bu @ Q.T, Bv @ Q.T
    if which == "u_only":
        Vp = np.zeros_like(Vp)
    if which == "v_only":
        Up = np.zeros_like(Up)
    R, q = itq.joint_itq(Up, Vp, 3)
    assert np.allclose(R, Q, atol=1e-12)
    zero_rows = Up.shape[0] * r if which == "v_only" else (Vp.shape[0] * r if which == "u_only" else 0)
    # a zero factor sits at distance 1 from its code (sign(0) = +1) in every entry
    assert q[1] == pytest.approx(zero_rows, abs=1e-9)
    assert q[0] > q[1]
    if which != "v_only":
        assert np.allclose(Up @ R, Bu, atol=1e-12)


def test_itq_objective_of_zero_factors():
    """sign(0) = +1: every entry of a zero factor is at distance 1 from its code."""
    assert itq.objective(np.zeros((5, 3)), np.zeros((7, 3)), np.eye(3)) == 36.0


def test_itq_objective_never_increases():
    """Each half-step is an exact minimisation, so the objective is monotone;
    the rotation stays orthogonal and the factor product is unchanged."""
    W = synth.dense_weight(5, 96, 80)
    Up, Vp = svid.truncated_factors(W, 24)
    R, q = itq.joint_itq(Up, Vp, 30)
    q = np.asarray(q)
    assert np.all(np.diff(q) <= 1e-12 * q[0])
    assert q[-1] < q[0]
    assert np.allclose(R.T @ R, np.eye(24), atol=1e-12)
    assert np.allclose((Up @ R) @ (Vp @ R).T, Up @ Vp.T, rtol=0, atol=1e-12 * np.abs(Up @ Vp.T).max())


def test_itq_leaves_hypercube_factors_alone():
    """Factors that already are scaled orthogonal +-1 columns are a fixed point:
    Z is a positive multiple of I, so R = I; a Hadamard layer initialised with
    Joint-ITQ is then reproduced exactly, as without it."""
    r = 8
    Up, Vp = 0.3 * _sylvester(16)[:, :r], 0.7 * _sylvester(32)[:, :r]
    R, q = itq.joint_itq(Up, Vp, 5)
    assert np.allclose(R, np.eye(r), atol=1e-13)
    lam = 2.0 ** -np.arange(r)
    W = _sylvester(16)[:, :r] @ np.diag(lam) @ _sylvester(32)[:, :r].T * 0.125
    U, V, h, g, l = svid.dual_svid(W, r, residual=False, f16=False, itq_iters=5)
    assert oracle.rel_l2(svid.reconstruction(U, V, h, g, l), W) < 1e-12


def test_itq_scale_covariance():
    """Scaling both factors by 4 (a power of two) scales Z by 4 and leaves its
    polar factor, hence every step, unchanged."""
    W = synth.dense_weight(6, 64, 72)
    Up, Vp = svid.truncated_factors(W, 16)
    Ra, _ = itq.joint_itq(Up, Vp, 10)
    Rb, _ = itq.joint_itq(4.0 * Up, 4.0 * Vp, 10)
    assert np.allclose(Ra, Rb, atol=1e-12)


def test_itq_in_dual_svid_lowers_the_sign_fit():
    """With Joint-ITQ the initialised factors sit closer to their signs (the
    objective the rotation minimises) than the plain Dual-SVID factors, and a
    rotation of the factors before the sign step keeps their product."""
    W = synth.dense_weight(7, 128, 96)
    U0, V0, *_ = svid.dual_svid(W, 32, residual=False, f16=False)
    U1, V1, *_ = svid.dual_svid(W, 32, residual=False, f16=False, itq_iters=20)
    q0 = itq.objective(U0[0], V0[0], np.eye(32))
    q1 = itq.objective(U1[0], V1[0], np.eye(32))
    assert q1 < q0
    assert np.allclose(U1[0] @ V1[0].T, U0[0] @ V0[0].T, atol=1e-12 * np.abs(W).max())
