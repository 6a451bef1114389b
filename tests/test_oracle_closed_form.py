"""Pins for oracle.closed_form against closed forms, independent library
routines (Schur-based scipy functions) and 50-digit brute force (mpmath)."""
import mpmath
import numpy as np
import pytest
import scipy.linalg as sla

import workloads as W
from oracle import closed_form as cf


def test_stats_constant_gradient_geometric_series():
    # L_t = beta L_{t-1} + (1-beta) C + eps I has the fixed point
    # L* = C + eps/(1-beta) I, and L_T - L* = beta^T (L_0 - L*).
    rng = np.random.default_rng(0)
    G = rng.standard_normal((6, 9))
    beta, eps, T = 0.95, 1e-3, 10
    L0 = 0.5 * np.eye(6)
    R0 = 2.0 * np.eye(9)
    L, R = cf.stats_sequence(L0, R0, [G] * T, beta, eps)
    Ls = G @ G.T + eps / (1 - beta) * np.eye(6)
    Rs = G.T @ G + eps / (1 - beta) * np.eye(9)
    np.testing.assert_allclose(L, Ls + beta ** T * (L0 - Ls), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(R, Rs + beta ** T * (R0 - Rs), rtol=1e-12, atol=1e-13)


def test_stats_rank_one():
    # G = u v^T: G G^T = |v|^2 u u^T and G^T G = |u|^2 v v^T
    u = np.array([1.0, -2.0, 0.5])
    v = np.array([3.0, 0.0, 1.0, -1.0])
    G = np.outer(u, v)
    L, R = cf.stats_update(np.zeros((3, 3)), np.zeros((4, 4)), G, 0.0, 0.0)
    np.testing.assert_allclose(L, (v @ v) * np.outer(u, u), rtol=1e-15)
    np.testing.assert_allclose(R, (u @ u) * np.outer(v, v), rtol=1e-15)
    L, R = cf.stats_update(np.eye(3), np.eye(4), G, 0.25, 0.5)
    np.testing.assert_allclose(L, 0.25 * np.eye(3) + 0.75 * (v @ v) * np.outer(u, u) + 0.5 * np.eye(3))


def test_roots_diagonal():
    lam = np.array([1e-3, 0.25, 1.0, 7.0, 16.0])
    X2, A2 = cf.inv_root(np.diag(lam), 2)
    X4, A4 = cf.inv_root(np.diag(lam), 4)
    np.testing.assert_allclose(np.diag(X2), lam ** -0.5, rtol=1e-13)
    np.testing.assert_allclose(np.diag(A2), lam ** 0.5, rtol=1e-13)
    np.testing.assert_allclose(np.diag(X4), lam ** -0.25, rtol=1e-13)
    np.testing.assert_allclose(np.diag(A4), lam ** 0.25, rtol=1e-13)
    assert np.max(np.abs(X4 - np.diag(np.diag(X4)))) < 1e-13


def test_roots_known_spectrum():
    # A = Q Lambda Q^T with the Q and Lambda used to build it
    A, Q, lam = W.spd_logu(32, 5)
    A = W.spd_from_spectrum(Q, lam)
    X, Xa = cf.inv_root(A, 4)
    np.testing.assert_allclose(X, (Q * lam ** -0.25) @ Q.T, rtol=0, atol=1e-11)
    np.testing.assert_allclose(Xa, (Q * lam ** 0.25) @ Q.T, rtol=0, atol=1e-12)
    # invariants X^4 A = I, (A^{1/2})^2 = A, A^{1/2} A^{-1/2} = I
    np.testing.assert_allclose(np.linalg.matrix_power(X, 4) @ A, np.eye(32), atol=1e-9)
    X2, A2 = cf.inv_root(A, 2)
    np.testing.assert_allclose(A2 @ A2, A, atol=1e-13)
    np.testing.assert_allclose(A2 @ X2, np.eye(32), atol=1e-10)


def test_roots_2x2_closed_form():
    # sqrt of a 2x2 SPD: (A + s I) / t, s = sqrt(det A), t = sqrt(tr A + 2 s)
    A = np.array([[4.0, 1.5], [1.5, 2.0]])
    s = np.sqrt(np.linalg.det(A))
    t = np.sqrt(np.trace(A) + 2 * s)
    sq = (A + s * np.eye(2)) / t
    X2, A2 = cf.inv_root(A, 2)
    np.testing.assert_allclose(A2, sq, rtol=1e-14)
    np.testing.assert_allclose(X2, np.linalg.inv(sq), rtol=1e-13)
    s2 = np.sqrt(np.linalg.det(sq))
    qr = (sq + s2 * np.eye(2)) / np.sqrt(np.trace(sq) + 2 * s2)
    X4, A4 = cf.inv_root(A, 4)
    np.testing.assert_allclose(A4, qr, rtol=1e-13)
    np.testing.assert_allclose(X4, np.linalg.inv(qr), rtol=1e-13)


def test_roots_mpmath_4x4():
    mpmath.mp.dps = 50
    rng = np.random.default_rng(11)
    B = rng.standard_normal((4, 4))
    A = B @ B.T + 0.1 * np.eye(4)
    Am = mpmath.matrix(A.tolist())
    E, Q = mpmath.eigsy(Am)
    for p in (2, 4):
        D = mpmath.diag([e ** (mpmath.mpf(-1) / p) for e in E])
        ref = np.array((Q * D * Q.T).tolist(), dtype=np.float64)
        X, _ = cf.inv_root(A, p)
        np.testing.assert_allclose(X, ref, rtol=1e-12, atol=1e-13)


def test_roots_against_schur_routines():
    A, Q, lam = W.spd_logu(24, 9, 1e-2, 1.0)
    A = A.astype(np.float64)
    X4, A4 = cf.inv_root(A, 4)
    np.testing.assert_allclose(X4, np.real(sla.fractional_matrix_power(cf.sym(A), -0.25)), atol=1e-10)
    X2, A2 = cf.inv_root(A, 2)
    np.testing.assert_allclose(A2, np.real(sla.sqrtm(cf.sym(A))), atol=1e-11)


def test_roots_reject_indefinite():
    with pytest.raises(ValueError):
        cf.inv_root(np.diag([1.0, -0.5]), 2)


def test_polar_against_scipy_and_invariants():
    G = W.gaussian(40, 12, 3).astype(np.float64)
    U, H = cf.polar(G)
    Us, Hs = sla.polar(G)
    np.testing.assert_allclose(U, Us, atol=1e-12)
    np.testing.assert_allclose(U.T @ U, np.eye(12), atol=1e-13)
    np.testing.assert_allclose(U @ H, G, atol=1e-12)
    assert np.all(np.linalg.eigvalsh(0.5 * (U.T @ G + G.T @ U)) > 0)


def test_polar_known_factors():
    # G = Q H with Q (m x n) orthonormal columns and H SPD: the factor is Q
    rng = np.random.default_rng(4)
    Q = W.random_orthogonal(rng, 20, 7)
    B = rng.standard_normal((7, 7))
    H = B @ B.T + np.eye(7)
    U, Hc = cf.polar(Q @ H)
    np.testing.assert_allclose(U, Q, atol=1e-12)
    np.testing.assert_allclose(Hc, H, atol=1e-11)


def test_polar_mpmath_and_rank_deficient():
    mpmath.mp.dps = 50
    rng = np.random.default_rng(8)
    G = rng.standard_normal((5, 3))
    U, S, V = mpmath.svd_r(mpmath.matrix(G.tolist()), full_matrices=False)
    ref = np.array((U * V).tolist(), dtype=np.float64)
    np.testing.assert_allclose(cf.polar(G)[0], ref, atol=1e-13)
    # rank 1: the partial isometry u v^T / (|u||v|)
    u = np.array([1.0, 2.0, -1.0, 0.5])
    v = np.array([0.5, -1.0, 2.0])
    Up, _ = cf.polar(np.outer(u, v))
    np.testing.assert_allclose(Up, np.outer(u, v) / (np.linalg.norm(u) * np.linalg.norm(v)), atol=1e-14)


def test_apply_kronecker_identity():
    # row-major vec: vec(L G R) = (L kron R^T) vec(G)
    rng = np.random.default_rng(1)
    m, n = 5, 3
    L = rng.standard_normal((m, m))
    R = rng.standard_normal((n, n))
    G = rng.standard_normal((m, n))
    P = cf.precond_apply(L, G, R)
    np.testing.assert_allclose(P.reshape(-1), np.kron(L, R.T) @ G.reshape(-1), rtol=1e-12)
