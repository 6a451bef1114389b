"""Pins for the coupled inverse Newton reference (oracle.inv_newton)."""
import numpy as np
import pytest
from scipy.special import binom

import workloads as W
from oracle import closed_form as cf
from oracle import eigen_model as em
from oracle import interval, inv_newton as inw, philox, prism


def test_root_coefficients_binomial_series():
    for p in (2, 4):
        for j in range(6):
            assert inw.root_coeff(j, p) == pytest.approx(binom(-1.0 / p, j) * (-1) ** j, rel=1e-14)


@pytest.mark.parametrize("d,p", [(1, 4), (2, 4), (1, 2), (2, 2)])
def test_residual_map_direct_evaluation(d, p):
    rng = np.random.default_rng(d + 10 * p)
    xi = rng.uniform(-1, 1, 40)
    for alpha in (0.0, 0.2, inw.root_coeff(d, p), 0.55):
        f = sum(inw.root_coeff(j, p) * xi ** j for j in range(d))
        direct = 1 - (1 - xi) * (f + alpha * xi ** d) ** p
        np.testing.assert_allclose(inw.residual_map(xi, alpha, d, p), direct, atol=1e-13)
    for a in inw.map_coeffs(d, p):
        assert a[0] == 0.0
    if p == 2:
        # the square-root family's map
        for a, b in zip(inw.map_coeffs(d, 2), prism.map_coeffs(d)):
            np.testing.assert_allclose(a, b, atol=1e-15)


def test_taylor_coefficient_is_classical_inverse_newton():
    # d = 1, alpha = 1/4: X <- X (5I - M)/4, M <- ((5I - M)/4)^4 M (Iannazzo's
    # coupled inverse Newton for the 4th root), X_0 = I, M_0 = A/c
    A, _, _ = W.spd_logu(20, 4, 1e-2, 1.0)
    A = A.astype(np.float64)
    c = np.linalg.norm(A)
    X, _, info = inw.inv_root(A, p=4, d=1, lo=0.25, hi=0.25, tol=1e-12, max_iter=60)
    st = info["stages"][0]
    Xt, M = np.eye(20), A / c
    for _ in range(st.iters):
        T = (5 * np.eye(20) - M) / 4
        Xt, M = Xt @ T, np.linalg.matrix_power(T, 4) @ M
    np.testing.assert_allclose(X, Xt * c ** -0.25, atol=1e-12)
    _, _, info2 = inw.inv_root(A, p=4, d=1, accelerate=False, tol=1e-12, max_iter=60)
    assert info2["stages"][0].iters == st.iters


@pytest.mark.parametrize("d", [1, 2])
def test_exact_objective_equals_explicit_next_residual(d):
    # with S = I the fitted alpha minimises ||I - M_{k+1}||_F^2 computed by
    # doing the update for every alpha on a grid
    A, _, _ = W.spd_logu(12, 9, 1e-3, 1.0)
    A = A.astype(np.float64)
    M = A / np.linalg.norm(A)
    I = np.eye(12)
    lo, hi = inw.default_interval(d, 4)
    for _ in range(3):
        R = I - M
        alpha = inw.fit_alpha(inw.krylov_gram(R, I, 4 * d + 1), d, 4, lo, hi)

        def g_of(a):
            g = sum(inw.root_coeff(j, 4) * np.linalg.matrix_power(R, j) for j in range(d))
            return g + a * np.linalg.matrix_power(R, d)

        explicit = lambda a: np.linalg.norm(I - np.linalg.matrix_power(g_of(a), 4) @ M) ** 2
        grid = np.linspace(lo, hi, 20001)
        vals = np.array([explicit(a) for a in grid])
        assert abs(alpha - grid[np.argmin(vals)]) <= 2 * (hi - lo) / 20000 + 1e-9
        M = np.linalg.matrix_power(g_of(alpha), 4) @ M


def test_sketched_alpha_brute_force_grid():
    A, _, _ = W.spd_logu(40, 8, 1e-3, 1.0)
    R = np.eye(40) - A.astype(np.float64) / np.linalg.norm(A)
    S = philox.sketch(77, 0, 0, 0, 40, 8)
    for d in (1, 2):
        lo, hi = inw.default_interval(d, 4)
        J = 4 * d + 1
        alpha = inw.fit_alpha(inw.krylov_gram(R, S, J), d, 4, lo, hi)
        K = [S]
        for _ in range(J):
            K.append(R @ K[-1])
        # || sum_j r_j(alpha) K_j ||^2 on a fine grid, straight from the map
        Kf = np.stack([k.reshape(-1) for k in K])
        A_ = inw.map_coeffs(d, 4)
        grid = np.linspace(lo, hi, 400_001)
        C = sum(grid[:, None] ** i * A_[i][None, :] for i in range(5))
        vals = np.einsum("ij,jk,ik->i", C, Kf @ Kf.T, C)
        assert abs(alpha - grid[np.argmin(vals)]) < 5e-6


@pytest.mark.parametrize("p", [2, 4])
def test_converges_to_closed_form(p):
    c = W.spd_64()
    A = c["A"].astype(np.float64)
    for d in (1, 2):
        X, Xa, info = inw.inv_root(A, p=p, d=d, sketch_fn=prism.make_sketch_fn(3), tol=1e-10,
                                   max_iter=60)
        Xr, Xar = cf.inv_root(A, p)
        assert info["status"] == prism.CONVERGED
        assert cf.rel_fro(X, Xr) < 1e-9 and cf.rel_fro(Xa, Xar) < 1e-9
        st = info["stages"][0]
        # products: (d - 1) powers, log2(p) powers of g, g^p M, X g (not at k = 0)
        per = (d - 1) + (1 if p == 2 else 2) + 1
        assert st.gemms == per * st.iters + st.iters - 1


@pytest.mark.parametrize("d", [1, 2])
def test_iteration_counts_match_eigen_model(d):
    c = W.spd_64()
    Q, lam = c["Q"], c["lam"]
    A = W.spd_from_spectrum(Q, lam)
    lo, hi = inw.default_interval(d, 4)
    _, _, info = inw.inv_root(A, p=4, d=d, sketch_fn=prism.exact_sketch_fn(), max_iter=60)
    st = info["stages"][0]
    model = em.run(1 - lam / np.linalg.norm(lam), d, lo, hi, 1e-6, 60,
                   rmap=lambda x, a, dd: inw.residual_map(x, a, dd, 4),
                   taylor=lambda dd: inw.root_coeff(dd, 4))
    assert st.iters == model["iters"]
    np.testing.assert_allclose(st.alpha, model["alpha"], atol=1e-7)


def test_interval_rule_for_the_fourth_root_map():
    # the same rule as the square-root family's: d = 1 gives 1/2 exactly (the
    # linear coefficient 1 - 4 alpha binds), d = 2 about 0.6039
    rm = lambda d: (lambda x, a: inw.residual_map(x, a, d, 4))
    u1 = interval.upper_bound(1, top=2.0, iters=24, samples=50, rmap=rm(1), lo=0.25)
    assert abs(u1 - 0.5) < 1e-6
    u2 = interval.upper_bound(2, top=2.0, iters=24, samples=50, rmap=rm(2), lo=5 / 32)
    assert 0.6030 < u2 < 0.6045
    assert inw.default_interval(1, 4) == (0.25, 0.5)
    lo2, hi2 = inw.default_interval(2, 4)
    assert lo2 == 5 / 32 and hi2 <= u2
    assert inw.default_interval(2, 2) == prism.default_interval(2)


def test_fewer_products_than_the_chained_square_roots():
    # the comparison the method is built for (fp64, same sketches)
    A, _, _ = W.spd_logu(64, 3, 1e-4, 1.0)
    A = A.astype(np.float64)
    _, _, nw = inw.inv_root(A, p=4, d=2, sketch_fn=prism.make_sketch_fn(1))
    _, _, ch = prism.inv_root(A, p=4, d=2, sketch_fn=prism.make_sketch_fn(1))
    assert nw["stages"][0].gemms < sum(s.gemms for s in ch["stages"])
