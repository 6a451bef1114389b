"""Pins for the step-by-step PRISM reference (oracle.prism), the interval rule
(oracle.interval) and the scalar eigenvalue model (oracle.eigen_model)."""
import numpy as np
import pytest
from scipy.special import binom

import workloads as W
from oracle import closed_form as cf
from oracle import eigen_model as em
from oracle import interval, philox, prism


def test_taylor_coefficients_binomial_series():
    # (1 - xi)^{-1/2} = sum_j binom(-1/2, j) (-xi)^j
    for j in range(8):
        assert prism.taylor_coeff(j) == pytest.approx(binom(-0.5, j) * (-1) ** j, rel=1e-15)


@pytest.mark.parametrize("d", [1, 2, 3])
def test_residual_map_direct_evaluation(d):
    # r(xi; alpha) = 1 - (1 - xi) (f_{d-1}(xi) + alpha xi^d)^2, evaluated directly
    rng = np.random.default_rng(d)
    xi = rng.uniform(-1, 1, 50)
    for alpha in (0.0, 0.3, prism.taylor_coeff(d), 1.2):
        f = sum(prism.taylor_coeff(j) * xi ** j for j in range(d))
        direct = 1 - (1 - xi) * (f + alpha * xi ** d) ** 2
        np.testing.assert_allclose(prism.residual_map(xi, alpha, d), direct, atol=1e-14)
    # the map has no constant term: K_0 = S never contributes
    for a in prism.map_coeffs(d):
        assert a[0] == 0.0


def _textbook_ns(Y0, d, iters):
    """Classical coupled Newton-Schulz (Higham's coupled iteration):
    d = 1: M = (3I - ZY)/2;  d = 2: M = (15I - 10 ZY + 3 (ZY)^2)/8;
    d = 3: M = (35I - 35 ZY + 21 (ZY)^2 - 5 (ZY)^3)/16;  Y <- Y M, Z <- M Z."""
    n = Y0.shape[0]
    Y, Z = Y0.copy(), np.eye(n)
    for _ in range(iters):
        T = Z @ Y
        if d == 1:
            M = (3 * np.eye(n) - T) / 2
        elif d == 2:
            M = (15 * np.eye(n) - 10 * T + 3 * T @ T) / 8
        else:
            M = (35 * np.eye(n) - 35 * T + 21 * T @ T - 5 * T @ T @ T) / 16
        Y, Z = Y @ M, M @ Z
    return Y, Z


@pytest.mark.parametrize("d", [1, 2, 3])
def test_taylor_interval_is_classical_newton_schulz(d):
    A, _, _ = W.spd_logu(16, 3, 1e-2, 1.0)
    A = A.astype(np.float64)
    Y0 = A / np.linalg.norm(A)
    cd = prism.taylor_coeff(d)
    Y, Z, tr = prism.coupled_sqrt_stage(Y0, d=d, lo=cd, hi=cd, tol=1e-12, max_iter=40,
                                        sketch_fn=prism.make_sketch_fn(1))
    Yt, Zt = _textbook_ns(Y0, d, tr.iters)
    np.testing.assert_allclose(Y, Yt, atol=1e-13)
    np.testing.assert_allclose(Z, Zt, atol=1e-12)
    assert all(a == cd for a in tr.alpha)
    # accelerate=False is the same iteration
    Y2, Z2, tr2 = prism.coupled_sqrt_stage(Y0, d=d, tol=1e-12, max_iter=40, accelerate=False)
    assert tr2.iters == tr.iters
    np.testing.assert_allclose(Y2, Yt, atol=1e-13)


@pytest.mark.parametrize("d", [1, 2, 3])
def test_exact_objective_equals_explicit_next_residual(d):
    # with S = I, fit_alpha minimises ||I - Z_{k+1} Y_{k+1}||_F^2 computed by
    # actually performing the update for every alpha on a grid
    A, _, _ = W.spd_logu(12, 21, 1e-3, 1.0)
    A = A.astype(np.float64)
    Y = A / np.linalg.norm(A)
    Z = np.eye(12)
    lo, hi = prism.default_interval(d)
    for _ in range(3):
        R = np.eye(12) - Z @ Y
        alpha = prism.fit_alpha(prism.krylov_gram(R, np.eye(12), d), d, lo, hi)

        def explicit(a):
            g = sum(prism.taylor_coeff(j) * np.linalg.matrix_power(R, j) for j in range(d))
            g = g + a * np.linalg.matrix_power(R, d)
            return np.linalg.norm(np.eye(12) - (g @ Z) @ (Y @ g)) ** 2

        grid = np.linspace(lo, hi, 20001)
        vals = np.array([explicit(a) for a in grid])
        a_bf = grid[np.argmin(vals)]
        assert abs(alpha - a_bf) <= 2 * (hi - lo) / 20000 + 1e-9
        assert explicit(alpha) <= vals.min() + 1e-12 * max(1.0, vals.min())
        g = sum(prism.taylor_coeff(j) * np.linalg.matrix_power(R, j) for j in range(d))
        g = g + alpha * np.linalg.matrix_power(R, d)
        Y, Z = Y @ g, g @ Z


@pytest.mark.parametrize("d", [1, 2, 3])
def test_sketched_alpha_brute_force_grid(d):
    A, _, _ = W.spd_logu(40, 8, 1e-3, 1.0)
    A = A.astype(np.float64)
    R = np.eye(40) - A / np.linalg.norm(A)
    lo, hi = prism.default_interval(d)
    S = philox.sketch(77, 0, 0, 0, 40, 8)
    alpha = prism.fit_alpha(prism.krylov_gram(R, S, d), d, lo, hi)
    grid = np.linspace(lo, hi, 1_000_001)
    a0, a1, a2 = prism.map_coeffs(d)
    K = [S]
    for _ in range(2 * d + 1):
        K.append(R @ K[-1])
    # phi_S(alpha) = || sum_j c_j(alpha) K_j ||^2 evaluated on the grid via the
    # Gram of K, independently of the quartic coefficients
    Kf = np.stack([k.reshape(-1) for k in K])          # (2d+2, n p)
    C = a0[None, :] + grid[:, None] * a1[None, :] + grid[:, None] ** 2 * a2[None, :]
    G = Kf @ Kf.T
    vals = np.einsum("ij,jk,ik->i", C, G, C)
    assert abs(alpha - grid[np.argmin(vals)]) < 2e-6


def test_alpha_stays_in_interval_and_degenerate_cases():
    rng = np.random.default_rng(5)
    for d in (1, 2, 3):
        lo, hi = prism.default_interval(d)
        for _ in range(200):
            B = rng.standard_normal((2 * d + 2, 2 * d + 2)) * 10.0 ** rng.uniform(-8, 2)
            M = B @ B.T
            a = prism.fit_alpha(M, d, lo, hi)
            assert lo <= a <= hi
        # a zero Gram (R = 0) and a non-finite Gram fall back to the Taylor coefficient
        assert prism.fit_alpha(np.zeros((2 * d + 2,) * 2), d, lo, hi) == prism.taylor_coeff(d)
        bad = np.eye(2 * d + 2)
        bad[1, 1] = np.nan
        assert prism.fit_alpha(bad, d, lo, hi) == prism.taylor_coeff(d)
        assert prism.fit_alpha(np.eye(2 * d + 2), d, 0.7, 0.7) == 0.7


def test_eigenbasis_route_gives_same_alpha():
    # A = Q Lambda Q^T: phi_S(alpha) = sum_i w_i r(xi_i; alpha)^2 with
    # w_i = ||row_i(Q^T S)||^2 (O(n p) route, no Krylov products)
    c = W.spd_64()
    Q, lam = c["Q"], c["lam"]
    A = W.spd_from_spectrum(Q, lam)
    nrm = np.linalg.norm(A)
    R = np.eye(64) - A / nrm
    xi = 1 - lam / nrm
    for d in (1, 2):
        lo, hi = prism.default_interval(d)
        for k in range(3):
            S = philox.sketch(5, 0, 0, k, 64, 8)
            a_mat = prism.fit_alpha(prism.krylov_gram(R, S, d), d, lo, hi)
            w = np.sum((Q.T @ S) ** 2, axis=1)
            a_eig = em.argmin_alpha(xi, w, d, lo, hi)
            assert abs(a_mat - a_eig) < 1e-7


@pytest.mark.parametrize("d", [1, 2, 3])
def test_eigen_model_iteration_counts_match_matrix_iteration(d):
    c = W.spd_64()
    Q, lam = c["Q"], c["lam"]
    A = W.spd_from_spectrum(Q, lam)
    lo, hi = prism.default_interval(d)
    _, _, info = prism.inv_root(A, p=2, d=d, sketch_fn=prism.exact_sketch_fn())
    st = info["stages"][0]
    model = em.run(1 - lam / np.linalg.norm(lam), d, lo, hi, 1e-6, 100)
    assert st.iters == model["iters"]
    np.testing.assert_allclose(st.alpha, model["alpha"], atol=1e-7)
    np.testing.assert_allclose(st.r, model["r"], rtol=1e-6, atol=1e-12)
    assert st.gemms == em.products_sqrt_stage(st.iters, d)


def test_hutchinson_unbiased():
    # E[tr(S^T R^j S)] = p tr(R^j) for Gaussian S
    A, _, _ = W.spd_logu(16, 2)
    R = np.eye(16) - A.astype(np.float64) / np.linalg.norm(A)
    p = 8
    for j in (1, 2, 3):
        Rj = np.linalg.matrix_power(R, j)
        est = []
        for s in range(400):
            S = philox.sketch(1000 + s, 0, 0, 0, 16, p)
            est.append(np.trace(S.T @ Rj @ S) / p)
        est = np.array(est)
        se = est.std() / np.sqrt(len(est))
        assert abs(est.mean() - np.trace(Rj)) < 5 * se


@pytest.mark.parametrize("p", [2, 4])
def test_prism_roots_converge_to_closed_form(p):
    c = W.spd_64()
    A = c["A"].astype(np.float64)
    X, Xa, info = prism.inv_root(A, p=p, sketch_fn=prism.make_sketch_fn(3), tol=1e-9)
    Xr, Xar = cf.inv_root(A, p)
    assert info["status"] == prism.CONVERGED
    assert cf.rel_fro(X, Xr) < 1e-9
    assert cf.rel_fro(Xa, Xar) < 1e-9
    assert len(info["stages"]) == (1 if p == 2 else 2)


def test_prism_polar_converges_to_closed_form():
    G = W.gaussian(64, 32, 102).astype(np.float64)
    U, info = prism.polar(G, sketch_fn=prism.make_sketch_fn(3), tol=1e-10)
    assert info["status"] == prism.CONVERGED
    assert cf.rel_fro(U, cf.polar(G)[0]) < 1e-9
    Uw, info = prism.polar(G.T, sketch_fn=prism.make_sketch_fn(3), tol=1e-10)
    assert cf.rel_fro(Uw, cf.polar(G.T)[0]) < 1e-9
    st = info["stages"][0]
    assert st.gemms == em.products_polar(st.iters, 2)


def test_prism_needs_fewer_products_than_taylor():
    # the pages report fewer multiplications with PRISM (ratio unpinned)
    for lam_lo in (1e-3, 1e-5):
        A, _, _ = W.spd_logu(48, 31, lam_lo, 1.0)
        _, _, fast = prism.inv_root(A.astype(np.float64), p=2, sketch_fn=prism.make_sketch_fn(1))
        _, _, slow = prism.inv_root(A.astype(np.float64), p=2, accelerate=False)
        assert fast["stages"][0].gemms < slow["stages"][0].gemms


def test_interval_rule_reproduces_page_interval():
    # the rule gives the page's [1/2, 1] for d = 1 and about 1.4722 for d = 2
    u1 = interval.upper_bound(1)
    assert abs(u1 - 1.0) < 1e-6
    u2 = interval.upper_bound(2)
    assert 1.4715 < u2 < 1.4730
    assert prism.default_interval(2)[1] <= u2
    assert prism.default_interval(1) == (0.5, 1.0)


def test_interval_rule_degree_three():
    # d = 3 (the Taylor coefficient 5/16 and the same rule): about 2.4686
    u3 = interval.upper_bound(3, iters=24, samples=60)
    assert 2.4680 < u3 < 2.4692
    lo, hi = prism.default_interval(3)
    assert lo == prism.taylor_coeff(3) == 5 / 16
    assert hi <= u3 and interval.admissible(hi, 3)
    assert not interval.admissible(2.6, 3)


@pytest.mark.parametrize("p", [2, 4])
def test_degree_three_roots_and_polar_converge(p):
    c = W.spd_64()
    A = c["A"].astype(np.float64)
    X, Xa, info = prism.inv_root(A, p=p, d=3, sketch_fn=prism.make_sketch_fn(3), tol=1e-9)
    Xr, Xar = cf.inv_root(A, p)
    assert info["status"] == prism.CONVERGED
    assert cf.rel_fro(X, Xr) < 1e-9 and cf.rel_fro(Xa, Xar) < 1e-9
    for st in info["stages"]:
        assert st.gemms == em.products_sqrt_stage(st.iters, 3)
    if p == 2:
        G = W.gaussian(64, 32, 102).astype(np.float64)
        U, pinfo = prism.polar(G, d=3, sketch_fn=prism.make_sketch_fn(3), tol=1e-10)
        assert pinfo["status"] == prism.CONVERGED
        assert cf.rel_fro(U, cf.polar(G)[0]) < 1e-9
        assert pinfo["stages"][0].gemms == em.products_polar(pinfo["stages"][0].iters, 3)


def test_status_codes():
    # indefinite input: a residual eigenvalue above 1 grows until r > 2
    A = np.diag([1.0, 0.5, -0.3, 0.2])
    _, _, info = prism.inv_root(A, p=2, sketch_fn=prism.make_sketch_fn(0))
    assert info["status"] == prism.DIVERGED
    A = np.eye(4)
    A[1, 2] = np.nan
    _, _, info = prism.inv_root(A, p=2)
    assert info["status"] == prism.NONFINITE
    _, _, info = prism.inv_root(np.zeros((3, 3)), p=4)
    assert info["status"] == prism.NONFINITE
    A64 = W.spd_64()["A"].astype(np.float64)
    _, _, info = prism.inv_root(A64, p=2, max_iter=1)
    assert info["status"] == prism.MAXITER and info["stages"][0].iters == 1
    _, _, info = prism.inv_root(A64, p=2, tol=0.0)
    assert info["status"] == prism.STAGNATED
    # rank-deficient polar input: zero singular values stay at xi = 1
    G = np.outer(np.arange(1.0, 9.0), np.ones(4))
    U, info = prism.polar(G, max_iter=30)
    assert info["status"] in (prism.MAXITER, prism.STAGNATED)
    np.testing.assert_allclose(U, cf.polar(G)[0], atol=1e-6)


def test_predicted_contraction_is_the_sketched_next_residual():
    # q = sqrt(phi_S(alpha)) / ||R S|| equals ||r(R; alpha) S|| / ||R S|| with
    # r(R; alpha) = I - (I - R) g(R)^2 formed explicitly
    A, _, _ = W.spd_logu(30, 12, 1e-3, 1.0)
    R = np.eye(30) - A.astype(np.float64) / np.linalg.norm(A)
    S = philox.sketch(9, 0, 0, 0, 30, 8)
    for d in (1, 2, 3):
        lo, hi = prism.default_interval(d)
        M = prism.krylov_gram(R, S, d)
        alpha = prism.fit_alpha(M, d, lo, hi)
        g = sum(prism.taylor_coeff(j) * np.linalg.matrix_power(R, j) for j in range(d))
        g = g + alpha * np.linalg.matrix_power(R, d)
        rR = np.eye(30) - (np.eye(30) - R) @ g @ g
        q = np.linalg.norm(rR @ S) / np.linalg.norm(R @ S)
        assert prism.predicted_contraction(M, d, alpha) == pytest.approx(q, rel=1e-9)


@pytest.mark.parametrize("ratio", [0.3, 0.6])
def test_adaptive_degree_matches_eigen_model(ratio):
    # exact sketch (S = I): the matrix iteration's degree schedule, alphas and
    # iteration count equal the scalar model's, whose contraction is computed
    # from the residual spectrum directly
    c = W.spd_64()
    Q, lam = c["Q"], c["lam"]
    A = W.spd_from_spectrum(Q, lam)
    _, _, info = prism.inv_root(A, p=2, d=2, degree_max=3, adapt_ratio=ratio,
                                sketch_fn=prism.exact_sketch_fn())
    st = info["stages"][0]
    lo, hi = prism.default_interval(2)
    model = em.run(1 - lam / np.linalg.norm(lam), 2, lo, hi, 1e-6, 100, degree_max=3,
                   adapt_ratio=ratio, intervals={3: prism.default_interval(3)})
    assert st.degree == model["degree"]
    assert st.iters == model["iters"]
    np.testing.assert_allclose(st.alpha, model["alpha"], atol=1e-7)
    assert 3 in st.degree
    # dense products: per update (d - 1) powers, Y g, g Z (not at k = 0), Z Y
    assert st.gemms == sum(d - 1 + 2 for d in st.degree) + len(st.degree) - 1


def test_adaptive_degree_limits():
    A, _, _ = W.spd_logu(40, 6, 1e-4, 1.0)
    A = A.astype(np.float64)
    fn = prism.make_sketch_fn(2)
    _, _, fixed = prism.inv_root(A, p=2, d=2, sketch_fn=fn)
    _, _, never = prism.inv_root(A, p=2, d=2, degree_max=3, adapt_ratio=np.inf, sketch_fn=fn)
    _, _, always = prism.inv_root(A, p=2, d=2, degree_max=3, adapt_ratio=-1.0, sketch_fn=fn)
    f, nv, al = fixed["stages"][0], never["stages"][0], always["stages"][0]
    assert nv.iters == f.iters and nv.alpha == f.alpha and set(nv.degree) == {2}
    assert al.degree[0] == 2 and set(al.degree[1:]) == {3}


@pytest.mark.parametrize("p", [2, 4])
def test_adaptive_degree_converges_to_closed_form(p):
    A, _, _ = W.spd_logu(48, 17, 1e-5, 1.0)
    A = A.astype(np.float64)
    X, Xa, info = prism.inv_root(A, p=p, d=2, degree_max=3, sketch_fn=prism.make_sketch_fn(4),
                                 tol=1e-9)
    Xr, Xar = cf.inv_root(A, p)
    assert info["status"] == prism.CONVERGED
    assert cf.rel_fro(X, Xr) < 1e-9 and cf.rel_fro(Xa, Xar) < 1e-9
    G = W.gaussian(64, 40, 5).astype(np.float64)
    U, pinfo = prism.polar(G, d=2, degree_max=3, sketch_fn=prism.make_sketch_fn(4), tol=1e-10)
    assert pinfo["status"] == prism.CONVERGED
    assert cf.rel_fro(U, cf.polar(G)[0]) < 1e-9
