"""Pins of the oracle's power estimate of the input scale (oracle.prism.power_scale).

The pages leave the scaling of Y_0 = A / c open; the option estimates the top
eigenvalue with eight block power passes and sets c = ||A||_F min(1, 2 mu).
Pinned here against values that do not come from the function itself: a
brute-force per-eigenvalue formula on diagonal matrices, the closed forms for
a scaled identity and a rank-one matrix, the norm bounds that hold for any
input, and the end-to-end roots against the eigendecomposition.
"""
import numpy as np
import pytest

import workloads as W
from oracle import closed_form as cf
from oracle import inv_newton as inw
from oracle import prism


def _brute_diag(lam, c, V, passes, factor):
    # diagonal A: column j of K_t has entries (lam_i / c)^t V[i, j]; the
    # norms are sums over i of those squares, computed one entry at a time
    n, p = V.shape
    best = 0.0
    for j in range(p):
        s_prev = s_last = 0.0
        for i in range(n):
            x = lam[i] / c
            s_prev += (x ** (passes - 1) * V[i, j]) ** 2
            s_last += (x ** passes * V[i, j]) ** 2
        best = max(best, (s_last / s_prev) ** 0.5)
    return c * min(1.0, factor * best)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_diagonal_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = 40
    lam = rng.uniform(0.1, 3.0, n)
    V = rng.standard_normal((n, 8))
    c = float(np.linalg.norm(lam))
    for passes in (1, 2, 4):
        got = prism.power_scale(np.diag(lam), c, V, passes=passes)
        assert got == pytest.approx(_brute_diag(lam, c, V, passes, 2.0), rel=1e-12)


def test_scaled_identity_and_rank_one():
    # a I_n: every ratio is a / (a sqrt(n)) = 1 / sqrt(n), so c = 2 a (n >= 4)
    n, a = 64, 3.0
    V = np.random.default_rng(5).standard_normal((n, 8))
    c = a * np.sqrt(n)
    assert prism.power_scale(a * np.eye(n), c, V) == pytest.approx(2.0 * a, rel=1e-14)
    # lambda u u^T: ||A||_F = lambda and K_t is parallel to u, ratio 1, so
    # min(1, 2) keeps c = lambda
    u = np.random.default_rng(6).standard_normal(n)
    u /= np.linalg.norm(u)
    A = 7.0 * np.outer(u, u)
    assert prism.power_scale(A, 7.0, V) == pytest.approx(7.0, rel=1e-12)
    # a start block orthogonal to the range leaves c unchanged (all ratios 0/0)
    w = np.linalg.qr(np.column_stack([u, V]))[0][:, 1:9]
    assert prism.power_scale(A, 7.0, w - np.outer(u, u @ w)) == 7.0


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_bounds_on_random_spd(seed):
    n = 96
    A, _, lam = W.spd_logu(n, 300 + seed, 10.0 ** -(seed + 1), 1.0)
    A = A.astype(np.float64)
    lmax = float(np.max(lam))
    cF = float(np.linalg.norm(A))
    V = prism.make_sketch_fn(seed)(prism.POWER_STAGE, 0, n)
    c = prism.power_scale(A, cF, V)
    # mu <= ||A / cF||_2, so c <= 2 lambda_max, and c <= cF always
    assert c <= cF * (1 + 1e-15)
    assert c <= 2.0 * lmax * (1 + 1e-12)
    # eight passes from eight Gaussian columns reach at least half of
    # lambda_max here, so c is an upper bound of the spectrum
    assert c >= lmax


def test_isolated_top_eigenvalue():
    # one eigenvalue 1 over a bulk of 0.45 at n = 4096: the start block puts a
    # weight of about 1/n on the top direction, and eight passes raise it by
    # (1/0.45)^16 ~ 3.5e5 against the bulk, so mu reaches the top and
    # c = 2 mu ||A||_F covers it (four passes would stop near the bulk)
    n = 4096
    lam = np.full(n, 0.45)
    lam[1234] = 1.0
    cF = float(np.linalg.norm(lam))
    V = prism.make_sketch_fn(0)(prism.POWER_STAGE, 0, n)
    c8 = prism.power_scale(np.diag(lam), cF, V)
    assert c8 == pytest.approx(_brute_diag(lam, cF, V, 8, 2.0), rel=1e-12)
    assert 1.0 <= c8 <= 2.0
    c4 = prism.power_scale(np.diag(lam), cF, V, passes=4)
    assert c4 < c8


def test_roots_and_iterations():
    # a flat spectrum of large order: ||A||_F ~ sqrt(n) lambda, the
    # Frobenius scale starts every eigenvalue near 0, the power scale near 1
    n = 200
    A, _, _ = W.spd_logu(n, 11, 0.5, 1.0)
    A = A.astype(np.float64)
    sk = prism.make_sketch_fn(3)
    for p in (2, 4):
        # results at a tight tolerance, iteration counts at the default one
        Xp, Ap, inf_p = prism.inv_root(A, p, sketch_fn=sk, max_iter=40, tol=1e-13,
                                       scale="power")
        ref, ref_aux = cf.inv_root(A, p)
        assert cf.rel_fro(Xp, ref) < 1e-9 and cf.rel_fro(Ap, ref_aux) < 1e-9
        _, _, inf_f = prism.inv_root(A, p, sketch_fn=sk, max_iter=40)
        _, _, inf_p = prism.inv_root(A, p, sketch_fn=sk, max_iter=40, scale="power")
        assert inf_p["status"] == prism.CONVERGED
        it_f = sum(t.iters for t in inf_f["stages"])
        it_p = sum(t.iters for t in inf_p["stages"])
        assert it_p < it_f, (p, it_p, it_f)
        assert inf_p["c"] < inf_f["c"]
    # the inverse Newton iteration takes the same scale
    X, XA, _ = inw.inv_root(A, 4, sketch_fn=sk, scale="power", tol=1e-13)
    ref, ref_aux = cf.inv_root(A, 4)
    assert cf.rel_fro(X, ref) < 1e-9 and cf.rel_fro(XA, ref_aux) < 1e-9
    _, _, inf = inw.inv_root(A, 4, sketch_fn=sk, scale="power")
    _, _, inf_f = inw.inv_root(A, 4, sketch_fn=sk)
    assert inf["stages"][0].iters <= inf_f["stages"][0].iters
    assert inf["status"] == prism.CONVERGED and inf["c"] < inf_f["c"]
    with pytest.raises(ValueError):
        prism.inv_root(A, 2, scale="spectral")


def test_polar_scale():
    # G with orthogonal columns of norm a: X_0^T X_0 = I / n, every ratio is
    # 1 / n, s^2 = 2 / n, so X_0 / s has singular values 1 / sqrt(2)
    n = 32
    Q = np.linalg.qr(np.random.default_rng(8).standard_normal((128, n)))[0]
    G = 3.0 * Q
    X0 = G / np.linalg.norm(G)
    R0 = np.eye(n) - X0.T @ X0
    V = prism.make_sketch_fn(1)(prism.POWER_STAGE, 0, n)
    s = prism.polar_power_scale(R0, V)
    assert s == pytest.approx(np.sqrt(2.0 / n), rel=1e-12)
    assert np.linalg.svd(X0 / s, compute_uv=False) == pytest.approx(np.full(n, 2 ** -0.5),
                                                                    rel=1e-12)
    # the scale shrinks c only, the factor matches the SVD, fewer updates on a
    # spread spectrum (the Muon workload's geometric singular values)
    rng = np.random.default_rng(9)
    U0 = np.linalg.qr(rng.standard_normal((512, 256)))[0]
    V0 = np.linalg.qr(rng.standard_normal((256, 256)))[0]
    G = (U0 * np.geomspace(1e-3, 1.0, 256)) @ V0.T
    sk = prism.make_sketch_fn(2)
    Up, ip = prism.polar(G, sketch_fn=sk, tol=1e-12, max_iter=60, scale="power")
    assert cf.rel_fro(Up, cf.polar(G)[0]) < 1e-9
    _, ip = prism.polar(G, sketch_fn=sk, tol=1e-2, scale="power")
    _, i_f = prism.polar(G, sketch_fn=sk, tol=1e-2)
    assert ip["c"] < i_f["c"]
    assert ip["stages"][0].iters < i_f["stages"][0].iters
    # s never exceeds 1 (X_0^T X_0 has eigenvalues at most 1)
    for seed in range(3):
        Gr = np.random.default_rng(seed).standard_normal((96, 40))
        X0 = Gr / np.linalg.norm(Gr)
        V40 = prism.make_sketch_fn(seed)(prism.POWER_STAGE, 0, 40)
        assert prism.polar_power_scale(np.eye(40) - X0.T @ X0, V40) <= 1.0
    # wide inputs go through G^T with the same scale
    Uw, iw = prism.polar(G.T, sketch_fn=sk, tol=1e-12, max_iter=60, scale="power")
    assert cf.rel_fro(Uw, cf.polar(G.T)[0]) < 1e-9 and iw["c"] == pytest.approx(ip["c"])
