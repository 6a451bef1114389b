"""Coupled inverse Newton iteration for A^{-1/p} with the PRISM coefficient
(CPU, fp64).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The [PRISM synthesis] (key contributions) names inverse Newton methods among
the iterations PRISM accelerates; the pages give no formulas for them.  The
reading used here is the standard coupled form written in the residual
language of Part I:
  c = ||A||_F, M_0 = A / c, X_0 = I, R_k = I - M_k;
  g(xi; alpha) = f_{d-1}(xi) + alpha xi^d, f the Taylor polynomial of
  (1 - xi)^{-1/p} (coefficients b_j = prod_{i<j} (1/p + i) / (i + 1));
  X_{k+1} = X_k g(R_k),  M_{k+1} = g(R_k)^p M_k,
so that M_k = X_k^p M_0 and X -> (A/c)^{-1/p} as M -> I; A^{-1/p} = c^{-1/p} X
and A^{1/p} = c^{1/p} (A/c) X^{p-1}.  In exact arithmetic the residual
eigenvalues follow r(xi; alpha) = 1 - (1 - xi) g(xi; alpha)^p, a polynomial of
degree p in alpha, so the sketched objective phi_S(alpha) = ||r(R_k; alpha) S||^2
has degree 2p in alpha (an octic for p = 4) with coefficients from the Gram
matrix of K_j = R_k^j S, j = 1..p d + 1.  alpha_k is its minimiser over
[lo, hi]; with lo = hi = b_d and d = 1 the iteration is the classical coupled
inverse Newton X <- X ((p + 1) I - M) / p, M <- (((p + 1) I - M) / p)^p M.
The interval: lo = b_d and hi = the bound of oracle.interval's rule applied to
this r (for p = 2 the map is the square-root family's, so the same interval).
Stopping rule as oracle.prism.
"""
from math import comb, sqrt

import numpy as np
from numpy.polynomial import polynomial as npoly

from . import prism


def root_coeff(j, p):
    """j-th Taylor coefficient of (1 - xi)^{-1/p} at 0."""
    c = 1.0
    for i in range(j):
        c *= (1.0 / p + i) / (i + 1)
    return c


def map_coeffs(d, p):
    """Vectors A_0..A_p (increasing powers of xi, length p d + 2) with
    r(xi; alpha) = sum_i alpha^i A_i(xi), r = 1 - (1 - xi) (f + alpha xi^d)^p."""
    f = np.array([root_coeff(j, p) for j in range(d)], dtype=np.float64)
    om = np.array([1.0, -1.0])
    L = p * d + 2
    out = []
    for i in range(p + 1):
        fp = np.array([1.0])
        for _ in range(p - i):
            fp = npoly.polymul(fp, f)
        xdi = np.zeros(d * i + 1)
        xdi[d * i] = 1.0
        a = -comb(p, i) * npoly.polymul(om, npoly.polymul(fp, xdi))
        if i == 0:
            a = npoly.polyadd([1.0], a)
        v = np.zeros(L)
        v[: len(a)] = a
        out.append(v)
    return out


def residual_map(xi, alpha, d, p):
    """r(xi; alpha) from the coefficient vectors."""
    A = map_coeffs(d, p)
    c = sum(alpha ** i * A[i] for i in range(p + 1))
    return npoly.polyval(np.asarray(xi, np.float64), c)


def objective(M, d, p):
    """Coefficients w_0..w_{2p} of phi(alpha) = c(alpha)^T M c(alpha),
    c(alpha) = sum_i alpha^i A_i, M the Gram matrix of K_0..K_{p d + 1}."""
    A = map_coeffs(d, p)
    M = np.asarray(M, np.float64)
    w = np.zeros(2 * p + 1)
    for i in range(p + 1):
        for j in range(p + 1):
            w[i + j] += float(A[i] @ M @ A[j])
    return w


def fit_alpha(M, d, p, lo, hi):
    """argmin over [lo, hi] of phi: candidates lo, hi and the real roots of
    phi' inside; the smallest phi wins, ties to the smaller alpha.  A
    degenerate or non-finite objective gives b_d."""
    w = objective(M, d, p)
    bd = root_coeff(d, p)
    if not np.all(np.isfinite(w)) or np.max(np.abs(w[1:])) <= 1e-300:
        return min(max(bd, lo), hi)
    if hi <= lo:
        return lo
    phi = lambda a: float(npoly.polyval(a, w))
    cands = [lo, hi]
    dw = npoly.polyder(w)
    scale = np.max(np.abs(dw))
    if scale > 0:
        dw = dw / scale
        while len(dw) > 1 and dw[-1] == 0.0:
            dw = dw[:-1]
        if len(dw) >= 2:
            for root in npoly.polyroots(dw):
                if abs(root.imag) <= 1e-9 * max(1.0, abs(root.real)):
                    a = float(root.real)
                    if lo < a < hi:
                        cands.append(a)
    cands.sort()
    vals = [phi(a) for a in cands]
    best = min(range(len(cands)), key=lambda i: (vals[i], cands[i]))
    return float(cands[best])


# hi of the interval rule for p = 4 (oracle.interval.upper_bound with this
# map): d = 1 gives 1/2 exactly (the linear term 1 - 4 alpha binds, as 1 - 2
# alpha gives the page's 1 for the square root); d = 2 gives 0.6039, rounded
# down to two decimals
_HI4 = {1: 0.5, 2: 0.60}


def default_interval(d, p):
    if p == 2:
        return prism.default_interval(d)
    if p == 4 and d in _HI4:
        return root_coeff(d, 4), _HI4[d]
    raise ValueError("p must be 2 or 4 and d 1 or 2")


def krylov_gram(R, S, J):
    """Gram matrix of K_j = R^j S, j = 0..J."""
    K = [np.asarray(S, np.float64)]
    for _ in range(J):
        K.append(R @ K[-1])
    Kf = np.stack([k.reshape(-1) for k in K])
    return Kf @ Kf.T


def inv_root(A, p=4, d=2, lo=None, hi=None, tol=1e-6, max_iter=30, sketch_fn=None,
             accelerate=True, scale="frobenius"):
    """A^{-1/p} and A^{1/p} by the PRISM coupled inverse Newton iteration, on
    A / c with c from prism.input_scale.
    Returns (X, X_aux, info) with info = dict(status, stages=[StageTrace], c)."""
    A = np.asarray(A, np.float64)
    n = A.shape[0]
    if lo is None or hi is None:
        lo, hi = default_interval(d, p)
    if sketch_fn is None:
        sketch_fn = prism.make_sketch_fn(0)
    tr = prism.StageTrace()
    c = prism.input_scale(A, scale, sketch_fn)
    if not np.isfinite(c) or c == 0.0:
        tr.status = prism.NONFINITE
        nan = np.full((n, n), np.nan)
        return nan, nan, dict(status=prism.NONFINITE, stages=[tr], c=c)
    I = np.eye(n)
    M = A / c
    X = I.copy()
    R = I - M
    k = 0
    J = p * d + 1
    while True:
        r = float(np.linalg.norm(R) / sqrt(n))
        tr.r.append(r)
        st = prism._check(tr, r, k, max_iter, tol)
        if st is not None:
            tr.status = st
            break
        if accelerate:
            S = sketch_fn(0, k, n)
            tr.sketch_products += J
            alpha = fit_alpha(krylov_gram(R, S, J), d, p, lo, hi)
        else:
            alpha = root_coeff(d, p)
        tr.alpha.append(alpha)
        tr.degree.append(d)
        g = sum(root_coeff(j, p) * np.linalg.matrix_power(R, j) for j in range(d))
        g = g + alpha * np.linalg.matrix_power(R, d)
        tr.gemms += d - 1                      # R^2 .. R^d
        gp = g
        for _ in range(int(round(np.log2(p)))):
            gp = gp @ gp                       # g^2, g^4
            tr.gemms += 1
        X = g if k == 0 else X @ g             # X_0 = I: the first update is free
        tr.gemms += 0 if k == 0 else 1
        M = gp @ M
        tr.gemms += 1
        R = I - M
        k += 1
    tr.iters = k
    Xs = X * c ** (-1.0 / p)
    aux = (c ** (1.0 / p)) * (A / c) @ np.linalg.matrix_power(X, p - 1)
    return Xs, aux, dict(status=tr.status, stages=[tr], c=c)
