"""The PRISM iteration on a known spectrum (scalar eigenvalue model, fp64).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

In exact arithmetic, when the input is A = Q diag(lambda) Q^T, every residual
R_k of the coupled square-root iteration is Q diag(xi^(k)) Q^T, and
xi^(k+1) = r(xi^(k); alpha_k) with r(xi; alpha) = 1 - (1 - xi) g(xi; alpha)^2
([PRISM synthesis] Part I / Part II.1).  The sketched objective becomes
  phi_S(alpha) = sum_i w_i r(xi_i; alpha)^2,  w_i = || row_i(Q^T S) ||^2,
and the exact objective is the same with w_i = 1.  This module minimises that
sum directly (dense grid plus bounded Brent refinement), an independent route
to the quartic/polynomial-root solver in oracle.prism.
"""
from math import sqrt

import numpy as np
from scipy.optimize import minimize_scalar

from .prism import (CONVERGED, DIVERGE_LEVEL, DIVERGED, MAXITER, STAG_FACTOR,
                    STAG_LEVEL, STAGNATED, residual_map, taylor_coeff)


def argmin_alpha(xi, w, d, lo, hi, npts=2001, rmap=None):
    """argmin over [lo, hi] of sum_i w_i r(xi_i; alpha)^2."""
    xi = np.asarray(xi, np.float64)
    w = np.asarray(w, np.float64)
    if rmap is None:
        rmap = residual_map
    obj = lambda a: float(np.sum(w * rmap(xi, a, d) ** 2))
    grid = np.linspace(lo, hi, npts)
    vals = np.array([obj(a) for a in grid])
    i = int(np.argmin(vals))
    a, b = grid[max(i - 1, 0)], grid[min(i + 1, npts - 1)]
    res = minimize_scalar(obj, bounds=(a, b), method="bounded", options={"xatol": 1e-13})
    best = float(res.x) if res.fun <= vals[i] else float(grid[i])
    # the ends are candidates too
    for e in (lo, hi):
        if obj(e) < obj(best):
            best = e
    return best


def run(xi0, d, lo, hi, tol, max_iter, weights_fn=None, accelerate=True, degree_max=None,
        adapt_ratio=0.3, intervals=None, rmap=None, taylor=None):
    """Iterate the scalar map on the residual spectrum xi0 (eigenvalues of R_0).
    weights_fn(k) returns the weights w_i for iteration k (None: exact, w = 1).
    degree_max > d: after an update whose contraction of the weighted
    residual, sqrt(sum w r(xi)^2 / sum w xi^2), exceeds adapt_ratio the degree
    rises by one (intervals[d] gives the interval of each raised degree).
    rmap(xi, alpha, d) replaces the square-root family's residual map and
    taylor(d) its Taylor coefficient (another iteration family).
    Returns dict(iters, status, r, alpha, degree)."""
    if rmap is None:
        rmap = residual_map
    if taylor is None:
        taylor = taylor_coeff
    xi = np.asarray(xi0, np.float64).copy()
    n = xi.size
    rs, alphas, degrees = [], [], []
    dmax = d if degree_max is None else degree_max
    k = 0
    while True:
        r = sqrt(float(np.sum(xi * xi)) / n)
        rs.append(r)
        if r <= tol:
            status = CONVERGED
            break
        if r > DIVERGE_LEVEL:
            status = DIVERGED
            break
        if k >= 1 and rs[-2] < STAG_LEVEL and r > STAG_FACTOR * rs[-2]:
            status = STAGNATED
            break
        if k >= max_iter:
            status = MAXITER
            break
        w = np.ones(n) if weights_fn is None else weights_fn(k)
        if accelerate:
            alpha = argmin_alpha(xi, w, d, lo, hi, rmap=rmap)
        else:
            alpha = taylor(d)
        alphas.append(alpha)
        degrees.append(d)
        nxt = rmap(xi, alpha, d)
        if accelerate and d < dmax:
            q = sqrt(float(np.sum(w * nxt * nxt)) / float(np.sum(w * xi * xi)))
            if q > adapt_ratio:
                d += 1
                lo, hi = intervals[d]
        xi = nxt
        k += 1
    return dict(iters=k, status=status, r=rs, alpha=alphas, degree=degrees)


def products_sqrt_stage(iters, d):
    """Dense products of one coupled square-root stage with `iters` updates:
    the first update needs no g Z_0 product (Z_0 = I)."""
    if iters == 0:
        return 0
    per = d + 2  # (d-1) powers of R, Y g, g Z, Z Y
    return per * iters - 1


def products_polar(iters, d):
    """Dense products of the polar iteration: the initial X^T X plus, per
    update, (d-1) powers of R, X g and X^T X."""
    return 1 + (d + 1) * iters
