"""The [lo, hi] rule for the adaptive coefficient alpha (CPU, fp64).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The [PRISM synthesis] (Part II.1) confines alpha to a fixed interval and gives
[1/2, 1] for d = 1, but no interval for d = 2.  The reading used here:
lo = c_d (the Taylor coefficient, so alpha = lo is classical Newton-Schulz) and
hi = the largest u such that, for every alpha' in [lo, u],
  (i)  |r(xi; alpha')| <= xi for all xi in [0, 1]  (no residual eigenvalue grows), and
  (ii) with m = min(0, min_{xi in [0,1]} r(xi; alpha')) the reachable interval
       [m, 1] is mapped into itself by r(.; alpha').
Applied to d = 1 the rule gives u = 1 exactly, the page's interval; for d = 2 it
gives u ~= 1.4722.
"""
import numpy as np
from scipy.optimize import minimize_scalar

from .prism import residual_map, taylor_coeff


def _extreme(f, lo, hi, npts=4001):
    """min of f over [lo, hi]: dense grid, then bounded Brent around the best
    grid point."""
    xs = np.linspace(lo, hi, npts)
    v = f(xs)
    i = int(np.argmin(v))
    a, b = xs[max(i - 1, 0)], xs[min(i + 1, npts - 1)]
    res = minimize_scalar(f, bounds=(a, b), method="bounded", options={"xatol": 1e-14})
    return min(float(res.fun), float(v.min()))


def admissible(alpha, d, tol=1e-9, rmap=None):
    """Conditions (i) and (ii) for one alpha.  rmap(xi, alpha) is the residual
    map (default: the square-root / polar family's r of degree d)."""
    if rmap is None:
        rmap = lambda x, a: residual_map(x, a, d)
    xs = np.linspace(1e-6, 1.0, 20001)
    r = rmap(xs, alpha)
    if np.any(np.abs(r) > xs * (1 + tol)):
        return False
    f = lambda x: rmap(x, alpha)
    m = min(0.0, _extreme(f, 0.0, 1.0))
    lo_img = _extreme(f, m, 1.0)
    hi_img = -_extreme(lambda x: -rmap(x, alpha), m, 1.0)
    return lo_img >= m - tol and hi_img <= 1.0 + tol


def upper_bound(d, top=3.0, iters=30, samples=100, rmap=None, lo=None):
    """Largest u (bisection to ~3e-9 relative) with every alpha' in [lo, u]
    admissible (checked on ``samples`` equally spaced alpha'); lo defaults to
    the square-root family's Taylor coefficient c_d."""
    if lo is None:
        lo = taylor_coeff(d)
    a, b = lo, top
    for _ in range(iters):
        mid = 0.5 * (a + b)
        if all(admissible(x, d, rmap=rmap) for x in np.linspace(lo, mid, samples)):
            a = mid
        else:
            b = mid
    return a
