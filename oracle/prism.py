"""Step-by-step fp64 PRISM Newton-Schulz iterations (CPU reference).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows the [PRISM synthesis]:
  Part I  -- the matrix function is computed by an iterative polynomial
             approximation X_{k+1} = X_k f_d(R_k), R_k a residual matrix (for
             sign-type functions I - X_k^2), f_d the degree-d Taylor
             polynomial of the residual function at xi = 0.
  Part II.1 -- the top Taylor coefficient is replaced by alpha:
             g_d(xi; alpha) = f_{d-1}(xi) + alpha xi^d, alpha_k minimises the
             Frobenius norm of the next residual and is confined to [lo, hi]
             (the page gives [1/2, 1] for d = 1).
  Part II.2 -- the minimisation is done on a Gaussian sketch of the residual.

Readings taken where the pages are silent (the same readings the GPU library
implements; every one is listed in the design notes):
  * residual function: for the square-root family f(xi) = (1 - xi)^{-1/2}, with
    Taylor coefficients c_j = binom(2j, j) / 4^j;
  * coupled square root: R_k = I - Z_k Y_k, Y_{k+1} = Y_k g, Z_{k+1} = g Z_k
    (Y -> A^{1/2}, Z -> A^{-1/2} after scaling A by c = ||A||_F);
  * polar factor: R_k = I - X_k^T X_k, X_{k+1} = X_k g (X_0 = G / ||G||_F);
  * inverse 4th root: a second coupled square-root stage started from the
    first stage's Y (eigenvalues already in (0, 1], no rescaling);
  * in exact arithmetic R_{k+1} = r(R_k; alpha) with
    r(xi; alpha) = 1 - (1 - xi) g(xi; alpha)^2, so the sketched objective is
    phi_S(alpha) = || r(R_k; alpha) S ||_F^2, a quartic in alpha whose
    coefficients come from the Gram matrix of K_j = R_k^j S;
  * alpha_k = argmin of phi_S over [lo, hi] (candidates: both ends and the real
    critical points inside); default [lo, hi] = [1/2, 1] for d = 1,
    [3/8, 1.47] for d = 2 and [5/16, 2.46] for d = 3 (see oracle.interval);
  * stopping: r_k = ||R_k||_F / sqrt(n) <= tol; stagnation when r_{k-1} < 1e-2
    and r_k > 0.9 r_{k-1}; divergence when r_k > 2; max_iter updates at most;
  * adaptive degree ([PRISM summary], methodology step 3: the degree is raised
    only when the sketched residual shows it is needed): a stage starts at
    degree d; after alpha_k is fitted, the sketch predicts the contraction of
    the update, q_k = sqrt(phi_S(alpha_k)) / ||R_k S||_F (phi_S(alpha_k) is the
    sketched ||R_{k+1} S||_F^2); when q_k > adapt_ratio and d < degree_max the
    following updates of the stage use d + 1.  The update k itself keeps d.
"""
from math import comb, sqrt

import numpy as np
from numpy.polynomial import polynomial as npoly

from . import philox

# numerical outcome codes (same values as the C header's pmx_numeric)
CONVERGED, MAXITER, STAGNATED, NONFINITE, DIVERGED = 0, 1, 2, 3, 4
_SEVERITY = {CONVERGED: 0, STAGNATED: 1, MAXITER: 2, DIVERGED: 3, NONFINITE: 4}

DIVERGE_LEVEL = 2.0
STAG_LEVEL = 1e-2
STAG_FACTOR = 0.9


def taylor_coeff(j):
    """j-th Taylor coefficient of (1 - xi)^{-1/2} at xi = 0: binom(2j, j) / 4^j."""
    return comb(2 * j, j) / 4.0 ** j


def default_interval(d):
    """[lo, hi] for the adaptive coefficient ([PRISM synthesis] Part II.1 gives
    [1/2, 1] for d = 1; for d = 2 and d = 3 the same rule, see oracle.interval:
    lo = c_d and hi = the rule's bound (1.4722, 2.4686) rounded down to two
    decimals)."""
    if d == 1:
        return 0.5, 1.0
    if d == 2:
        return 0.375, 1.47
    if d == 3:
        return 0.3125, 2.46
    raise ValueError("degree must be 1, 2 or 3")


def map_coeffs(d):
    """Coefficient vectors a0, a1, a2 (length 2d + 2, increasing powers of xi)
    with r(xi; alpha) = sum_j (a0_j + alpha a1_j + alpha^2 a2_j) xi^j, where
    r = 1 - (1 - xi) (f_{d-1} + alpha xi^d)^2."""
    f = np.array([taylor_coeff(j) for j in range(d)], dtype=np.float64)
    one_minus = np.array([1.0, -1.0])
    xd = np.zeros(d + 1)
    xd[d] = 1.0
    x2d = np.zeros(2 * d + 1)
    x2d[2 * d] = 1.0
    A0 = npoly.polysub([1.0], npoly.polymul(one_minus, npoly.polymul(f, f)))
    A1 = -2.0 * npoly.polymul(one_minus, npoly.polymul(f, xd))
    A2 = -1.0 * npoly.polymul(one_minus, x2d)
    L = 2 * d + 2

    def pad(a):
        out = np.zeros(L)
        out[: len(a)] = a
        return out

    return pad(A0), pad(A1), pad(A2)


def residual_map(xi, alpha, d):
    """r(xi; alpha) evaluated from the coefficient vectors."""
    a0, a1, a2 = map_coeffs(d)
    return npoly.polyval(np.asarray(xi, np.float64), a0 + alpha * a1 + alpha * alpha * a2)


def quartic(M, d):
    """Coefficients w0..w4 of phi(alpha) = c(alpha)^T M c(alpha),
    c(alpha) = a0 + alpha a1 + alpha^2 a2, M the (2d+2) x (2d+2) Gram matrix of
    K_0..K_{2d+1}."""
    a0, a1, a2 = map_coeffs(d)
    M = np.asarray(M, np.float64)
    q = lambda x, y: float(x @ M @ y)
    return np.array([
        q(a0, a0),
        q(a0, a1) + q(a1, a0),
        q(a1, a1) + q(a0, a2) + q(a2, a0),
        q(a1, a2) + q(a2, a1),
        q(a2, a2),
    ])


def fit_alpha(M, d, lo, hi):
    """alpha = argmin over [lo, hi] of the quartic phi built from the Gram
    matrix M ([PRISM synthesis] Part II.1).  Candidates are lo, hi and the real
    roots of phi' inside (lo, hi); the smallest phi wins, ties to the smaller
    alpha.  A degenerate or non-finite quartic gives the Taylor coefficient."""
    w = quartic(M, d)
    cd = taylor_coeff(d)
    if not np.all(np.isfinite(w)) or np.max(np.abs(w[1:])) <= 1e-300:
        return min(max(cd, lo), hi)
    if hi <= lo:
        return lo
    phi = lambda a: w[0] + a * (w[1] + a * (w[2] + a * (w[3] + a * w[4])))
    cands = [lo, hi]
    deriv = [4 * w[4], 3 * w[3], 2 * w[2], w[1]]  # highest power first
    scale = max(abs(c) for c in deriv)
    deriv = [c / scale for c in deriv]
    while deriv and deriv[0] == 0.0:
        deriv = deriv[1:]
    if len(deriv) >= 2:
        for root in np.roots(deriv):
            if abs(root.imag) <= 1e-9 * max(1.0, abs(root.real)):
                a = float(root.real)
                if lo < a < hi:
                    cands.append(a)
    cands.sort()
    vals = [phi(a) for a in cands]
    best = min(range(len(cands)), key=lambda i: (vals[i], cands[i]))
    return float(cands[best])


def krylov_gram(R, S, d):
    """K_j = R^j S for j = 0..2d+1 and their Gram matrix M_ab = <K_a, K_b>_F
    ([PRISM synthesis] Part II.2: the least-squares problem on a sketch)."""
    K = [np.asarray(S, np.float64)]
    for _ in range(2 * d + 1):
        K.append(R @ K[-1])
    L = len(K)
    M = np.empty((L, L))
    for a in range(L):
        for b in range(L):
            M[a, b] = float(np.sum(K[a] * K[b]))
    return M


def predicted_contraction(M, d, alpha):
    """q = sqrt(phi_S(alpha)) / ||R S||_F from the Gram matrix of K_0..K_{2d+1}
    (M[1, 1] = ||R S||_F^2): the sketch's estimate of ||R_{k+1}|| / ||R_k||."""
    w = quartic(M, d)
    phi = w[0] + alpha * (w[1] + alpha * (w[2] + alpha * (w[3] + alpha * w[4])))
    m11 = float(M[1, 1])
    return sqrt(max(phi, 0.0) / m11) if m11 > 0.0 else 0.0


class StageTrace:
    """Per-stage record: r_k at the start of every iteration, alpha_k and the
    degree used by every update, number of updates, dense and sketch products,
    status."""

    def __init__(self):
        self.r = []
        self.alpha = []
        self.degree = []
        self.q = []
        self.iters = 0
        self.gemms = 0
        self.sketch_products = 0
        self.status = None


def _check(trace, r, k, max_iter, tol):
    """Stopping rule; returns a status code or None to continue."""
    if not np.isfinite(r):
        return NONFINITE
    if r <= tol:
        return CONVERGED
    if r > DIVERGE_LEVEL:
        return DIVERGED
    if k >= 1 and trace.r[-2] < STAG_LEVEL and r > STAG_FACTOR * trace.r[-2]:
        return STAGNATED
    if k >= max_iter:
        return MAXITER
    return None


def _poly_g(R, alpha, d, trace):
    """g = f_{d-1}(R) + alpha R^d; counts the dense products R^2..R^d."""
    n = R.shape[0]
    g = np.eye(n) * taylor_coeff(0)
    P = np.eye(n)
    for j in range(1, d + 1):
        if j == 1:
            P = R.copy()
        else:
            P = P @ R
            trace.gemms += 1
        g = g + (alpha if j == d else taylor_coeff(j)) * P
    return g


def _alpha_for(R, d, lo, hi, accelerate, sketch_fn, stage, k, trace):
    if not accelerate:
        return taylor_coeff(d)
    S = sketch_fn(stage, k, R.shape[0])
    trace.sketch_products += 2 * d + 1
    M = krylov_gram(R, S, d)
    alpha = fit_alpha(M, d, lo, hi)
    trace.q.append(predicted_contraction(M, d, alpha))
    return alpha


class DegreeRule:
    """Degree of each update of a stage: fixed at d, or (degree_max > d)
    raised by one after an update whose predicted contraction exceeds
    adapt_ratio.  Intervals: the given [lo, hi] for the starting degree, the
    default interval of every raised degree."""

    def __init__(self, d, lo, hi, degree_max=None, adapt_ratio=0.3):
        self.d = d
        self.dmax = d if degree_max is None else max(d, degree_max)
        self.ratio = adapt_ratio
        self.lo0, self.hi0 = (lo, hi) if lo is not None and hi is not None else default_interval(d)

    def interval(self, d):
        return (self.lo0, self.hi0) if d == self.d else default_interval(d)

    def next(self, d, q):
        return d + 1 if (d < self.dmax and q > self.ratio) else d


def coupled_sqrt_stage(Y0, d=2, lo=None, hi=None, tol=1e-6, max_iter=30,
                       sketch_fn=None, stage=0, accelerate=True, degree_max=None,
                       adapt_ratio=0.3):
    """One coupled Newton-Schulz square-root stage from Y_0 (Z_0 = I).
    Y_0 must have its spectrum in (0, 1].  Returns (Y, Z, StageTrace)
    with Y -> Y_0^{1/2}, Z -> Y_0^{-1/2}.  degree_max > d: adaptive degree."""
    rule = DegreeRule(d, lo, hi, degree_max, adapt_ratio)
    Y0 = np.asarray(Y0, np.float64)
    n = Y0.shape[0]
    I = np.eye(n)
    Y = Y0.copy()
    Z = I.copy()
    R = I - Y  # Z_0 Y_0 = Y_0: no product
    tr = StageTrace()
    k = 0
    while True:
        r = float(np.linalg.norm(R) / sqrt(n))
        tr.r.append(r)
        st = _check(tr, r, k, max_iter, tol)
        if st is not None:
            tr.status = st
            break
        lo, hi = rule.interval(d)
        alpha = _alpha_for(R, d, lo, hi, accelerate, sketch_fn, stage, k, tr)
        tr.alpha.append(alpha)
        tr.degree.append(d)
        g = _poly_g(R, alpha, d, tr)
        if accelerate:
            d = rule.next(d, tr.q[-1])
        Y = Y @ g
        tr.gemms += 1
        if k == 0:
            Z = g  # g Z_0 = g
        else:
            Z = g @ Z
            tr.gemms += 1
        R = I - Z @ Y
        tr.gemms += 1
        k += 1
    tr.iters = k
    return Y, Z, tr


def _worst(a, b):
    return a if _SEVERITY[a] >= _SEVERITY[b] else b


def make_sketch_fn(seed, b=0, p=8):
    """Gaussian sketch provider for matrix b of a batch (oracle.philox)."""
    return lambda stage, k, n: philox.sketch(seed, b, stage, k, n, p)


def exact_sketch_fn():
    """S = I_n: phi_S becomes the exact objective ||I - X_{k+1}^2||_F^2."""
    return lambda stage, k, n: np.eye(n)


# The power estimate of the input scale (an option; the pages leave the
# scaling open): the start block is the sketch of stage POWER_STAGE, k = 0.
POWER_STAGE, POWER_PASSES, POWER_FACTOR = 2, 8, 2.0


def power_scale(A, c, V0, passes=POWER_PASSES, factor=POWER_FACTOR):
    """c * min(1, factor * mu) with mu = max_j ||K_t[:, j]|| / ||K_{t-1}[:, j]||,
    K_0 = V0 and K_t = (A / c) K_{t-1} for t = 1..passes.  Every ratio is at
    most the spectral norm of A / c (||M x|| <= ||M||_2 ||x||), so the result
    never exceeds c and stays at most factor * lambda_max; zero or non-finite
    ratios leave c unchanged."""
    M = np.asarray(A, np.float64) / c
    prev, K = None, np.asarray(V0, np.float64)
    for _ in range(passes):
        prev, K = K, M @ K
    n0 = np.linalg.norm(prev, axis=0)
    n1 = np.linalg.norm(K, axis=0)
    ok = (n0 > 0) & np.isfinite(n0) & np.isfinite(n1)
    if not np.any(ok):
        return c
    mu = float(np.max(n1[ok] / n0[ok]))
    if not (mu > 0.0) or not np.isfinite(mu):
        return c
    return c * min(1.0, factor * mu)


def input_scale(A, scale, sketch_fn):
    """The scale c of Y_0 = A / c: ||A||_F ("frobenius") or its power estimate
    ("power", start block sketch_fn(POWER_STAGE, 0, n))."""
    c = float(np.linalg.norm(A))
    if scale == "power" and np.isfinite(c) and c > 0.0:
        c = power_scale(A, c, sketch_fn(POWER_STAGE, 0, A.shape[0]))
    elif scale not in ("frobenius", "power"):
        raise ValueError("scale must be 'frobenius' or 'power'")
    return c


def inv_root(A, p=2, d=2, lo=None, hi=None, tol=1e-6, max_iter=30,
             sketch_fn=None, accelerate=True, degree_max=None, adapt_ratio=0.3,
             scale="frobenius"):
    """PRISM A^{-1/p} (p in {2, 4}) with the auxiliary A^{1/p}.
    Scaling c = ||A||_F (or its power estimate, input_scale), stage 1 on
    A / c; for p = 4 stage 2 on stage 1's Y.
    Returns (X, X_aux, info) with info = dict(status, stages=[StageTrace...], c)."""
    A = np.asarray(A, np.float64)
    if sketch_fn is None:
        sketch_fn = make_sketch_fn(0)
    c = input_scale(A, scale, sketch_fn)
    if not np.isfinite(c) or c == 0.0:
        n = A.shape[0]
        nan = np.full((n, n), np.nan)
        t = StageTrace()
        t.status = NONFINITE
        return nan, nan, dict(status=NONFINITE, stages=[t], c=c)
    Y, Z, t1 = coupled_sqrt_stage(A / c, d, lo, hi, tol, max_iter, sketch_fn, 0, accelerate,
                                  degree_max, adapt_ratio)
    stages = [t1]
    status = t1.status
    if p == 2:
        return Z / sqrt(c), Y * sqrt(c), dict(status=status, stages=stages, c=c)
    if p != 4:
        raise ValueError("p must be 2 or 4")
    if status in (NONFINITE, DIVERGED):
        return Z * np.nan, Y * np.nan, dict(status=status, stages=stages, c=c)
    Y2, Z2, t2 = coupled_sqrt_stage(Y, d, lo, hi, tol, max_iter, sketch_fn, 1, accelerate,
                                    degree_max, adapt_ratio)
    stages.append(t2)
    status = _worst(status, t2.status)
    return Z2 * c ** -0.25, Y2 * c ** 0.25, dict(status=status, stages=stages, c=c)


def polar_power_scale(R0, V0, passes=POWER_PASSES, factor=POWER_FACTOR):
    """s with s^2 = min(1, factor mu), mu the largest column growth ratio of
    K_t = (I - R0) K_{t-1} = X0^T X0 K_{t-1} from K_0 = V0 (power_scale on
    X0^T X0 with c = 1): X0 / s has its top singular value at most 1 once mu
    reaches half of the top eigenvalue of X0^T X0."""
    M = np.eye(R0.shape[0]) - np.asarray(R0, np.float64)
    return sqrt(power_scale(M, 1.0, V0, passes, factor))


def polar(G, d=2, lo=None, hi=None, tol=1e-6, max_iter=30, sketch_fn=None,
          accelerate=True, degree_max=None, adapt_ratio=0.3, scale="frobenius"):
    """PRISM polar factor of G (m x n).  Wide inputs are handled through G^T.
    R_k = I - X_k^T X_k, X_{k+1} = X_k g.  X_0 = G / c with c = ||G||_F; with
    scale="power" X_0 is then divided by s = polar_power_scale(R_0, V_0)
    (V_0 the sketch of stage POWER_STAGE), c becomes c s and R_0 is formed
    again.  Returns (U, info)."""
    G = np.asarray(G, np.float64)
    if scale not in ("frobenius", "power"):
        raise ValueError("scale must be 'frobenius' or 'power'")
    if G.shape[0] < G.shape[1]:
        U, info = polar(G.T, d, lo, hi, tol, max_iter, sketch_fn, accelerate, degree_max,
                        adapt_ratio, scale)
        return U.T, info
    rule = DegreeRule(d, lo, hi, degree_max, adapt_ratio)
    if sketch_fn is None:
        sketch_fn = make_sketch_fn(0)
    m, n = G.shape
    tr = StageTrace()
    c = float(np.linalg.norm(G))
    if not np.isfinite(c) or c == 0.0:
        tr.status = NONFINITE
        return np.full_like(G, np.nan), dict(status=NONFINITE, stages=[tr], c=c)
    I = np.eye(n)
    X = G / c
    R = I - X.T @ X
    tr.gemms += 1
    if scale == "power":
        sc = polar_power_scale(R, sketch_fn(POWER_STAGE, 0, n))
        if sc < 1.0:
            X = X / sc
            R = I - X.T @ X
            c *= sc
    k = 0
    while True:
        r = float(np.linalg.norm(R) / sqrt(n))
        tr.r.append(r)
        st = _check(tr, r, k, max_iter, tol)
        if st is not None:
            tr.status = st
            break
        lo, hi = rule.interval(d)
        alpha = _alpha_for(R, d, lo, hi, accelerate, sketch_fn, 0, k, tr)
        tr.alpha.append(alpha)
        tr.degree.append(d)
        g = _poly_g(R, alpha, d, tr)
        if accelerate:
            d = rule.next(d, tr.q[-1])
        X = X @ g
        tr.gemms += 1
        R = I - X.T @ X
        tr.gemms += 1
        k += 1
    tr.iters = k
    return X, dict(status=tr.status, stages=[tr], c=c)
