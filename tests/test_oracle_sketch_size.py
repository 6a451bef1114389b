"""How the sketch width p decides the fitted alpha (oracle study, CPU).

The [PRISM synthesis] Part II.2 ("Randomized Sketching") replaces the exact
least-squares fit of alpha by its restriction to a Gaussian sketch S (n x p)
and argues that p = O(log n) keeps the convergence of the exact fit; the
[PRISM summary] ("局限性与未来工作") names the sensitivity to the sketch size as
the method's main limitation.  Along a sketched coupled square-root stage of
the oracle, every update's alpha from a sketch of width p is compared with the
exact fit on the same residual (S = I, the objective ||I - X_{k+1}^2||_F^2 of
Part II.1), for p = 2 .. 32, on three spectra of order 256: the power law of
the blocked-Shampoo workload (kappa = 1e6), a damped Shampoo statistic
(G G^T / m + eps I) and the Marchenko-Pastur spectrum of the 10^4 square
root (ratio 1/2).  Pins: the alpha error shrinks as p grows (it is a sample
of a least-squares fit: its spread falls roughly as 1 / sqrt(p)); with
p >= 8 the update count equals the exact fit's within one.
"""
import numpy as np
import pytest

import workloads as W
from oracle import prism


def _spectra(n=256):
    rng = np.random.default_rng(1234)
    out = {}
    A, _, _ = W.spd_power_batch(1, n, 77)
    out["power law (kappa 1e6)"] = A[0].astype(np.float64)
    G = rng.standard_normal((n, 4 * n))
    out["Shampoo statistic"] = G @ G.T / (4 * n) + 1e-6 * np.eye(n)
    Wm = rng.standard_normal((n, 2 * n))
    out["Marchenko-Pastur 1/2"] = Wm @ Wm.T / (2 * n) + 1e-4 * np.eye(n)
    return out


def _stage(A, d, sketch, exact_too, max_iter=40, tol=1e-6):
    """One sketched coupled square-root stage of A / ||A||_F; returns the
    update count and the per-update (alpha_S, alpha_exact, r_k)."""
    n = A.shape[0]
    I = np.eye(n)
    lo, hi = prism.default_interval(d)
    Y = A / np.linalg.norm(A)
    Z = I.copy()
    R = I - Y
    recs = []
    for k in range(max_iter):
        r = float(np.linalg.norm(R) / np.sqrt(n))
        if r <= tol:
            return k, recs
        a_s = prism.fit_alpha(prism.krylov_gram(R, sketch(k, n), d), d, lo, hi)
        a_e = prism.fit_alpha(prism.krylov_gram(R, I, d), d, lo, hi) if exact_too else None
        recs.append((a_s, a_e, r))
        g = I + 0.5 * R + a_s * (R @ R)
        Y = Y @ g
        Z = g if k == 0 else g @ Z
        R = I - Z @ Y
    return max_iter, recs


@pytest.mark.slow
def test_alpha_error_shrinks_with_sketch_width(capsys):
    from oracle import philox
    ps = (2, 4, 8, 16, 32)
    seeds = tuple(range(8))
    table = {}
    for name, A in _spectra().items():
        exact_iters, _ = _stage(A, 2, lambda k, n: np.eye(n), False)
        for p in ps:
            errs, worst, iters = [], [], []
            for sd in seeds:
                it, recs = _stage(A, 2, lambda k, n: philox.sketch(sd, 0, 0, k, n, p), True)
                iters.append(it)
                # alpha is only determined while the residual is not tiny
                e = [abs(a - b) for a, b, r in recs if r >= 1e-3]
                errs.extend(e)
                worst.append(max(e) if e else 0.0)
            table[(name, p)] = (float(np.sqrt(np.mean(np.square(errs)))), float(np.max(worst)),
                                max(iters), exact_iters)
    with capsys.disabled():
        print("\nsketch width p: rms and max over updates (r_k >= 1e-3) and %d seeds of "
              "|alpha_S - alpha_exact|, worst update count (exact fit's)" % len(seeds))
        for (name, p), (e, w, it, ex) in table.items():
            print("  %-24s p=%-2d  alpha err rms %.3e max %.3e  updates %d (exact %d)"
                  % (name, p, e, w, it, ex))
    for name in _spectra():
        e = [table[(name, p)][0] for p in ps]
        assert e[-1] < e[0], name          # p = 32 fits closer than p = 2
        assert e[2] <= e[0] + 1e-12, name  # p = 8 no worse than p = 2
        for p in (8, 16, 32):
            _, _, it, ex = table[(name, p)]
            assert abs(it - ex) <= 1, (name, p)
