"""Closed-form definitions of what the path computes (fp64, CPU).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Every function takes the exact arrays handed to the GPU (fp32 or bf16 values,
upcast to fp64) and returns fp64 results.
"""
import numpy as np


def sym(a):
    """Symmetric part (A + A^T)/2; roots are defined for the symmetric input."""
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * (a + a.T)


def stats_update(L, R, G, beta, eps):
    """One Shampoo statistics update ([Shampoo blog] section 2.3, step 2):
    L <- beta L + (1-beta) G G^T + eps I,  R <- beta R + (1-beta) G^T G + eps I.
    """
    G = np.asarray(G, dtype=np.float64)
    L = np.asarray(L, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    m, n = G.shape
    Ln = beta * L + (1.0 - beta) * (G @ G.T) + eps * np.eye(m)
    Rn = beta * R + (1.0 - beta) * (G.T @ G) + eps * np.eye(n)
    return Ln, Rn


def stats_sequence(L0, R0, Gs, beta, eps):
    """Apply stats_update once per gradient in Gs, in order."""
    L, R = np.asarray(L0, np.float64), np.asarray(R0, np.float64)
    for G in Gs:
        L, R = stats_update(L, R, G, beta, eps)
    return L, R


def matrix_power_sym(A, expo):
    """A^expo for symmetric positive definite A via A = Q Lambda Q^T
    ([Shampoo blog] section 3.1: L^{-1/4} = Q Lambda^{-1/4} Q^T).
    Raises ValueError if the symmetric part is not positive definite."""
    w, Q = np.linalg.eigh(sym(A))
    if not np.all(w > 0):
        raise ValueError("matrix is not positive definite (min eigenvalue %g)" % w.min())
    return (Q * w ** expo) @ Q.T


def inv_root(A, p):
    """Returns (A^{-1/p}, A^{1/p}) for p in {2, 4}; the second is the auxiliary
    output (A^{1/2} for p = 2, A^{1/4} for p = 4)."""
    if p not in (2, 4):
        raise ValueError("p must be 2 or 4")
    w, Q = np.linalg.eigh(sym(A))
    if not np.all(w > 0):
        raise ValueError("matrix is not positive definite (min eigenvalue %g)" % w.min())
    return (Q * w ** (-1.0 / p)) @ Q.T, (Q * w ** (1.0 / p)) @ Q.T


def polar(G, rank_tol=None):
    """Polar factor of G (m x n): G = U_p H with U_p = U V^T from the thin SVD
    G = U Sigma V^T and H = V Sigma V^T.  For rank-deficient G the factor is the
    partial isometry sum over sigma_i > rank_tol of u_i v_i^T (a Newton-Schulz
    type iteration maps zero singular values to zero).  The [PRISM synthesis]
    lists the polar decomposition among the sign-type functions of Part I."""
    G = np.asarray(G, dtype=np.float64)
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    if rank_tol is None:
        rank_tol = max(G.shape) * np.finfo(np.float64).eps * (s.max() if s.size else 0.0)
    keep = s > rank_tol
    Up = (U[:, keep]) @ Vt[keep, :]
    H = (Vt.T * s) @ Vt
    return Up, H


def precond_apply(Linv, G, Rinv):
    """P = L^{-1/4} G R^{-1/4} ([Shampoo blog] section 2.3, step 4; section 2.1
    Kronecker identity (L (x) R) vec(X) = vec(L X R^T))."""
    return np.asarray(Linv, np.float64) @ np.asarray(G, np.float64) @ np.asarray(Rinv, np.float64)


def rel_fro(x, ref):
    """Relative Frobenius distance ||x - ref||_F / ||ref||_F."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))
