"""Pins for the whole-step Shampoo reference (oracle.shampoo_step)."""
import numpy as np

from oracle import shampoo_step as ss


def test_conv_view_matches_the_page_index_map():
    # K'[(o h + y) w + x][i] = K[o][i][y][x]
    rng = np.random.default_rng(1)
    K = rng.standard_normal((3, 4, 2, 5))
    V = ss.matrix_view(K)
    assert V.shape == (3 * 2 * 5, 4)
    for o in range(3):
        for i in range(4):
            for y in range(2):
                for x in range(5):
                    assert V[(o * 2 + y) * 5 + x, i] == K[o, i, y, x]
    np.testing.assert_array_equal(ss.from_matrix_view(V, K.shape), K)


def _root4(A):
    # an independent route to A^{-1/4}: scipy's Schur-based fractional power
    # (not the eigendecomposition the oracle uses)
    from scipy.linalg import fractional_matrix_power
    return np.real(fractional_matrix_power(A, -0.25))


def test_one_block_is_the_dense_shampoo_update():
    # block >= the matrix: the step is W - lr L^{-1/4} G R^{-1/4} (the update
    # of the Shampoo page, section 2.3), checked with Schur-based roots and
    # the Kronecker form of section 2.1: vec_r(L G R) = (L (x) R^T) vec_r(G)
    # for row-major vectorisation
    rng = np.random.default_rng(2)
    W = rng.standard_normal((6, 9))
    Gs = [rng.standard_normal((6, 9)) for _ in range(3)]
    st = ss.ShampooState([(6, 9)], block=16, eps=1e-3)
    L, R = 1e-3 * np.eye(6), 1e-3 * np.eye(9)
    Wr = W.copy()
    for t, G in enumerate(Gs):
        W = ss.step(st, [W], [G], t, 0.9, 1e-3, 0.1)[0]
        L = 0.9 * L + 0.1 * np.einsum("ik,jk->ij", G, G) + 1e-3 * np.eye(6)
        R = 0.9 * R + 0.1 * np.einsum("ki,kj->ij", G, G) + 1e-3 * np.eye(9)
        P = (np.kron(_root4(L), _root4(R).T) @ G.reshape(-1)).reshape(6, 9)
        Wr = Wr - 0.1 * P
    np.testing.assert_allclose(W, Wr, atol=1e-9)


def test_blocks_are_independent_parameters():
    # a 2 x 2 grid of blocks equals four separate one-block problems
    rng = np.random.default_rng(3)
    W = rng.standard_normal((10, 7))
    Gs = [rng.standard_normal((10, 7)) for _ in range(2)]
    st = ss.ShampooState([(10, 7)], block=5, eps=1e-2)
    Wn = W.copy()
    for t, G in enumerate(Gs):
        Wn = ss.step(st, [Wn], [G], t, 0.8, 1e-2, 0.05)[0]
    for r0, c0 in ((0, 0), (0, 5), (5, 0), (5, 5)):
        sub = ss.ShampooState([(5, min(5, 7 - c0))], block=5, eps=1e-2)
        w = W[r0:r0 + 5, c0:c0 + 5].copy()
        for t, G in enumerate(Gs):
            w = ss.step(sub, [w], [G[r0:r0 + 5, c0:c0 + 5]], t, 0.8, 1e-2, 0.05)[0]
        np.testing.assert_allclose(Wn[r0:r0 + 5, c0:c0 + 5], w, atol=1e-12)


def test_momentum_and_stale_roots_and_adaptive_rate():
    # constant gradient, roots every 100 steps (only t = 0): P is the same
    # every step, so M_t = P (1 - g^{t+1}) / (1 - g) and
    # W_T = W_0 - eta sum_t M_t; the adaptive rate divides by
    # sqrt(1 + (t + 1) ||G||^2)
    rng = np.random.default_rng(4)
    G = rng.standard_normal((4, 3))
    W0 = rng.standard_normal((4, 3))
    st = ss.ShampooState([(4, 3)], block=8, eps=1e-2)
    W = W0.copy()
    for t in range(5):
        W = ss.step(st, [W], [G], t, 0.9, 1e-2, 0.1, momentum=0.5, root_every=100)[0]
    L1 = 0.9 * 1e-2 * np.eye(4) + 0.1 * G @ G.T + 1e-2 * np.eye(4)
    R1 = 0.9 * 1e-2 * np.eye(3) + 0.1 * G.T @ G + 1e-2 * np.eye(3)
    P = _root4(L1) @ G @ _root4(R1)
    expect = W0 - 0.1 * sum(P * (1 - 0.5 ** (t + 1)) / 0.5 for t in range(5))
    np.testing.assert_allclose(W, expect, atol=1e-10)
    st2 = ss.ShampooState([(4, 3)], block=8, eps=1e-2)
    W = W0.copy()
    for t in range(3):
        W = ss.step(st2, [W], [G], t, 0.9, 1e-2, 0.1, root_every=100, adaptive_lr=True)[0]
    g2 = float(np.sum(G * G))
    expect = W0 - sum(0.1 / np.sqrt(1 + (t + 1) * g2) for t in range(3)) * P
    np.testing.assert_allclose(W, expect, atol=1e-10)
