"""A whole Shampoo step over the layers of a model (CPU, fp64).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows the [Shampoo blog]: the update of section 2.3 (statistics EMA with
+eps I, inverse 4th roots, W <- W - eta L^{-1/4} G R^{-1/4}), the
block-diagonal approximation of section 3.2, the adaptive learning rate of
section 5.1 (eta_t = eta_0 / sqrt(1 + sum_{i <= t} ||G_i||^2)), momentum of
section 5.2 (M_t = gamma M_{t-1} + P_t, W <- W - eta M_t) and the
convolution reshape of section 5.3 (a c_out x c_in x h x w kernel as the
(c_out h w) x c_in matrix).  Readings: every block of at most B x B of a
layer's matrix view is a parameter of its own (its own L, R, M; blocks cut
row-wise then column-wise from the top left); the roots are recomputed when
t % root_every == 0 and kept otherwise (L^{-1/4} = R^{-1/4} = I before the
first); the gradient norm of 5.1 is summed over all layers.  Roots are the
closed forms (eigendecomposition) of oracle.closed_form.
"""
import numpy as np

from . import closed_form as cf


def matrix_view(x):
    """The matrix a layer's tensor is preconditioned as."""
    x = np.asarray(x)
    if x.ndim == 2:
        return x
    co, ci, h, w = x.shape
    return x.transpose(0, 2, 3, 1).reshape(co * h * w, ci)


def from_matrix_view(m, shape):
    if len(shape) == 2:
        return m.reshape(shape)
    co, ci, h, w = shape
    return m.reshape(co, h, w, ci).transpose(0, 3, 1, 2)


class ShampooState:
    """Per-block statistics, roots and momentum for a list of layer shapes."""

    def __init__(self, shapes, block, eps):
        self.shapes = [tuple(s) for s in shapes]
        self.block = block
        self.blocks = []  # (layer, r0, c0, rows, cols)
        for l, s in enumerate(self.shapes):
            rows, cols = matrix_view(np.zeros(s)).shape
            for r0 in range(0, rows, block):
                for c0 in range(0, cols, block):
                    self.blocks.append((l, r0, c0, min(block, rows - r0), min(block, cols - c0)))
        self.L = [eps * np.eye(b[3]) for b in self.blocks]
        self.R = [eps * np.eye(b[4]) for b in self.blocks]
        self.Li = [np.eye(b[3]) for b in self.blocks]
        self.Ri = [np.eye(b[4]) for b in self.blocks]
        self.M = [np.zeros((b[3], b[4])) for b in self.blocks]
        self.norm_sum = 0.0


def step(state, Ws, Gs, t, beta, eps, lr, momentum=0.0, root_every=1, adaptive_lr=False):
    """One step; returns the new weights (fp64 arrays in the layers' shapes)."""
    Gm = [matrix_view(np.asarray(g, np.float64)) for g in Gs]
    Wm = [matrix_view(np.asarray(w, np.float64)).copy() for w in Ws]
    eta = lr
    if adaptive_lr:
        state.norm_sum += sum(float(np.sum(g * g)) for g in Gm)
        eta = lr / np.sqrt(1.0 + state.norm_sum)
    for i, (l, r0, c0, m, n) in enumerate(state.blocks):
        G = Gm[l][r0:r0 + m, c0:c0 + n]
        state.L[i], state.R[i] = cf.stats_update(state.L[i], state.R[i], G, beta, eps)
        if t % root_every == 0:
            state.Li[i] = cf.inv_root(state.L[i], 4)[0]
            state.Ri[i] = cf.inv_root(state.R[i], 4)[0]
        P = state.Li[i] @ G @ state.Ri[i]
        state.M[i] = momentum * state.M[i] + P if momentum != 0.0 else P
        Wm[l][r0:r0 + m, c0:c0 + n] -= eta * state.M[i]
    return [from_matrix_view(w, s) for w, s in zip(Wm, state.shapes)]
