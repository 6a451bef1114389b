"""Philox4x32-10 and the Gaussian sketch it defines (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11): a 4x32-bit counter and
a 2x32-bit key go through ten rounds; each round multiplies counter words 0 and
2 by two fixed odd constants, keeps the high and low halves of the 64-bit
products, and mixes the high halves with the other two counter words and the
key; between rounds the key is advanced by two Weyl constants.

The sketch S (n x p, row-major) for matrix ``b`` of a batch, iteration stage
``stage`` and iteration ``k`` is defined here (the [PRISM synthesis], Part II
"Randomized Sketching", asks only for a Gaussian oblivious subspace embedding;
the counter layout is this library's own choice):
  element e = i*p + j  ->  Philox call q = e // 4, output word w = e % 4,
  counter = (q, k, stage, b), key = (seed mod 2^32, seed >> 32).
  uniform u_w = ((x_w >> 8) + 1/2) * 2^-24, in (0, 1).
  Box-Muller on the pairs (u0, u1) and (u2, u3):
    z0 = sqrt(-2 ln u0) cos(2 pi u1), z1 = sqrt(-2 ln u0) sin(2 pi u1),
    z2 = sqrt(-2 ln u2) cos(2 pi u3), z3 = sqrt(-2 ln u2) sin(2 pi u3).
  S[e] = z_w.
"""
import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds.

    counter: uint32 array of shape (..., 4); key: two Python ints (k0, k1).
    Returns a uint32 array of the same shape as ``counter``.
    """
    c = np.asarray(counter, dtype=np.uint64) & _MASK
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + _W0) & 0xFFFFFFFF
            k1 = (k1 + _W1) & 0xFFFFFFFF
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0)), lo1, (hi0 ^ c3 ^ np.uint64(k1)), lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def sketch_words(seed, b, stage, k, n, p):
    """The raw uint32 word behind every sketch element, shape (n, p)."""
    total = n * p
    ncalls = (total + 3) // 4
    ctr = np.zeros((ncalls, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(ncalls, dtype=np.uint64)
    ctr[:, 1] = k
    ctr[:, 2] = stage
    ctr[:, 3] = b
    out = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    return out.reshape(-1)[:total].reshape(n, p)


def sketch(seed, b, stage, k, n, p):
    """Gaussian sketch S (n x p, fp64) for matrix b, stage, iteration k."""
    total = n * p
    ncalls = (total + 3) // 4
    ctr = np.zeros((ncalls, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(ncalls, dtype=np.uint64)
    ctr[:, 1] = k
    ctr[:, 2] = stage
    ctr[:, 3] = b
    x = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    u = ((x >> np.uint32(8)).astype(np.float64) + 0.5) * 2.0 ** -24
    rad01 = np.sqrt(-2.0 * np.log(u[:, 0]))
    rad23 = np.sqrt(-2.0 * np.log(u[:, 2]))
    th01 = 2.0 * np.pi * u[:, 1]
    th23 = 2.0 * np.pi * u[:, 3]
    z = np.stack([rad01 * np.cos(th01), rad01 * np.sin(th01),
                  rad23 * np.cos(th23), rad23 * np.sin(th23)], axis=-1)
    return z.reshape(-1)[:total].reshape(n, p)
