"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds input recipes only (random matrices with prescribed spectra,
casts to fp32 / bf16); none of the method's arithmetic lives here.  numpy PCG64
streams, one SeedSequence child per matrix of a batch; everything is formed in
fp64 and then cast.

Workloads (sizes from the library's five headline configurations):
  spd_64        one SPD 64 x 64, lambda log-uniform in [1e-3, 1], plus a
                64 x 32 Gaussian for the polar factor
  shampoo_1024x4096  ten gradients 1024 x 4096 with N(0, 0.1^2) entries and the
                statistics start L0 = eps I, R0 = eps I (eps = 1e-6, beta = 0.95)
  blocks_64x512 64 SPD blocks 512 x 512, spectrum i^{-1.5} mapped affinely onto
                [1e-6, 1], random orthogonal eigenvectors per block
  muon_32x4096x1024  32 bf16 matrices U diag(sigma) V^T, sigma geometrically
                spaced over [1e-4, 1]
  mp_10000      A = W W^T / 20000 + 1e-4 I with W 10000 x 20000 Gaussian
                (Marchenko-Pastur spectrum, ratio 1/2)
The PRISM synthesis tests on Gaussian and heavy-tailed Marchenko-Pastur
spectra; the last two workloads stand in for those.
"""
import numpy as np


def rngs(seed, count):
    """One independent PCG64 generator per matrix."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(count)]


def random_orthogonal(rng, n, m=None):
    """Q from the QR factorisation of an n x m Gaussian (m = n by default),
    columns sign-fixed by diag(R) > 0."""
    m = n if m is None else m
    Q, R = np.linalg.qr(rng.standard_normal((n, m)))
    return Q * np.sign(np.diag(R))


def spd_from_spectrum(Q, lam):
    """Q diag(lam) Q^T in fp64, symmetrised exactly."""
    A = (Q * lam) @ Q.T
    return 0.5 * (A + A.T)


def to_bf16_bits(x):
    """fp32 -> bf16 with round-to-nearest-even; returns uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns -> the fp32 values they represent (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- small cases

def spd_logu(n, seed, lo=1e-3, hi=1.0):
    """SPD n x n with lambda = 10^U(log10 lo, log10 hi); returns (A_f32, Q, lam)."""
    rng = np.random.default_rng(seed)
    Q = random_orthogonal(rng, n)
    lam = 10.0 ** rng.uniform(np.log10(lo), np.log10(hi), size=n)
    A = spd_from_spectrum(Q, lam)
    return A.astype(np.float32), Q, lam


def spd_power_batch(batch, n, seed, lmin=1e-6, lmax=1.0, expo=1.5):
    """Batch of SPD blocks with lambda_i = i^{-expo} mapped affinely onto
    [lmin, lmax]; same spectrum, independent Q per block.
    Returns (A_f32 [batch, n, n], Qs, lam)."""
    i = np.arange(1, n + 1, dtype=np.float64)
    raw = i ** (-expo)
    lam = lmin + (raw - raw.min()) * (lmax - lmin) / (raw.max() - raw.min())
    out = np.empty((batch, n, n), np.float32)
    Qs = []
    for b, rng in enumerate(rngs(seed, batch)):
        Q = random_orthogonal(rng, n)
        out[b] = spd_from_spectrum(Q, lam).astype(np.float32)
        Qs.append(Q)
    return out, Qs, lam


def gaussian(m, n, seed, std=1.0):
    """m x n Gaussian, fp32."""
    return (np.random.default_rng(seed).standard_normal((m, n)) * std).astype(np.float32)


def irregular_blocks(count, seed, lo=8, hi=64):
    """`count` Gaussian blocks (fp32) whose sides are drawn uniformly from
    [lo, hi], one generator per block: the many small irregular blocks of a
    block-diagonal preconditioner's per-block orthogonalisation."""
    out = []
    for rng in rngs(seed, count):
        m, n = (int(x) for x in rng.integers(lo, hi + 1, 2))
        out.append(rng.standard_normal((m, n)).astype(np.float32))
    return out


def polar_batch(batch, m, n, seed, smin=1e-4, smax=1.0, bf16=True):
    """Batch of m x n matrices U diag(sigma) V^T, sigma geometric over [smin, smax].
    Returns (values_f32 [batch, m, n], bits_u16 or None, sigma)."""
    sigma = np.geomspace(smin, smax, n)
    vals = np.empty((batch, m, n), np.float32)
    bits = np.empty((batch, m, n), np.uint16) if bf16 else None
    for b, rng in enumerate(rngs(seed, batch)):
        U = random_orthogonal(rng, m, n)
        V = random_orthogonal(rng, n)
        G = (U * sigma) @ V.T
        if bf16:
            bits[b] = to_bf16_bits(G.astype(np.float32))
            vals[b] = bf16_bits_to_f32(bits[b])
        else:
            vals[b] = G.astype(np.float32)
    return vals, bits, sigma


def polar_spectrum_batch(batch, m, n, seed, sigma):
    """Batch of m x n fp32 matrices U diag(sigma) V^T with U, V from the QR of
    seeded Gaussians and the given singular values (length n)."""
    sigma = np.asarray(sigma, np.float64)
    vals = np.empty((batch, m, n), np.float32)
    for b, rng in enumerate(rngs(seed, batch)):
        U = random_orthogonal(rng, m, n)
        V = random_orthogonal(rng, n)
        vals[b] = ((U * sigma) @ V.T).astype(np.float32)
    return vals


def mp_shape(m, n, seed):
    """The singular values of an m x n Gaussian (the square roots of a
    Marchenko-Pastur spectrum of ratio n / m), ascending, mapped affinely onto
    [0, 1]: the heavy-tailed shape of the spectrum sweeps."""
    s = np.linalg.svd(np.random.default_rng(seed).standard_normal((m, n)), compute_uv=False)
    s = np.sort(s)
    return (s - s[0]) / (s[-1] - s[0])


# ---------------------------------------------------------------- headline workloads

def spd_64():
    """n = 64 SPD (seed 101) and the 64 x 32 Gaussian for the polar factor (seed 102)."""
    A, Q, lam = spd_logu(64, 101)
    G = gaussian(64, 32, 102)
    return dict(A=A, Q=Q, lam=lam, G=G, d=2, p=8, tol=1e-6)


def shampoo_1024x4096(steps=10, m=1024, n=4096, seed=201):
    """Gradients G_1..G_steps (fp32, N(0, 0.1^2)), eps = 1e-6, beta = 0.95."""
    rng = np.random.default_rng(seed)
    Gs = [(rng.standard_normal((m, n)) * 0.1).astype(np.float32) for _ in range(steps)]
    eps = 1e-6
    return dict(Gs=Gs, beta=0.95, eps=eps,
                L0=(eps * np.eye(m)).astype(np.float32),
                R0=(eps * np.eye(n)).astype(np.float32))


def blocks_64x512(batch=64, n=512, seed=301):
    A, Qs, lam = spd_power_batch(batch, n, seed)
    return dict(A=A, Qs=Qs, lam=lam)


def muon_32x4096x1024(batch=32, m=4096, n=1024, seed=401):
    vals, bits, sigma = polar_batch(batch, m, n, seed)
    return dict(G=vals, G_bits=bits, sigma=sigma, tol=1e-2)


def mp_square(n=10000, m=20000, seed=501, block=2000):
    """A = W W^T / m + 1e-4 I, W n x m Gaussian, built blockwise in fp64 and
    cast to fp32."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((n, m)).astype(np.float32).astype(np.float64)
    A = np.empty((n, n), np.float64)
    for i in range(0, n, block):
        A[i:i + block] = W[i:i + block] @ W.T / m
    A[np.diag_indices(n)] += 1e-4
    A = 0.5 * (A + A.T)
    return A.astype(np.float32)


def mp_square_device(n=10000, m=20000, seed=501, device="cuda"):
    """The 10^4 Marchenko-Pastur workload built on the GPU (torch, seeded):
    W ~ N(0, 1) fp32 (n x m), A = W W^T / m + 1e-4 I formed in fp64, cast to
    fp32.  Returns a torch fp32 tensor on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    W = torch.randn(n, m, generator=g, device=device, dtype=torch.float32).double()
    A = (W @ W.T) / m
    del W
    A.diagonal().add_(1e-4)
    A = 0.5 * (A + A.T)
    return A.float()

