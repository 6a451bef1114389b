"""Pins for oracle.philox: published known-answer vectors and the statistics
of the Gaussian sketch."""
import os

import numpy as np
import pytest

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v = [int(x, 16) for x in line.split()]
            rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat_rows())
def test_known_answer_vectors(ctr, key, expect):
    out = philox.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
    assert [int(x) for x in out] == expect


def test_counter_layout_and_determinism():
    # element e of the sketch uses word e % 4 of call e // 4 with counter (e//4, k, stage, b)
    n, p, seed = 13, 8, 0x1234_5678_9ABC
    w = philox.sketch_words(seed, b=3, stage=1, k=5, n=n, p=p).reshape(-1)
    for e in (0, 1, 2, 3, 4, 57, n * p - 1):
        ctr = np.array([[e // 4, 5, 1, 3]], dtype=np.uint64)
        ref = philox.philox4x32_10(ctr, (seed & 0xFFFFFFFF, seed >> 32))[0][e % 4]
        assert w[e] == ref
    s1 = philox.sketch(seed, 3, 1, 5, n, p)
    s2 = philox.sketch(seed, 3, 1, 5, n, p)
    assert np.array_equal(s1, s2)
    assert not np.array_equal(s1, philox.sketch(seed, 3, 1, 6, n, p))
    assert not np.array_equal(s1, philox.sketch(seed, 2, 1, 5, n, p))
    assert not np.array_equal(s1, philox.sketch(seed, 3, 0, 5, n, p))


def test_box_muller_pairs():
    # z0^2 + z1^2 = -2 ln u0 for every pair, and the angle is 2 pi u1
    seed = 99
    n, p = 64, 4
    S = philox.sketch(seed, 0, 0, 0, n, p).reshape(-1, 4)
    x = philox.sketch_words(seed, 0, 0, 0, n, p).reshape(-1, 4)
    u = ((x >> 8).astype(np.float64) + 0.5) * 2.0 ** -24
    assert np.all((u > 0) & (u < 1))
    np.testing.assert_allclose(S[:, 0] ** 2 + S[:, 1] ** 2, -2 * np.log(u[:, 0]), rtol=1e-12)
    np.testing.assert_allclose(S[:, 2] ** 2 + S[:, 3] ** 2, -2 * np.log(u[:, 2]), rtol=1e-12)
    ang = np.mod(np.arctan2(S[:, 1], S[:, 0]), 2 * np.pi)
    np.testing.assert_allclose(ang, 2 * np.pi * u[:, 1], atol=1e-9)


def test_gaussian_moments():
    # 2^20 draws: mean 0, variance 1, kurtosis 3 within ~6 standard errors
    S = philox.sketch(2024, 0, 0, 0, 1 << 17, 8).reshape(-1)
    N = S.size
    assert abs(S.mean()) < 6 / np.sqrt(N)
    assert abs(S.var() - 1) < 6 * np.sqrt(2 / N)
    assert abs(np.mean(S ** 4) - 3) < 6 * np.sqrt(96 / N)
    # tail mass beyond 2 sigma: 0.0455
    frac = np.mean(np.abs(S) > 2)
    assert abs(frac - 0.04550026) < 6 * np.sqrt(0.0455 * 0.9545 / N)
