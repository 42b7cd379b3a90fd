"""Pins of the Beta Lloyd-Max codebook against closed forms, quadrature and
the Gaussian Lloyd-Max table (CPU only)."""
import math
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import codebook as cb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _quad(f, lo, hi):
    return integrate.quad(f, lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]


@pytest.mark.parametrize("d", [16, 128, 1024])
def test_density_integrates_to_one(d):
    # Quadrature of the density is independent of the incomplete-beta cdf.
    w = 12.0 / math.sqrt(d)
    total = _quad(lambda t: cb.pdf(t, d), -min(1, w), min(1, w))
    assert abs(total - 1.0) < 1e-10
    assert abs(cb.cdf(0.3, d) - _quad(lambda t: cb.pdf(t, d), -1, 0.3)) < 1e-10


def test_density_is_sphere_marginal():
    # Monte Carlo: a coordinate of a uniform unit vector in R^d.
    d = 32
    x = np.random.default_rng(0).standard_normal((100000, d))
    t = x[:, 0] / np.linalg.norm(x, axis=1)
    assert stats.kstest(t, lambda v: cb.cdf(v, d)).pvalue > 1e-3


@pytest.mark.parametrize("d,bits", [(128, 1), (128, 2), (128, 3), (128, 4), (1024, 4), (32, 3), (1024, 2)])
def test_lloyd_conditions(d, bits):
    c, t = cb.lloyd_max(d, bits)
    K = 1 << bits
    assert len(c) == K and len(t) == K - 1
    assert np.all(np.diff(c) > 0)
    assert np.allclose(c, -c[::-1], atol=0, rtol=0)
    assert np.max(np.abs(t - 0.5 * (c[:-1] + c[1:]))) < 1e-16
    if True:
        # Centroid condition by plain quadrature (independent of the closed form).
        edges = np.concatenate(([-1.0], t, [1.0]))
        for k in range(K):
            lo, hi = edges[k], edges[k + 1]
            m0 = _quad(lambda s: cb.pdf(s, d), lo, hi)
            m1 = _quad(lambda s: s * cb.pdf(s, d), lo, hi)
            assert abs(m1 / m0 - c[k]) < 1e-11 / math.sqrt(d) + 1e-12 * abs(c[k])


@pytest.mark.parametrize("d", [32, 128, 1024])
def test_one_bit_closed_form(d):
    # E|T| for a coordinate of a uniform unit vector: Gamma(d/2)/(sqrt(pi) Gamma((d+1)/2)).
    c, t = cb.lloyd_max(d, 1)
    ref = math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c[1] - ref) < 1e-14
    assert t[0] == 0.0


def test_known_one_bit_values():
    assert abs(cb.lloyd_max(128, 1)[0][1] - 0.0706615727) < 1e-10
    assert abs(cb.lloyd_max(1024, 1)[0][1] - 0.0249399806) < 1e-10


def _gaussian_table():
    rows = {}
    for line in open(os.path.join(GOLDEN, "gaussian_lloyd_max.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v = line.split()
        rows[int(v[0])] = (float(v[1]), [float(x) for x in v[2:]])
    return rows


def _gaussian_lloyd_max(bits, iters=20000):
    """Lloyd-Max for N(0,1) with closed-form cell moments (Phi and phi)."""
    K = 1 << bits
    c = stats.norm.ppf((np.arange(K) + 0.5) / K)
    for _ in range(iters):
        e = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        m0 = stats.norm.cdf(e[1:]) - stats.norm.cdf(e[:-1])
        m1 = stats.norm.pdf(e[:-1]) - stats.norm.pdf(e[1:])
        new = m1 / m0
        if np.max(np.abs(new - c)) < 1e-14:
            c = new
            break
        c = new
    return c


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_limit(bits):
    """sqrt(d) c(d, b) tends to the Gaussian Lloyd-Max levels as d grows
    ([P1] "Marco Teórico": the Beta marginal tends to a Gaussian), with a gap
    that shrinks monotonically; the limit agrees with Max's table."""
    mse, levels = _gaussian_table()[bits]
    g = _gaussian_lloyd_max(bits)
    assert np.allclose(g[len(g) // 2:], levels, rtol=1.5e-3, atol=0)
    gaps = []
    for d in (16, 64, 256, 1024, 4096, 65536):
        c, t = cb.lloyd_max(d, bits)
        gaps.append(np.max(np.abs(math.sqrt(d) * c - g)))
    assert all(g1 > g2 for g1, g2 in zip(gaps[:-1], gaps[1:]))
    assert gaps[-1] < 1e-3
    c, t = cb.lloyd_max(65536, bits)
    assert abs(65536 * cb.distortion(65536, c, t) - mse) < 2e-3 * mse
    if bits == 1:
        assert abs(math.sqrt(65536) * c[1] - math.sqrt(2 / math.pi)) < 1e-4


@pytest.mark.parametrize("bits", [2, 4])
def test_distortion_by_monte_carlo(bits):
    d = 64
    c, t = cb.lloyd_max(d, bits)
    x = np.random.default_rng(1).standard_normal((200000, d))
    y = (x / np.linalg.norm(x, axis=1, keepdims=True))[:, :4].ravel()
    err = (y - c[cb.quantize_index(y, t)]) ** 2
    D = cb.distortion(d, c, t)
    assert abs(err.mean() - D) < 4 * err.std() / math.sqrt(err.size)


def test_index_tie_goes_up():
    c, t = cb.lloyd_max(128, 2)
    assert list(cb.quantize_index(np.array([t[0], t[1], t[2], -1.0, 1.0]), t)) == [1, 2, 3, 0, 3]
