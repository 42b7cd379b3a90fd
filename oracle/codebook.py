"""Beta((d-1)/2,(d-1)/2) Lloyd-Max codebook, float64.   [oracle]

[P1] section "Marco Teórico": a coordinate of a vector uniform on the sphere
S^{d-1} follows Beta((d-1)/2,(d-1)/2) (read on [-1,1]: t = 2x-1), which tends
to a Gaussian as d grows.  [P2] section "Configuração Experimental": the
codebook is a data-oblivious Beta Lloyd-Max codebook.

Reading: the Beta law is that of (1+t)/2, so t has density
    f_d(t) = (1-t^2)^((d-3)/2) / B(1/2, (d-1)/2)   on [-1, 1].
Lloyd-Max: boundaries are midpoints of neighbouring centroids, centroids are
conditional means of their cells; iterate to a fixed point.
"""
import math
import numpy as np
from scipy import special


def _a(d):
    return (d - 1) / 2.0


def log_norm_const(d):
    """log B(1/2, (d-1)/2), from the beta function itself (a difference of
    two large log-gamma values would lose ~1e-13 relative at d = 1024)."""
    return math.log(special.beta(0.5, _a(d)))


def pdf(t, d):
    """Density of one coordinate of a uniform unit vector in R^d."""
    t = np.asarray(t, dtype=np.float64)
    a = _a(d)
    with np.errstate(divide="ignore"):
        logf = (a - 1.0) * np.log1p(-t * t) - log_norm_const(d)
    return np.where(np.abs(t) < 1.0, np.exp(logf), 0.0)


def cdf(t, d):
    """P(T <= t) = I_{(1+t)/2}(a, a)."""
    a = _a(d)
    x = np.clip((1.0 + np.asarray(t, dtype=np.float64)) / 2.0, 0.0, 1.0)
    return special.betainc(a, a, x)


def cell_mass(lo, hi, d):
    """Probability of the cell [lo, hi).  The upper tail uses the complement
    so that far-tail cells keep their relative precision."""
    a = _a(d)
    xlo = np.clip((1.0 + lo) / 2.0, 0.0, 1.0)
    xhi = np.clip((1.0 + hi) / 2.0, 0.0, 1.0)
    if lo >= 0.0:
        return special.betaincc(a, a, xlo) - special.betaincc(a, a, xhi)
    return special.betainc(a, a, xhi) - special.betainc(a, a, xlo)


def cell_first_moment(lo, hi, d):
    """Integral of t f_d(t) over [lo, hi].  Closed form: the antiderivative of
    t (1-t^2)^(a-1) is -(1-t^2)^a / (2a)."""
    a = _a(d)

    def g(t):
        if abs(t) >= 1.0:
            return 0.0
        return math.exp(a * math.log1p(-t * t))

    return (g(lo) - g(hi)) / (2.0 * a * math.exp(log_norm_const(d)))


def lloyd_max(d, bits, tol=1e-15, max_iter=200000):
    """Return (centroids[2^bits], boundaries[2^bits-1]) in float64, ascending.

    Starts from the quantile midpoints, iterates the two Lloyd conditions,
    then makes the result exactly symmetric (the density is even, so the
    optimum is symmetric and the middle boundary is 0)."""
    K = 1 << bits
    a = _a(d)
    probs = (np.arange(K) + 0.5) / K
    c = 2.0 * special.betaincinv(a, a, probs) - 1.0
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        new = np.empty(K)
        for k in range(K):
            m0 = cell_mass(edges[k], edges[k + 1], d)
            m1 = cell_first_moment(edges[k], edges[k + 1], d)
            new[k] = m1 / m0
        delta = np.max(np.abs(new - c))
        c = new
        if delta < tol:
            break
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    if K % 2 == 0:
        t[K // 2 - 1] = 0.0
    return c, t


def distortion(d, centroids, boundaries):
    """Per-coordinate MSE E[(T - c[idx(T)])^2] of the codebook, by the
    closed-form second moment per cell: E[T^2 1_cell] = m0 - E[(1-T^2) 1_cell]
    where the latter uses the density of dimension d+2 (ratio of norming
    constants)."""
    K = len(centroids)
    edges = np.concatenate(([-1.0], boundaries, [1.0]))
    # (1-t^2) f_d(t) = f_{d+2}(t) * B(1/2,(d+1)/2) / B(1/2,(d-1)/2)
    ratio = math.exp(log_norm_const(d + 2) - log_norm_const(d))
    D = 0.0
    for k in range(K):
        m0 = cell_mass(edges[k], edges[k + 1], d)
        m1 = cell_first_moment(edges[k], edges[k + 1], d)
        m2 = m0 - ratio * cell_mass(edges[k], edges[k + 1], d + 2)
        c = centroids[k]
        D += m2 - 2.0 * c * m1 + c * c * m0
    return D


def quantize_index(y, boundaries):
    """idx_i = number of boundaries t_k with y_i >= t_k (ties go up)."""
    y = np.asarray(y, dtype=np.float64)
    return np.searchsorted(boundaries, y, side="right").astype(np.int64)


def boundary_distance(y, boundaries):
    """Distance of each coordinate to its nearest decision boundary."""
    y = np.asarray(y, dtype=np.float64)
    return np.min(np.abs(y[..., None] - boundaries), axis=-1)
