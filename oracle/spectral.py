"""SpectralQuant with uniform allocation (SQU-KV): a calibrated per-head
eigenbasis, the same bit width on every eigen-coordinate, no QJL.   [oracle]

[P2] section "Configuração Experimental", scheme 2 (SpectralQuant): a
data-adaptive quantiser that calibrates a per-head eigenvector basis from
representative tokens, allocates bits to the high-variance dimensions by
water-filling and adds a selective QJL sketch on the top effective
dimensions.  [P2] section "Recomendações Práticas" 2 and 3: SQU-KV is
SpectralQuant with uniform allocation, for structured (low-rank) data at
2-3 bits with separate K and V calibration sets; water-filling is dropped
(uniform allocation performs as well).

Readings (the pages give no formulas):
  calibration: per head and tensor, the centred covariance of the
      calibration vectors, C = V diag(lambda) V^T with the eigenvalues
      descending and each eigenvector's largest-|.| entry positive (the
      convention of the HeadQ basis); mu the calibration mean;
  the norm split of the TQ schemes, taken about mu: x - mu = nu u,
      nu = ||x - mu||, and the direction's eigen-coordinates z = V^T u (a unit
      vector, like TQ's rotated y);
  uniform allocation: every coordinate gets b bits and is coded against the
      b-bit Lloyd-Max codebook of N(0, 1) after standardising by its
      calibrated spread s_i = sqrt(lambda_i / sum(lambda)) (the rms of z_i
      for a vector of typical norm): idx_i = #{k : z_i >= s_i t_k} (ties up);
  no water-filling, no d_eff pruning, no QJL sketch (the "-KV" of the name,
      as in TQ-KV);
  dequantisation: x_hat = mu + nu V (s * c[idx]); nu = 0 gives x_hat = mu.
  The decision band (parity) is the distance of z_i to its nearest decision
  boundary s_i t_k, in the unit-vector units of the TQ codes' band.
"""
import numpy as np
from scipy import stats

from . import quantizer as qz


def gaussian_lloyd_max(bits, tol=1e-15, max_iter=100000):
    """Lloyd-Max codebook of N(0, 1): (centroids[2^bits], boundaries[2^bits-1]),
    ascending; cell moments in closed form (Phi and phi), symmetric."""
    K = 1 << bits
    c = stats.norm.ppf((np.arange(K) + 0.5) / K)
    for _ in range(max_iter):
        e = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        m0 = stats.norm.sf(e[:-1]) - stats.norm.sf(e[1:])
        m1 = stats.norm.pdf(e[:-1]) - stats.norm.pdf(e[1:])
        new = m1 / m0
        delta = np.max(np.abs(new - c))
        c = new
        if delta < tol:
            break
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    if K % 2 == 0:
        t[K // 2 - 1] = 0.0
    return c, t


def gaussian_distortion(c, t):
    """E[(X - c[idx(X)])^2] for X ~ N(0, 1), in closed form per cell."""
    e = np.concatenate(([-np.inf], t, [np.inf]))
    D = 0.0
    for k in range(len(c)):
        a, b = e[k], e[k + 1]
        m0 = stats.norm.cdf(b) - stats.norm.cdf(a)
        m1 = stats.norm.pdf(a) - stats.norm.pdf(b)
        # E[X^2 1_cell] = m0 + a phi(a) - b phi(b)   (with x phi(x) -> 0 at +-inf)
        fa = a * stats.norm.pdf(a) if np.isfinite(a) else 0.0
        fb = b * stats.norm.pdf(b) if np.isfinite(b) else 0.0
        m2 = m0 + fa - fb
        D += m2 - 2 * c[k] * m1 + c[k] * c[k] * m0
    return D


def fit(calib):
    """(basis V [d, d] with eigenvectors as columns, mean [d], scale [d]) of
    the calibration vectors calib [N, d], float64."""
    X = np.asarray(calib, dtype=np.float64)
    mu = X.mean(axis=0)
    Xc = X - mu
    C = Xc.T @ Xc / X.shape[0]
    w, V = np.linalg.eigh(C)
    order = np.argsort(w)[::-1]
    w, V = np.clip(w[order], 0.0, None), V[:, order]
    for j in range(V.shape[1]):
        k = np.argmax(np.abs(V[:, j]))
        if V[k, j] < 0:
            V[:, j] = -V[:, j]
    total = w.sum()
    scale = np.sqrt(w / total) if total > 0 else np.zeros_like(w)
    return V, mu, scale


class SQState:
    """Everything the quantiser of one head needs: the basis, mean and
    scales as given (float32 values, used exactly), the bit width and the
    Gaussian codebook."""

    def __init__(self, basis, mean, scale, bits):
        self.V = np.asarray(basis, dtype=np.float64)
        self.mu = np.asarray(mean, dtype=np.float64)
        self.s = np.asarray(scale, dtype=np.float64)
        self.d = self.V.shape[0]
        self.bits = bits
        self.centroids, self.boundaries = gaussian_lloyd_max(bits)


def _indices(Z, st):
    """idx_i = #{k : z_i >= s_i t_k}."""
    thr = st.s[None, :, None] * st.boundaries[None, None, :]
    return np.sum(Z[:, :, None] >= thr, axis=2).astype(np.int64)


def quantize(X, st, flip_codes=None, band=1e-6):
    """X [N, d] float64 -> dict of fields (nu, idx) plus the decision band
    diagnostic bdist (distance of z_i to its nearest boundary s_i t_k).
    flip_codes ([N, d] bool) selects decisions within `band` of a boundary
    that take the other valid outcome."""
    X = np.asarray(X, dtype=np.float64)
    Xc = X - st.mu[None, :]
    nu = np.sqrt(np.sum(Xc * Xc, axis=1))
    safe = np.where(nu > 0, nu, 1.0)
    Z = (Xc / safe[:, None]) @ st.V
    idx = _indices(Z, st)
    thr = st.s[None, :, None] * st.boundaries[None, None, :]
    dist = np.abs(Z[:, :, None] - thr)
    bdist = np.min(dist, axis=2)
    if flip_codes is not None and np.any(flip_codes):
        assert np.all(bdist[flip_codes] <= band), "flip requested outside the decision band"
        k = np.argmin(dist, axis=2)
        cur = idx[flip_codes]
        kk = k[flip_codes]
        assert np.all((cur == kk) | (cur == kk + 1))
        idx[flip_codes] = np.where(cur == kk, kk + 1, kk)
    zero = nu == 0
    idx[zero] = 0
    bdist[zero] = np.inf
    return {"nu": nu, "idx": idx, "z": Z, "bdist": bdist}


def dequantize(q, st):
    """x_hat = mu + nu V (s * c[idx]), [N, d] float64 (stored fp32 norm)."""
    nu = qz.stored(q["nu"])
    Y = st.s[None, :] * st.centroids[q["idx"]]
    Xh = st.mu[None, :] + nu[:, None] * (Y @ st.V.T)
    Xh[nu == 0] = st.mu
    return Xh


def pack(q, st):
    """Packed planes (the TQ layout: b-bit LSB-first fields, fp32 norms)."""
    return {"codes": qz.pack_bits(q["idx"], st.bits), "norms": q["nu"].astype(np.float32)}
