"""Pins of the oracle's SpectralQuant (uniform allocation, SQU-KV) quantiser
(CPU only): the Gaussian Lloyd-Max codebook against Max's table and the
Lloyd conditions, the calibration against a known covariance, a hand-worked
two-dimensional case, equivariance under a change of basis, the distortion
of isotropic data, and the pages' qualitative claims (SQ ahead of TQ-KV on
low-rank data at 2 bits, behind it on heavy-tailed data)."""
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import metrics as me
from oracle import quantizer as qz
from oracle import spectral as sq

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _max_table():
    rows = {}
    for line in open(os.path.join(GOLDEN, "gaussian_lloyd_max.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v = line.split()
        rows[int(v[0])] = (float(v[1]), [float(x) for x in v[2:]])
    return rows


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_codebook_matches_max_table_and_lloyd_conditions(bits):
    mse, levels = _max_table()[bits]
    c, t = sq.gaussian_lloyd_max(bits)
    # Max (1960) prints four significant digits.
    assert np.allclose(c[len(c) // 2:], levels, rtol=1.5e-3, atol=0)
    assert abs(sq.gaussian_distortion(c, t) - mse) < 2e-3 * mse
    assert np.array_equal(c, -c[::-1])
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-15)
    # Centroid condition by independent quadrature.
    e = np.concatenate(([-np.inf], t, [np.inf]))
    for k in range(len(c)):
        from scipy import integrate
        m0 = integrate.quad(stats.norm.pdf, e[k], e[k + 1])[0]
        m1 = integrate.quad(lambda x: x * stats.norm.pdf(x), e[k], e[k + 1])[0]
        assert abs(m1 / m0 - c[k]) < 1e-9
    if bits == 1:
        assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-14


def test_distortion_by_monte_carlo():
    c, t = sq.gaussian_lloyd_max(3)
    x = np.random.default_rng(2).standard_normal(400000)
    err = (x - c[np.searchsorted(t, x, side="right")]) ** 2
    assert abs(err.mean() - sq.gaussian_distortion(c, t)) < 4 * err.std() / math.sqrt(err.size)


def test_fit_recovers_a_known_covariance():
    """Calibration ([P2] "Configuração Experimental": a per-head eigenbasis
    from representative tokens): eigenvectors and spreads of data drawn with
    covariance W diag(lam) W^T (well separated) plus a mean."""
    d, N = 16, 200000
    rng = np.random.default_rng(3)
    W, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = 2.0 ** -np.arange(d)
    mu = rng.standard_normal(d)
    X = (rng.standard_normal((N, d)) * np.sqrt(lam)) @ W.T + mu
    V, m, s = sq.fit(X)
    assert np.allclose(V.T @ V, np.eye(d), atol=1e-12)
    assert np.allclose(m, X.mean(axis=0))
    assert abs(np.sum(s * s) - 1.0) < 1e-12
    assert np.all(np.diff(s) <= 0)
    assert np.allclose(s, np.sqrt(lam / lam.sum()), rtol=0.02)
    for j in range(4):  # the leading directions, up to sign, with the sign convention applied
        assert abs(abs(V[:, j] @ W[:, j]) - 1.0) < 1e-3
        assert V[np.argmax(np.abs(V[:, j])), j] > 0


def test_hand_worked_two_dimensional_case():
    """d = 2, basis a rotation by 30 degrees, mean (1, 2), spreads (0.8, 0.6),
    1 bit (c = +-sqrt(2/pi), the boundary at 0).  x = mu + 3 (cos 100deg,
    sin 100deg): nu = 3, z = (cos 70deg, sin 70deg) in the basis, so both
    codes are 1 and x_hat = mu + 3 V (0.8 c1, 0.6 c1)."""
    a = math.radians(30)
    V = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
    mu = np.array([1.0, 2.0])
    s = np.array([0.8, 0.6])
    st = sq.SQState(V, mu, s, 1)
    x = mu + 3.0 * np.array([math.cos(math.radians(100)), math.sin(math.radians(100))])
    q = sq.quantize(x[None], st)
    assert abs(q["nu"][0] - 3.0) < 1e-14
    assert np.allclose(q["z"][0], [math.cos(math.radians(70)), math.sin(math.radians(70))], atol=1e-14)
    assert list(q["idx"][0]) == [1, 1]
    c1 = math.sqrt(2 / math.pi)
    want = mu + 3.0 * (V @ np.array([0.8 * c1, 0.6 * c1]))
    assert np.allclose(sq.dequantize(q, st)[0], want, atol=1e-6)   # fp32 norm storage
    # Band: the distance of each z_i to its boundary s_i t = 0.
    assert np.allclose(q["bdist"][0], np.abs(q["z"][0]))
    # A vector equal to the mean: all fields 0, x_hat = mu.
    q0 = sq.quantize(mu[None], st)
    assert q0["nu"][0] == 0 and list(q0["idx"][0]) == [0, 0]
    assert np.array_equal(sq.dequantize(q0, st)[0], mu)


def test_equivariant_under_a_change_of_basis():
    """Rotating the data, the mean and the basis by one orthogonal Q leaves
    the codes unchanged and rotates the reconstruction (a transposed basis
    or a mean applied on the wrong side breaks this)."""
    d = 32
    rng = np.random.default_rng(5)
    V, _ = np.linalg.qr(rng.standard_normal((d, d)))
    mu = rng.standard_normal(d)
    s = np.sqrt(np.linspace(2.0, 0.1, d) / np.linspace(2.0, 0.1, d).sum())
    X = rng.standard_normal((500, d)) * 2 + mu
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    a = sq.SQState(V, mu, s, 3)
    b = sq.SQState(Q @ V, Q @ mu, s, 3)
    qa, qb = sq.quantize(X, a), sq.quantize(X @ Q.T, b)
    assert np.array_equal(qa["idx"], qb["idx"])
    assert np.allclose(sq.dequantize(qb, b), sq.dequantize(qa, a) @ Q.T, atol=1e-9)


def test_isotropic_distortion_is_the_gaussian_lloyd_max_distortion():
    """Isotropic Gaussian data, any basis, uniform spreads 1/sqrt(d): the
    standardised coordinate sqrt(d) z_i of a uniform direction tends to
    N(0, 1), so relMSE tends to the Gaussian Lloyd-Max distortion (d = 1024:
    within 1 %)."""
    d = 1024
    rng = np.random.default_rng(6)
    V, _ = np.linalg.qr(rng.standard_normal((d, d)))
    st = sq.SQState(V, np.zeros(d), np.full(d, 1 / math.sqrt(d)), 2)
    X = rng.standard_normal((3000, d))
    per = np.sum((X - sq.dequantize(sq.quantize(X, st), st)) ** 2, axis=1) / np.sum(X * X, axis=1)
    D = sq.gaussian_distortion(st.centroids, st.boundaries)
    assert abs(per.mean() - D) < 0.01 * D + 4 * per.std() / math.sqrt(per.size)


def _tq_kv_relmse(X, bits, seed=0):
    st = qz.QState(X.shape[1], qz.MSE, bits, seed)
    return me.rel_mse(X, qz.dequantize(qz.quantize(X, st), st))


def test_structured_data_favours_spectral_at_two_bits():
    """[P2] "Resultados e Recomendações": at b = 2 SQ variants win on
    structured (low-rank) data.  Rank-8 data plus 1 % noise, separate
    calibration set: SQU-KV relMSE below TQ-KV's (by 20 % on this draw)."""
    d, r = 128, 8
    rng = np.random.default_rng(7)
    W, _ = np.linalg.qr(rng.standard_normal((d, r)))
    lam = 0.7 ** np.arange(r)

    def draw(n):
        return (rng.standard_normal((n, r)) * np.sqrt(lam)) @ W.T + 0.01 * rng.standard_normal((n, d))
    V, mu, s = sq.fit(draw(4096))
    X = draw(2000)
    st = sq.SQState(V, mu, s, 2)
    sq_err = me.rel_mse(X, sq.dequantize(sq.quantize(X, st), st))
    assert sq_err < 0.9 * _tq_kv_relmse(X, 2)


def test_heavy_tailed_data_favours_tq_kv():
    """[P2] "Contribuições Principais" 3: eigenvector methods fail on
    heavy-tailed data (the calibrated basis is misaligned) while the WHT
    spreads outliers.  Student-t(3) entries with 1 % of vectors carrying a
    +-20 coordinate: SQU-KV relMSE above TQ-KV's at b = 3."""
    d = 128
    rng = np.random.default_rng(8)

    def draw(n):
        z = rng.standard_normal((n, d)) / np.sqrt(np.sum(rng.standard_normal((3, n, d)) ** 2, axis=0) / 3.0)
        hit = rng.random(n) < 0.01
        z[hit, rng.integers(0, d, hit.sum())] = 20.0 * np.sign(rng.standard_normal(hit.sum()))
        return z
    V, mu, s = sq.fit(draw(4096))
    X = draw(3000)
    st = sq.SQState(V, mu, s, 3)
    assert me.rel_mse(X, sq.dequantize(sq.quantize(X, st), st)) > _tq_kv_relmse(X, 3)


def test_in_band_flip_takes_the_other_cell():
    d = 8
    V = np.eye(d)
    s = np.full(d, 1 / math.sqrt(d))
    st = sq.SQState(V, np.zeros(d), s, 2)
    t = st.boundaries[2] * s[0]
    x = np.full(d, 0.1)
    # Put coordinate 0 of the unit direction on the boundary s_0 t_2.
    rest = math.sqrt((1 - t * t) / (d - 1))
    x = np.concatenate(([t], np.full(d - 1, rest)))
    q = sq.quantize(x[None], st)
    assert q["bdist"][0, 0] < 1e-12
    flip = np.zeros((1, d), dtype=bool)
    flip[0, 0] = True
    qf = sq.quantize(x[None], st, flip_codes=flip)
    assert abs(int(qf["idx"][0, 0]) - int(q["idx"][0, 0])) == 1
    with pytest.raises(AssertionError):
        bad = np.zeros((1, d), dtype=bool)
        bad[0, 1] = True
        sq.quantize(x[None], st, flip_codes=bad)
