"""Pins of the oracle's write side: packing, marginal law after rotation,
end-to-end MSE against the codebook distortion, QJL estimator moments
(CPU only)."""
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import codebook as cb
from oracle import quantizer as qz
from oracle.rng import gaussian_sketch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pack_cases():
    for line in open(os.path.join(GOLDEN, "pack_examples.txt")):
        if line.startswith("#") or not line.strip():
            continue
        w, vals, hexes = [p.strip() for p in line.split("|")]
        yield int(w), [int(v) for v in vals.split()], bytes.fromhex(hexes.replace(" ", ""))


@pytest.mark.parametrize("case", list(_pack_cases()))
def test_pack_golden(case):
    w, vals, expect = case
    got = qz.pack_bits(np.array([vals]), w)
    assert bytes(got[0]) == expect
    assert np.array_equal(qz.unpack_bits(got, w, len(vals))[0], vals)


def test_prod_fields_golden():
    """PROD code block: field i = idx_i | sign_i << b, b + 1 bits, LSB first.
    b = 3: (idx, sign) = (5, 1), (3, 0) -> fields 13, 3 -> byte 0x3d;
    (7, 0), (0, 1) -> 7, 8 -> 0x87.  b = 2: (2, 1), (1, 0), (3, 1) ->
    fields 6, 1, 7, LSB first 0 1 1 | 1 0 0 | 1 1 1 -> byte 0 =
    2 + 4 + 8 + 64 + 128 = 0xce, byte 1 = 0x01."""
    st = qz.QState(16, qz.PROD, 4, 0)            # n = 4: b = 3
    assert st.base_bits == 3
    q = {"idx": np.array([[5, 3, 7, 0] + [0] * 12]), "sign_bits": np.array([[1, 0, 0, 1] + [0] * 12]),
         "nu": np.ones(1), "gamma": np.ones(1)}
    pl = qz.pack(q, st)
    assert set(pl) == {"codes", "norms", "gamma"} and pl["codes"].shape == (1, 8)
    assert bytes(pl["codes"][0][:2]) == bytes([0x3D, 0x87])
    idx, sb = qz.unpack_fields(pl["codes"], st, 16)
    assert np.array_equal(idx, q["idx"]) and np.array_equal(sb, q["sign_bits"])
    st2 = qz.QState(16, qz.PROD, 3, 0)           # n = 3: b = 2
    q2 = {"idx": np.array([[2, 1, 3] + [0] * 13]), "sign_bits": np.array([[1, 0, 1] + [0] * 13]),
          "nu": np.ones(1), "gamma": np.ones(1)}
    c2 = qz.pack(q2, st2)["codes"]
    assert c2.shape == (1, 6) and bytes(c2[0][:2]) == bytes([0xCE, 0x01])


@pytest.mark.parametrize("w", [1, 2, 3, 4])
def test_pack_roundtrip(w):
    v = np.random.default_rng(w).integers(0, 1 << w, size=(7, 128))
    assert np.array_equal(qz.unpack_bits(qz.pack_bits(v, w), w, 128), v)


def test_rotated_coordinates_follow_beta_marginal():
    # [P1] "Marco Teórico": Pi x / ||x|| of a Gaussian x is uniform on the
    # sphere, so each coordinate follows the Beta marginal.
    d = 128
    st = qz.QState(d, qz.MSE, 2, seed=11)
    x = np.random.default_rng(2).standard_normal((20000, d))
    y = qz.quantize(x, st)["y"]
    for j in (0, 77):
        assert stats.kstest(y[:, j], lambda v: cb.cdf(v, d)).pvalue > 1e-3


@pytest.mark.parametrize("mode", [qz.MSE, qz.PLAIN])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_relmse_equals_codebook_distortion(mode, bits):
    """For isotropic data E[relMSE] = d D(d, b) exactly (norm split + a
    uniform direction), for the rotated and the plain quantiser alike."""
    d = 128
    st = qz.QState(d, mode, bits, seed=5)
    x = np.random.default_rng(bits).standard_normal((3000, d))
    q = qz.quantize(x, st)
    xh = qz.dequantize(q, st)
    per = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    D = d * cb.distortion(d, st.centroids, st.boundaries)
    assert abs(per.mean() - D) < 4 * per.std() / math.sqrt(per.size) + 1e-6
    # Direction: cos(x, x_hat) ~ sqrt(1 - D) for small D.
    if bits >= 3:
        cos = np.sum(x * xh, axis=1) / np.linalg.norm(x, axis=1) / np.linalg.norm(xh, axis=1)
        assert abs(cos.mean() - math.sqrt(1 - D)) < 0.01


def test_high_rate_roundtrip_is_close():
    # A transposed rotation or a wrong index would give relMSE ~ 2, not ~ 0.009.
    d = 64
    st = qz.QState(d, qz.MSE, 4, seed=1)
    x = np.random.default_rng(0).standard_normal((50, d)) * 3.0 + 1.0
    xh = qz.dequantize(qz.quantize(x, st), st)
    assert np.sum((x - xh) ** 2) / np.sum(x * x) < 0.02


def test_zero_vector():
    for mode in (qz.MSE, qz.PROD, qz.PLAIN):
        st = qz.QState(32, mode, 3, seed=0)
        x = np.zeros((2, 32))
        x[1, 3] = 2.0
        q = qz.quantize(x, st)
        assert q["nu"][0] == 0 and np.all(q["idx"][0] == 0)
        if mode == qz.PROD:
            assert q["gamma"][0] == 0 and np.all(q["sign_bits"][0] == 0)
        assert np.all(qz.dequantize(q, st)[0] == 0)


def test_qjl_unbiased_with_pinned_variance():
    """[P1] "Contribuciones Clave" 1: the 1-bit sketch estimate of <q, r> is
    unbiased; its variance is ((pi/2)||q||^2||r||^2 - <q,r>^2)/m, whose
    leading term for unit q and m = d is (pi/2)||r||^2/d."""
    d = 64
    rng = np.random.default_rng(0)
    q = rng.standard_normal(d)
    q /= np.linalg.norm(q)
    r = rng.standard_normal(d) * 0.1
    est, sq = [], []
    for seed in range(4000):
        S = gaussian_sketch(seed, d)
        sigma = np.where(S @ r >= 0, 1.0, -1.0)
        rh = math.sqrt(math.pi / 2) / d * np.linalg.norm(r) * (S.T @ sigma)
        est.append(q @ rh)
        sq.append(np.sum((rh - r) ** 2))
    est = np.array(est)
    exact = q @ r
    n = est.size
    var = ((math.pi / 2) * (r @ r) - exact ** 2) / d
    assert abs(est.mean() - exact) < 4 * math.sqrt(var / n)
    # Sample variance of a near-Gaussian statistic: SE ~ var sqrt(2/n).
    assert abs(est.var() - var) < 4 * var * math.sqrt(2 / n)
    # E||r_hat - r||^2 = ||r||^2 (pi d / 2 - 1) / m.
    sq = np.array(sq)
    exp_sq = (r @ r) * (math.pi * d / 2 - 1) / d
    assert abs(sq.mean() - exp_sq) < 4 * sq.std() / math.sqrt(n)


def test_fp16_sketch_bias_within_rounding_bound():
    """S is the fp16 rounding of Gaussian draws G (a reading: the pages fix
    only the law).  Rounding moves each entry by a relative error rho_i with
    |rho_i| <= eps = 2^-11, S = diag-scaled G, and for a fixed scaling
    D = diag(1 + rho) the Gaussian identity gives E<q, r_hat> =
    ||r|| <Dq, Dr> / ||Dr||, within (3 eps + eps^2) / (1 - eps) ||q|| ||r||
    of <q, r>.  Checked on coupled draws: the same G with and without the
    rounding, mean difference of the two estimates over 4000 sketches."""
    from oracle.rng import gaussian_draws
    d = 128
    rng = np.random.default_rng(3)
    q = rng.standard_normal(d)
    r = rng.standard_normal(d) * 0.2
    gam = np.linalg.norm(r)
    c = math.sqrt(math.pi / 2) / d * gam
    diff = []
    for seed in range(4000):
        G = gaussian_draws(seed, d)
        S = G.astype(np.float16).astype(np.float64)
        assert np.all(np.abs(S - G) <= 2.0 ** -11 * np.abs(G) + 2.0 ** -25)
        e16 = c * (S @ q) @ np.where(S @ r >= 0, 1.0, -1.0)
        e64 = c * (G @ q) @ np.where(G @ r >= 0, 1.0, -1.0)
        diff.append(e16 - e64)
    diff = np.array(diff)
    eps = 2.0 ** -11
    bound = (3 * eps + eps * eps) / (1 - eps) * np.linalg.norm(q) * gam
    se = diff.std() / math.sqrt(diff.size)
    assert abs(diff.mean()) <= bound + 4 * se, (diff.mean(), bound, se)
    # The bound is small against the spread of one sketch's estimate (m = d).
    assert bound < 0.02 * math.sqrt(math.pi / 2 / d) * np.linalg.norm(q) * gam


def test_prod_relmse_matches_closed_form():
    """relMSE of PROD(b+1) on isotropic data = d D(b) (pi/2 - 1/d) in
    expectation (the sketch adds the variance of the previous test)."""
    d = 128
    st = qz.QState(d, qz.PROD, 4, seed=2)
    x = np.random.default_rng(9).standard_normal((3000, d))
    q = qz.quantize(x, st)
    xh = qz.dequantize(q, st)
    per = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    D3 = d * cb.distortion(d, st.centroids, st.boundaries)
    assert abs(per.mean() - D3 * (math.pi / 2 - 1 / d)) < 4 * per.std() / math.sqrt(per.size)
    # Unbiased: the mean error vector of x_hat - x is ~0 along any direction.
    err = (xh - x).mean(axis=0)
    assert np.max(np.abs(err)) < 5 * math.sqrt(per.mean() * 1.0 / 3000) * 1.5


def test_jensen_amplification():
    # [P2] "Contribuições Principais" 2: E[exp(s + eps)] = exp(s) exp(sigma^2/2)
    # for zero-mean Gaussian eps.
    rng = np.random.default_rng(0)
    for sig in (0.1, 0.5, 1.0):
        e = np.exp(rng.standard_normal(400000) * sig)
        assert abs(e.mean() / math.exp(sig * sig / 2) - 1) < 4 * e.std() / math.sqrt(e.size)


def test_sign_band_is_distance_to_the_deciding_hyperplane():
    """The band of a sketch sign is the Euclidean distance, in the rotated
    unit-vector domain the residual lives in, from r to the hyperplane
    S_i . r = 0 that decides the sign (the same units as the code band):
    moving r by exactly that distance along S_i lands on the hyperplane."""
    d = 64
    st = qz.QState(d, qz.PROD, 3, seed=7)
    x = np.random.default_rng(4).standard_normal((5, d))
    q = qz.quantize(x, st)
    Y = x / np.linalg.norm(x, axis=1, keepdims=True) @ st.Pi.T
    R = Y - st.centroids[q["idx"]]
    for n in range(5):
        for i in (0, 17, 63):
            s = st.S[i]
            dist = q["sdist"][n, i]
            r_on = R[n] - np.sign(s @ R[n]) * dist * s / np.linalg.norm(s)
            assert abs(s @ r_on) <= 1e-12 * np.linalg.norm(s)
            assert abs(dist - abs(s @ R[n]) / np.linalg.norm(s)) <= 1e-15


def test_in_band_flip_takes_the_other_cell():
    """A coordinate placed exactly on a boundary has two valid codes; the
    flip selects the neighbour across that boundary and the sketch of the
    residual follows; a flip far from any boundary is refused."""
    d = 32
    st = qz.QState(d, qz.PROD, 3, seed=4)
    x = np.random.default_rng(1).standard_normal((1, d))
    q0 = qz.quantize(x, st)
    # Move coordinate 5 of y exactly onto boundary 1 and map back.
    y = q0["y"][0].copy()
    y[5] = st.boundaries[1]
    xb = (y @ st.Pi)[None, :] * 3.0
    q = qz.quantize(xb, st)
    mask = np.zeros((1, d), bool)
    mask[0, 5] = True
    assert q["bdist"][0, 5] < 1e-12
    qf = qz.quantize(xb, st, flip_codes=mask)
    assert {int(q["idx"][0, 5]), int(qf["idx"][0, 5])} == {1, 2}
    assert np.array_equal(np.delete(q["idx"], 5, axis=1), np.delete(qf["idx"], 5, axis=1))
    # On the midpoint the residual coordinate only changes sign (same gamma),
    # so the sketch of the residual changes.
    assert abs(q["gamma"][0] - qf["gamma"][0]) < 1e-12
    assert np.any(q["sign_bits"] != qf["sign_bits"])
    far = np.zeros((1, d), bool)
    far[0, np.argmax(q["bdist"][0])] = True
    with pytest.raises(AssertionError):
        qz.quantize(xb, st, flip_codes=far)
