"""Pins of the oracle's read side and metrics (CPU only)."""
import math

import numpy as np
import pytest

from oracle import attention as at
from oracle import headq as hq
from oracle import metrics as me
from oracle import quantizer as qz


def _data(T=300, d=64, G=3, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((G, d))


def test_softmax_shift_invariance():
    # [P3] section 2.1: adding one vector mu to every key adds q.mu/sqrt(d) to
    # every score, which softmax ignores.
    K, V, Q = _data()
    mu = np.random.default_rng(5).standard_normal(K.shape[1]) * 10
    o1, p1, _, _ = at.attend(Q, K, V)
    o2, p2, _, _ = at.attend(Q, K + mu, V)
    assert np.max(np.abs(p1 - p2)) < 1e-12 and np.max(np.abs(o1 - o2)) < 1e-12


def test_bypassed_quantizer_gives_zero_kl_and_full_recall():
    K, V, Q = _data()
    _, _, s, _ = at.attend(Q, K, V)
    assert np.allclose(me.kl_from_scores(s, s), 0, atol=1e-14)
    assert np.all(me.topk_recall(s, s) == 1.0)


def test_single_token_and_zero_query():
    K, V, Q = _data(T=1)
    o, _, _, _ = at.attend(Q, K, V)
    assert np.allclose(o, V[0])
    K, V, Q = _data(T=50)
    o, _, _, _ = at.attend(np.zeros_like(Q), K, V)
    assert np.allclose(o, V.mean(axis=0))


def test_textbook_attention_small_case():
    # Brute force with Python loops on a 3-token example.
    K = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    V = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    q = np.array([[2.0, -1.0]])
    s = [sum(q[0][i] * K[j][i] for i in range(2)) / math.sqrt(2) for j in range(3)]
    w = [math.exp(x) for x in s]
    o = [sum(w[j] * V[j][i] for j in range(3)) / sum(w) for i in range(2)]
    got, _, _, _ = at.attend(q, K, V)
    assert np.allclose(got[0], o, rtol=1e-14)


@pytest.mark.parametrize("kmode,vmode", [(qz.MSE, qz.PROD), (qz.PROD, qz.PROD), (qz.PLAIN, qz.PLAIN)])
def test_rotated_domain_identity(kmode, vmode):
    """The GPU scores and accumulates in the rotated domain:
    q.k_hat = nu (<Pi q, c[idx]> + sqrt(pi/2)/m gamma <S Pi q, sigma>) and
    sum p v_hat = Pi^T (sum p nu c[idx] + sqrt(pi/2)/m S^T sum p nu gamma sigma).
    The oracle's dense dequantisation must agree with that algebra."""
    d, T = 64, 200
    K, V, Q = _data(T=T, d=d, G=2, seed=3)
    sk = qz.QState(d, kmode, 4, seed=7)
    sv = qz.QState(d, vmode, 4, seed=7)
    qk, qv = qz.quantize(K, sk), qz.quantize(V, sv)
    Kh, Vh = qz.dequantize(qk, sk), qz.dequantize(qv, sv)
    o, p, s, _ = at.attend(Q, Kh, Vh)
    nuk = qz.stored(qk["nu"])
    qrot = Q @ sk.Pi.T
    srot = nuk[None, :] * (qrot @ sk.centroids[qk["idx"]].T)
    if kmode == qz.PROD:
        sig = 2.0 * qk["sign_bits"] - 1.0
        srot += nuk[None, :] * sk.qjl_const * qz.stored(qk["gamma"])[None, :] * ((qrot @ sk.S.T) @ sig.T)
    assert np.max(np.abs(srot / math.sqrt(d) - s)) < 1e-12
    nuv = qz.stored(qv["nu"])
    acc = (p * nuv[None, :]) @ sv.centroids[qv["idx"]]
    if vmode == qz.PROD:
        sig = 2.0 * qv["sign_bits"] - 1.0
        acc += sv.qjl_const * ((p * nuv * qz.stored(qv["gamma"])[None, :]) @ sig) @ sv.S
    assert np.max(np.abs(acc @ sv.Pi - o)) < 1e-12


def test_kl_nonnegative_and_fisher_limit():
    """[P3] section 2.1 (Eq. 6): for small score perturbations, KL is half
    the p-weighted variance of the score error."""
    rng = np.random.default_rng(0)
    s = rng.standard_normal((20, 500))
    for eps in (1e-1, 1e-2, 1e-3):
        ds = rng.standard_normal(s.shape) * eps
        kl = me.kl_from_scores(s, s + ds)
        assert np.all(kl >= 0)
        fisher = me.fisher_score_error(s, s + ds)
        ratio = kl / fisher
        assert np.all(np.abs(ratio - 1) < 3 * eps + 1e-6)
    # A constant shift is softmax-null.
    assert np.allclose(me.kl_from_scores(s, s + 3.0), 0, atol=1e-12)


def test_topk_ties_and_recall():
    s = np.array([[5.0, 1.0, 5.0, 3.0, 3.0, 3.0, 0.0]])
    assert list(me.topk_indices(s)[0]) == [0, 2, 3, 4, 5]
    s2 = np.array([[5.0, 1.0, 5.0, 3.0, 0.0, 3.0, 9.0]])
    assert me.topk_recall(s, s2)[0] == 4 / 5


def test_relmse_and_direction():
    X = np.array([[1.0, 0.0], [0.0, 2.0]])
    Xh = np.array([[1.0, 1.0], [0.0, 2.0]])
    assert me.rel_mse(X, Xh) == 1.0 / 5.0
    assert abs(me.direction_error(X, Xh) - 0.5 * (1 - 1 / math.sqrt(2))) < 1e-15


def test_headq_exact_in_span_when_side_quantizer_bypassed():
    """[P3] section 3: with z kept exactly, s_hat = q.k_base/sqrt(d) +
    q.U z/sqrt(d) equals the true score for q in span(U) (U orthonormal)."""
    d, r = 64, 8
    rng = np.random.default_rng(1)
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    K = rng.standard_normal((100, d))
    q = U @ rng.standard_normal(r)
    st = qz.QState(d, qz.MSE, 2, seed=3)
    out = hq.quantize(K, U, st, side_quantizer=False)
    s_true = K @ q / math.sqrt(d)
    s_hat = (out["kbase"] @ q + out["zhat"] @ (U.T @ q)) / math.sqrt(d)
    assert np.max(np.abs(s_hat - s_true)) < 1e-12
    s_base = out["kbase"] @ q / math.sqrt(d)
    assert np.max(np.abs(s_base - s_true)) > 1e-3


def test_headq_side_code_rules():
    d, r = 32, 8
    rng = np.random.default_rng(2)
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    st = qz.QState(d, qz.MSE, 2, seed=3)
    K = rng.standard_normal((50, d))
    out = hq.quantize(K, U, st, side_bits=4)
    code, s = out["side_code"], out["side_scale"]
    assert code.min() >= 0 and code.max() <= 14
    # The largest |z| maps to the extreme code.
    j = np.argmax(np.abs(out["z"]), axis=1)
    ext = code[np.arange(50), j]
    assert np.all((ext == 0) | (ext == 14))
    assert np.allclose(s, np.max(np.abs(out["z"]), axis=1) / 7)
    # Error of each side coefficient is at most half a step.
    assert np.all(np.abs(out["z"] - out["zhat"]) <= 0.5 * s[:, None] * (1 + 1e-6) + 1e-7)


def test_headq_side_code_score_error():
    """[P3] section 3 reads the side code as a logit correction
    q^T U z_hat / sqrt(d).  At the score level: for any q the error the side
    code leaves, q^T U (z_hat - z) / sqrt(d), is at most
    1/2 s_z ||U^T q||_1 / sqrt(d) (each coefficient within half a step); for
    q in span(U) the corrected score error is that alone, far below the
    base-only error q^T e / sqrt(d)."""
    d, r, T = 128, 16, 2000
    rng = np.random.default_rng(12)
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    K = rng.standard_normal((T, d))
    st = qz.QState(d, qz.MSE, 2, seed=4)
    out = hq.quantize(K, U, st, side_bits=4)
    s_z = out["side_scale"]
    for _ in range(20):
        q = rng.standard_normal(d)
        err = (out["zhat"] - out["z"]) @ (U.T @ q) / math.sqrt(d)
        bound = 0.5 * s_z * np.sum(np.abs(U.T @ q)) / math.sqrt(d)
        assert np.all(np.abs(err) <= bound * (1 + 1e-6) + 1e-7)
    E = K - out["kbase"]
    for _ in range(20):
        q = U @ rng.standard_normal(r)
        e_base = E @ q / math.sqrt(d)
        e_corr = (E @ q - out["zhat"] @ (U.T @ q)) / math.sqrt(d)
        assert np.mean(e_corr ** 2) < 0.05 * np.mean(e_base ** 2)
        # The wrong sign ([P3] section 4 control) makes it worse than none.
        e_wrong = (E @ q + out["zhat"] @ (U.T @ q)) / math.sqrt(d)
        assert np.mean(e_wrong ** 2) > np.mean(e_base ** 2)


def test_pca_basis_matches_dominant_subspace():
    d, r = 32, 4
    rng = np.random.default_rng(4)
    W, _ = np.linalg.qr(rng.standard_normal((d, r)))
    X = rng.standard_normal((5000, r)) * np.array([5.0, 4.0, 3.0, 2.0]) @ W.T + 0.05 * rng.standard_normal((5000, d)) + 3.0
    U, lam = hq.fit_basis(X, r)
    assert np.max(np.abs(U @ U.T - W @ W.T)) < 0.02
    assert np.all(np.diff(lam) <= 0)
    for j in range(r):
        assert U[np.argmax(np.abs(U[:, j])), j] > 0


def test_fisher_score_error_closed_forms():
    """Two tokens with p = (a, 1-a) and errors (x, y): Var_p = a (1-a) (x-y)^2.
    A common shift of all score errors changes nothing; a constant error
    gives zero.  The KL limit is pinned in test_kl_nonnegative_and_fisher_limit."""
    a, x, y = 0.3, 0.7, -0.2
    s = np.log(np.array([[a, 1 - a]]))
    f = me.fisher_score_error(s, s + np.array([[x, y]]))
    assert abs(f[0] - 0.5 * a * (1 - a) * (x - y) ** 2) < 1e-15
    rng = np.random.default_rng(3)
    s = rng.standard_normal((4, 50))
    ds = rng.standard_normal((4, 50)) * 0.1
    assert np.allclose(me.fisher_score_error(s, s + ds), me.fisher_score_error(s, s + ds + 2.5), atol=1e-15)
    assert np.allclose(me.fisher_score_error(s, s + 4.0), 0.0, atol=1e-15)
    # Adding one vector to every key is softmax-null ([P3] section 2.1): zero Fisher error.
    K, V, Q = _data()
    mu = rng.standard_normal(K.shape[1])
    _, _, s1, _ = at.attend(Q, K, V)
    _, _, s2, _ = at.attend(Q, K + mu, V)
    assert np.allclose(me.fisher_score_error(s1, s2), 0.0, atol=1e-12)


def test_spearman_textbook_values():
    """Ranks (1..5) against (2, 1, 4, 3, 5): rho = 1 - 6 sum d^2 / (n (n^2 - 1))
    = 1 - 24/120 = 0.8.  Ties: a = (1, 2, 2, 3), b = (1, 2, 3, 4) has average
    ranks (1, 2.5, 2.5, 4) and rho = 3 / sqrt(10).  Monotone maps give +-1."""
    assert abs(me.spearman([1, 2, 3, 4, 5], [2, 1, 4, 3, 5]) - 0.8) < 1e-15
    assert abs(me.spearman([1, 2, 2, 3], [1, 2, 3, 4]) - 3 / np.sqrt(10)) < 1e-15
    x = np.random.default_rng(4).standard_normal(40)
    assert abs(me.spearman(x, np.exp(3 * x)) - 1) < 1e-15
    assert abs(me.spearman(x, -x ** 3) + 1) < 1e-15
    assert list(me.average_ranks([3.0, 1.0, 3.0, 2.0])) == [3.5, 1.0, 3.5, 2.0]
    assert np.isnan(me.spearman([1, 1, 1], [1, 2, 3]))


def test_snr_and_angle_closed_forms():
    """x = 1 in R^4 (10 vectors), noise of norm 0.1 per vector: sum ||x||^2 = 40,
    sum ||e||^2 = 0.1, SNR = 10 log10(400).  SNR = -10 log10(relMSE).  A vector
    turned by theta in a plane and rescaled has angle theta."""
    X = np.ones((10, 4))
    E = np.zeros((10, 4))
    E[:, 1] = 0.1
    assert abs(me.snr_db(X, X + E) - 10 * np.log10(400)) < 1e-12
    rng = np.random.default_rng(6)
    Y, Yh = rng.standard_normal((30, 8)), rng.standard_normal((30, 8))
    assert abs(me.snr_db(Y, Yh) + 10 * np.log10(me.rel_mse(Y, Yh))) < 1e-12
    th = np.array([0.1, 0.5, 1.0, 2.0, np.pi])
    U = np.stack([np.cos(th), np.sin(th), np.zeros_like(th)], axis=1) * np.array([[3.0], [1.0], [0.5], [2.0], [1.0]])
    Xr = np.tile([1.0, 0.0, 0.0], (5, 1))
    assert abs(me.direction_angle(Xr, U) - th.mean()) < 1e-12
    # Zero vectors are left out.
    assert abs(me.direction_angle(np.vstack([Xr, np.zeros(3)]), np.vstack([U, np.ones(3)])) - th.mean()) < 1e-12


def test_a2_value_distortion_is_the_output_error_of_independent_value_errors():
    """[P3] section 2.2: with independent zero-mean value errors,
    E ||sum_j p_j dv_j||^2 = sum_j p_j^2 E ||dv_j||^2 (Monte Carlo, 40000
    draws, 1 % tolerance); a one-hot p reads exactly ||dv||^2 of its token."""
    rng = np.random.default_rng(7)
    T, d = 12, 5
    p = rng.dirichlet(np.ones(T))[None, :]
    sig = rng.uniform(0.2, 1.5, T)
    V = rng.standard_normal((T, d))
    expected = me.a2_value_distortion(p, V, V + sig[:, None] / np.sqrt(d) * np.ones((T, d)))[0]
    # E ||dv_j||^2 = sig_j^2 for dv_j ~ N(0, sig_j^2 / d I_d); the fixed draw above has the same norm.
    dv = rng.standard_normal((40000, T, d)) * (sig[None, :, None] / np.sqrt(d))
    mc = np.mean(np.sum(np.einsum("t,ntd->nd", p[0], dv) ** 2, axis=1))
    assert abs(mc - expected) < 0.01 * expected
    oh = np.zeros((1, T))
    oh[0, 4] = 1.0
    Vh = V + rng.standard_normal((T, d))
    assert abs(me.a2_value_distortion(oh, V, Vh)[0] - np.sum((Vh[4] - V[4]) ** 2)) < 1e-12
