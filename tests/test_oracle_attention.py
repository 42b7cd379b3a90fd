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
        p = np.exp(s - at.logsumexp(s)[:, None])
        fisher = 0.5 * (np.sum(p * ds ** 2, axis=1) - np.sum(p * ds, axis=1) ** 2)
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
