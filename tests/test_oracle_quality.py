"""Soft quality orderings the pages report, on small seeded inputs with wide
margins (CPU oracle only)."""
import math

import numpy as np

from compressed_decode_attention_kv_amd import synth
from oracle import attention as at
from oracle import headq as hq
from oracle import metrics as me
from oracle import quantizer as qz


def _kl_for(scheme_k, scheme_v, K, V, Q, n, seed=0):
    d = K.shape[1]
    sk = qz.QState(d, scheme_k, n, seed)
    sv = qz.QState(d, scheme_v, n, seed)
    Kh = qz.dequantize(qz.quantize(K, sk), sk)
    Vh = qz.dequantize(qz.quantize(V, sv), sv)
    _, _, s, _ = at.attend(Q, K, V)
    o_ref = at.attend(Q, K, V)[0]
    o, _, sh, _ = at.attend(Q, Kh, Vh)
    return me.kl_from_scores(s, sh).mean(), np.mean(np.linalg.norm(o - o_ref, axis=1) / np.linalg.norm(o_ref, axis=1))


def test_kqv_beats_qkqv_at_four_bits():
    """[P1] "Contribuciones Clave" 2: at n = 4, QJL only on V (KQV) gives a
    lower KL than QJL on both (QKQV)."""
    K, V, Q = synth.isotropic_small(seed=0, T=2048, d=128, nq=32)
    K, V, Q = K[0, 0].astype(float), V[0, 0].astype(float), Q[0].astype(float)
    kl_kqv, _ = _kl_for(qz.MSE, qz.PROD, K, V, Q, 4)
    kl_qkqv, _ = _kl_for(qz.PROD, qz.PROD, K, V, Q, 4)
    assert kl_kqv < kl_qkqv / 1.5


def test_rotation_protects_heavy_tails():
    """[P1] "Resultados" and [P2] "Contribuições Principais" 3: on heavy-tailed
    data with outliers, the rotated quantiser (TQ-KV) has a much lower
    relMSE than the plain one."""
    K, _ = synth.heavy_tailed(1, 1, 2000, 128, seed=3)
    K = K[0, 0].astype(float)
    res = {}
    for mode in (qz.PLAIN, qz.MSE):
        st = qz.QState(128, mode, 3, seed=1)
        res[mode] = me.rel_mse(K, qz.dequantize(qz.quantize(K, st), st))
    assert res[qz.MSE] < res[qz.PLAIN] / 2


def test_headq_sign_and_basis_controls():
    """[P3] section 4 ("Implantabilidade", "Direcionalidade"): the PCA basis
    beats a random basis of equal rank, and the correct sign of the
    correction beats none, which beats the wrong sign."""
    d, r = 128, 16
    K, V, Q, C = synth.rope_gqa(1, 1, 4, 2048, d, seed=5, n_calib=4096)
    K = K[0, 0].astype(float)
    Q = Q[0].astype(float)
    U, _ = hq.fit_basis(C[0], r)
    st = qz.QState(d, qz.MSE, 2, seed=1)
    s_ref = Q @ K.T / math.sqrt(d)

    def kl_with(Ub, sign=1.0):
        out = hq.quantize(K, Ub, st, side_bits=4)
        Keff = out["kbase"] + sign * out["zhat"] @ Ub.T
        return me.kl_from_scores(s_ref, Q @ Keff.T / math.sqrt(d)).mean()

    out = hq.quantize(K, U, st)
    kl_none = me.kl_from_scores(s_ref, Q @ out["kbase"].T / math.sqrt(d)).mean()
    kl_pca, kl_wrong = kl_with(U), kl_with(U, -1.0)
    R, _ = np.linalg.qr(np.random.default_rng(0).standard_normal((d, r)))
    kl_rand = kl_with(R)
    assert kl_pca < kl_none < kl_wrong
    assert kl_pca < 0.7 * kl_rand
