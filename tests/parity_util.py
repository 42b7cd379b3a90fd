"""Helpers for the GPU parity tests: run the oracle on the same inputs and
compare with what the library wrote.

Decision band.  A code, a sign bit or a side code may differ from the
oracle's only when the oracle puts that decision within BAND of its
boundary: 1e-6 in the domain of the rotated unit vector for codes (y_i to
its nearest boundary) and for sketch signs (the residual r to the hyperplane
S_i . r = 0, |(S r)_i| / ||S_i||), 1e-5 of a step for HeadQ side codes.  Such a decision has two valid
outcomes; the oracle then recomputes everything downstream (residual,
sketch, dense vectors, attention) with that decision taken the other way,
and the GPU must match that branch exactly as it would the first.  In-band
mismatches are counted and must stay below 1e-5 of all decisions."""
import math

import numpy as np

from oracle import attention as oat
from oracle import headq as ohq
from oracle import metrics as ome
from oracle import quantizer as oqz
from oracle import spectral as osq

BAND = 1e-6
SIDE_BAND = 1e-5
MAX_BAND_FRACTION = 1e-5
OUT_RTOL = 1e-3
KL_ATOL = 1e-5

MODE_NAMES = {0: oqz.PLAIN, 1: oqz.MSE, 2: oqz.PROD, 3: oqz.HEADQ}


def _state(d, mode, n_bits_index, seed):
    if mode == oqz.HEADQ:
        return oqz.QState(d, oqz.MSE, 2, seed)
    total = n_bits_index + 1 if mode == oqz.PROD else n_bits_index
    return oqz.QState(d, mode, total, seed)


def oracle_tensor(X, mode, n_bits_index, seed, U=None, side_bits=4):
    """Oracle quantisation of X [N, d] (float64), no in-band flips.
    Returns (q dict, dense x_hat, state)."""
    st = _state(X.shape[1], mode, n_bits_index, seed)
    if mode == oqz.HEADQ:
        out = ohq.quantize(X, U, st, side_bits=side_bits)
        return out, out["khat"], st
    q = oqz.quantize(X, st)
    return q, oqz.dequantize(q, st), st


def oracle_match(X, gpu, mode, n_bits_index, seed, U=None, side_bits=4, label=""):
    """Quantise X with the oracle, check the GPU planes `gpu` against it
    (codes/signs/side codes exact outside the band; norms, gamma and side
    scales to float32 rounding), and return the oracle branch that the GPU
    took: (q, x_hat, state, n_in_band, n_decisions)."""
    d = X.shape[1]
    N = X.shape[0]
    st = _state(d, mode, n_bits_index, seed)
    headq = mode == oqz.HEADQ
    quant = (lambda **kw: ohq.quantize(X, U, st, side_bits=side_bits, **kw)) if headq else \
            (lambda **kw: oqz.quantize(X, st, **kw))
    q = quant()
    base = q["base"] if headq else q
    g_idx, g_bits = oqz.unpack_fields(gpu["codes"][:N], st, d)
    cmis = g_idx != base["idx"]
    bad = cmis & (base["bdist"] > BAND)
    assert not bad.any(), "%s: %d code mismatches outside the band (first at %s, y=%r)" % (
        label, bad.sum(), np.argwhere(bad)[0], base["y"][tuple(np.argwhere(bad)[0])])
    n_band = int(cmis.sum())
    kw = {"flip_codes": cmis} if cmis.any() else {}
    if cmis.any():
        q = quant(**kw)
    ndec = N * d
    if mode == oqz.PROD:
        smis = g_bits != q["sign_bits"]
        sbad = smis & (q["sdist"] > BAND)
        assert not sbad.any(), "%s: %d sign mismatches outside the band" % (label, sbad.sum())
        if smis.any():
            q = quant(flip_signs=smis, **kw)
        n_band += int(smis.sum())
        ndec += N * d
        gam = gpu["gamma"][:N].astype(np.float64)
        assert np.all(np.abs(gam - q["gamma"]) <= 2e-6 * q["gamma"] + 1e-12), "%s: gamma differs" % label
    if headq:
        rank = q["side_code"].shape[1]
        g_side = oqz.unpack_bits(gpu["side"][:N], side_bits, rank)
        smis = g_side != q["side_code"]
        sbad = smis & (q["hdist"] > SIDE_BAND)
        assert not sbad.any(), "%s: %d side-code mismatches outside the band" % (label, sbad.sum())
        if smis.any():
            q = ohq.quantize(X, U, st, side_bits=side_bits, flip_side=smis, band=SIDE_BAND, **kw)
        n_band += int(smis.sum())
        ndec += N * rank
        ss = gpu["side_scale"][:N].astype(np.float64)
        assert np.all(np.abs(ss - q["side_scale"]) <= 1e-5 * q["side_scale"] + 1e-9), "%s: side scale" % label
    base = q["base"] if headq else q
    assert np.array_equal(oqz.unpack_fields(gpu["codes"][:N], st, d)[0], base["idx"])
    nu = gpu["norms"][:N].astype(np.float64)
    assert np.all(np.abs(nu - base["nu"]) <= 1e-6 * base["nu"]), "%s: norms differ" % label
    xhat = q["khat"] if headq else oqz.dequantize(q, st)
    return q, xhat, st, n_band, ndec


def spectral_match(X, gpu, st, label=""):
    """SpectralQuant counterpart of oracle_match: X [N, d] float64, st an
    oracle SQState built from the same float32 basis, mean and spreads the
    GPU read.  Codes exact outside the band (distance of z_i to its nearest
    boundary s_i t_k), norms to float32 rounding.  Returns (q, x_hat, st,
    n_in_band, n_decisions)."""
    N, d = X.shape
    q = osq.quantize(X, st)
    g_idx = oqz.unpack_bits(gpu["codes"][:N], st.bits, d)
    cmis = g_idx != q["idx"]
    bad = cmis & (q["bdist"] > BAND)
    assert not bad.any(), "%s: %d code mismatches outside the band (first at %s)" % (
        label, bad.sum(), np.argwhere(bad)[0])
    if cmis.any():
        q = osq.quantize(X, st, flip_codes=cmis)
    assert np.array_equal(g_idx, q["idx"])
    nu = gpu["norms"][:N].astype(np.float64)
    assert np.all(np.abs(nu - q["nu"]) <= 1e-6 * q["nu"]), "%s: norms differ" % label
    return q, osq.dequantize(q, st), st, int(cmis.sum()), N * d


def rel_l2(a, b):
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-30)


def oracle_decode(Q, Khat, Vhat):
    """Q [G, d], Khat/Vhat [T, d] -> out [G, d], lse [G], scores [G, T]."""
    o, _, s, lse = oat.attend(Q, Khat, Vhat)
    return o, lse, s


def kl_and_recall(Q, K, Khat):
    d = K.shape[1]
    s = Q @ K.T / math.sqrt(d)
    sh = Q @ Khat.T / math.sqrt(d)
    return ome.kl_from_scores(s, sh), ome.topk_recall(s, sh), s, sh


def top5_ambiguous(s, eps=1e-5):
    """Rows whose 5th and 6th largest scores are within eps (membership of the
    top-5 is then decided by rounding)."""
    srt = -np.sort(-s, axis=-1)
    return np.abs(srt[..., 4] - srt[..., 5]) < eps
