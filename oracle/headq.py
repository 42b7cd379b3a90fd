"""HeadQ key path: query-PCA basis, residual side code, logit correction.   [oracle]

[P3] section 3 "Metodologia: HeadQ":
  calibration: per layer and head, a rank-r basis U_h learned by PCA of
      post-RoPE calibration queries;
  cache write: a standard low-bit base quantiser gives k_base; the residual
      e = k - k_base is projected on the basis and coded by a low-bit side
      quantiser, z = Q_q(U_h^T e); the cache keeps the base code and z;
  cache read: s_hat = q^T k_base / sqrt(d) + q^T U_h z_hat / sqrt(d), an
      additive logit correction without rebuilding the key.

Readings (the pages leave these open):
  base quantiser: the framework's own rotated Beta Lloyd-Max (MSE) at b = 2;
  PCA: centred covariance of the calibration queries, eigenvectors of the
      r largest eigenvalues, each with its largest-|.| entry made positive;
  side quantiser Q_q (parity unpinned): per-token symmetric absmax uniform,
      L = 2^(q_s-1) - 1 levels per side (7 at 4 bits),
      s_z = max_i |z_i| / L, code_i = clamp(rne(z_i / s_z), -L, L) + L,
      z_hat = s_z (code - L); s_z = 0 gives all codes L.
"""
import numpy as np

from . import quantizer as qz


def fit_basis(calib_q, rank):
    """U [d, rank] from the centred covariance of calib_q [N, d]."""
    Qc = np.asarray(calib_q, dtype=np.float64)
    Qc = Qc - Qc.mean(axis=0, keepdims=True)
    C = Qc.T @ Qc / Qc.shape[0]
    w, V = np.linalg.eigh(C)
    order = np.argsort(w)[::-1][:rank]
    U = V[:, order]
    for j in range(rank):
        k = np.argmax(np.abs(U[:, j]))
        if U[k, j] < 0:
            U[:, j] = -U[:, j]
    return U, w[order]


def side_levels(side_bits):
    return (1 << (side_bits - 1)) - 1


def quantize(X, U, st_base, side_bits=4, side_quantizer=True, flip_codes=None, flip_side=None, band=1e-6):
    """X [N, d]; U [d, r]; st_base: an MSE QState (bits = 2).
    Returns base fields, side codes, scale and the effective dense key
    k_hat = k_base + U z_hat that enters every score.  flip_codes /
    flip_side select decisions within `band` of their boundary that take the
    other valid outcome (base index, or the rounding of z / s_z)."""
    X = np.asarray(X, dtype=np.float64)
    base = qz.quantize(X, st_base, flip_codes=flip_codes, band=band)
    kbase = qz.dequantize(base, st_base)
    E = X - kbase
    Z = E @ U
    L = side_levels(side_bits)
    if side_quantizer:
        s = np.max(np.abs(Z), axis=1) / L
        safe = np.where(s > 0, s, 1.0)
        ratio = Z / safe[:, None]
        code = np.clip(np.rint(ratio), -L, L).astype(np.int64) + L
        code[s == 0] = L
        frac = np.abs(ratio) - np.floor(np.abs(ratio))
        hdist = np.abs(frac - 0.5)  # distance to the rounding boundary, in steps
        if flip_side is not None and np.any(flip_side):
            assert np.all(hdist[flip_side] <= band), "side flip requested outside the band"
            lo = np.floor(ratio[flip_side]).astype(np.int64) + L
            cur = code[flip_side]
            code[flip_side] = np.where(cur == lo, lo + 1, lo)
        s32 = s.astype(np.float32).astype(np.float64)
        Zhat = s32[:, None] * (code - L)
    else:
        s, code, Zhat, hdist = None, None, Z, None
    return {"base": base, "kbase": kbase, "z": Z, "side_scale": s,
            "side_code": code, "zhat": Zhat, "khat": kbase + Zhat @ U.T,
            "hdist": hdist}
