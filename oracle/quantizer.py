"""Write side: norm split, rotation, Lloyd-Max index, QJL sketch, packing.   [oracle]

Modes (per tensor):
  PLAIN  [P1] "Esquemas de Cuantización" scheme KV and [P2] "Contribuições
         Principais" 1 (Plain-KV): scalar Lloyd-Max, no rotation, no sketch.
  MSE    [P2] "Contribuições Principais" 1 (TQ-KV): rotation + Beta Lloyd-Max.
  PROD   [P1] "Esquemas de Cuantización" (V of KQV, K and V of QKQV):
         rotation + (n-1)-bit Lloyd-Max + 1-bit QJL sketch of the residual.
  HEADQ  [P3] section 3 "Metodologia: HeadQ": low-bit base quantiser plus a
         side code of the residual in a learned rank-r basis (see headq.py).

Per vector x (length d), with nu = ||x||:
  nu = 0  -> every stored field is 0 and the dequantised vector is 0.
  y = Pi x / nu  (PLAIN: y = x / nu)
  idx_i = #{k : y_i >= t_k}
  PROD: r = y - c[idx], gamma = ||r||, bit_i = [(S r)_i >= 0]  (sign(0) = +1)
Dequantisation (x_hat):
  PLAIN: nu c[idx];  MSE: nu Pi^T c[idx];
  PROD:  nu Pi^T (c[idx] + sqrt(pi/2)/m gamma S^T sigma),  sigma = 2 bit - 1.
The constant sqrt(pi/2)/m is the one that makes the sketch estimate of the
residual unbiased ([P1] "Contribuciones Clave" 1: the QJL estimator is
unbiased), because E[s sign(s.r)] = sqrt(2/pi) r/||r|| for s ~ N(0, I).

Packing: per vector a little-endian LSB-first bitstream of d fields.  MSE
and PLAIN: field i is idx_i, b bits, at bits [b i, b i + b) of the d b / 8
byte code block.  PROD (m = d): field i is idx_i | bit_i << b, b + 1 bits,
at bits [(b+1) i, (b+1) i + b + 1) of the d (b+1) / 8 byte code block: the
code of coordinate i and the sign of sketch row i side by side (the pages fix
no layout; both are read at the same index i, see dequantize).
"""
import math
import numpy as np

from . import codebook as cb
from .rng import gaussian_sketch
from .rotation import rotation_matrix

PLAIN, MSE, PROD, HEADQ = "plain", "mse", "prod", "headq"


class QState:
    """Everything the quantiser of one (seed, d, mode, bits) needs."""

    def __init__(self, d, mode, bits, seed, m=None):
        self.d, self.mode, self.bits, self.seed = d, mode, bits, seed
        self.m = d if m is None else m
        self.base_bits = bits - 1 if mode == PROD else bits
        self.centroids, self.boundaries = cb.lloyd_max(d, self.base_bits)
        self.Pi = rotation_matrix(seed, d) if mode != PLAIN else np.eye(d)
        self.S = gaussian_sketch(seed, d, self.m) if mode == PROD else None
        self.qjl_const = math.sqrt(math.pi / 2.0) / self.m


def stored(v):
    """Norms and residual norms are stored as float32; dequantisation uses the
    stored values."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def other_side(Y, idx, boundaries, mask, band):
    """For coordinates in `mask` (each within `band` of a decision boundary),
    the index of the cell on the other side of that boundary.  A coordinate
    this close to a boundary has two valid codes; this is the second one."""
    idx = idx.copy()
    if not np.any(mask):
        return idx
    y = Y[mask]
    k = np.argmin(np.abs(y[:, None] - boundaries[None, :]), axis=1)
    assert np.all(np.abs(y - boundaries[k]) <= band), "flip requested outside the decision band"
    cur = idx[mask]
    assert np.all((cur == k) | (cur == k + 1))
    idx[mask] = np.where(cur == k, k + 1, k)
    return idx


def quantize(X, st, flip_codes=None, flip_signs=None, band=1e-6):
    """X: [N, d] float64.  Returns a dict of unpacked fields plus the
    parity-band diagnostics, both distances to a decision boundary in the
    domain of the rotated unit vector: for a code, the distance of y_i to its
    nearest boundary; for a sign bit, the distance of the residual r (which
    lives in that same domain) to the hyperplane S_i . r = 0 that decides it,
    |(S r)_i| / ||S_i||.

    flip_codes / flip_signs ([N, d] / [N, m] boolean, optional) select
    decisions taken within `band` of their boundary; those take the other
    valid outcome, and everything downstream (residual, sketch) follows."""
    X = np.asarray(X, dtype=np.float64)
    N, d = X.shape
    nu = np.sqrt(np.sum(X * X, axis=1))
    safe = np.where(nu > 0, nu, 1.0)
    U = X / safe[:, None]
    Y = U @ st.Pi.T
    idx = cb.quantize_index(Y, st.boundaries)
    if flip_codes is not None:
        idx = other_side(Y, idx, st.boundaries, flip_codes, band)
    zero = nu == 0
    idx[zero] = 0
    out = {"nu": nu, "idx": idx, "y": Y,
           "bdist": np.where(zero[:, None], np.inf, cb.boundary_distance(Y, st.boundaries))}
    if st.mode == PROD:
        R = Y - st.centroids[idx]
        gamma = np.sqrt(np.sum(R * R, axis=1))
        P = R @ st.S.T
        bits = (P >= 0).astype(np.int64)
        gamma[zero] = 0.0
        bits[zero] = 0
        row_norm = np.sqrt(np.sum(st.S * st.S, axis=1))
        sdist = np.where(zero[:, None], np.inf, np.abs(P) / row_norm[None, :])
        if flip_signs is not None and np.any(flip_signs):
            assert np.all(sdist[flip_signs] <= band), "sign flip requested outside the band"
            bits[flip_signs] = 1 - bits[flip_signs]
        out["gamma"] = gamma
        out["sign_bits"] = bits
        out["sdist"] = sdist
    return out


def dequantize(q, st):
    """Dense dequantised vectors in the original domain, [N, d] float64."""
    Yhat = st.centroids[q["idx"]]
    if st.mode == PROD:
        sigma = 2.0 * q["sign_bits"] - 1.0
        Yhat = Yhat + st.qjl_const * stored(q["gamma"])[:, None] * (sigma @ st.S)
    nu = stored(q["nu"])
    Xhat = nu[:, None] * (Yhat @ st.Pi)
    Xhat[nu == 0] = 0.0
    return Xhat


def pack_bits(values, width):
    """values: [N, L] non-negative ints < 2^width -> [N, L*width/8] uint8,
    LSB-first bitstream per row."""
    values = np.asarray(values, dtype=np.int64)
    N, L = values.shape
    nbits = L * width
    assert nbits % 8 == 0
    bitarr = np.zeros((N, nbits), dtype=np.uint8)
    for j in range(width):
        bitarr[:, j::width] = (values >> j) & 1
    out = np.zeros((N, nbits // 8), dtype=np.int64)
    for j in range(8):
        out |= bitarr[:, j::8].astype(np.int64) << j
    return out.astype(np.uint8)


def unpack_bits(packed, width, L):
    """Inverse of pack_bits."""
    packed = np.asarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    bitarr = np.zeros((N, packed.shape[1] * 8), dtype=np.int64)
    for j in range(8):
        bitarr[:, j::8] = (packed >> j) & 1
    vals = np.zeros((N, L), dtype=np.int64)
    for j in range(width):
        vals |= bitarr[:, j:L * width:width] << j
    return vals


def pack(q, st):
    """Packed planes of one batch of vectors, as the cache stores them."""
    if st.mode == PROD:
        fields = np.asarray(q["idx"], dtype=np.int64) | (np.asarray(q["sign_bits"], dtype=np.int64) << st.base_bits)
        return {"codes": pack_bits(fields, st.base_bits + 1), "norms": q["nu"].astype(np.float32),
                "gamma": q["gamma"].astype(np.float32)}
    return {"codes": pack_bits(q["idx"], st.base_bits), "norms": q["nu"].astype(np.float32)}


def unpack_fields(codes, st, d):
    """Inverse of pack's code block: (idx [N, d], sign bits [N, d] or None)."""
    if st.mode == PROD:
        f = unpack_bits(codes, st.base_bits + 1, d)
        return f & ((1 << st.base_bits) - 1), f >> st.base_bits
    return unpack_bits(codes, st.base_bits, d), None
