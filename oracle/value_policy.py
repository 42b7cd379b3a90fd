"""A^2-weighted value policy: per-token value bit widths chosen by the
A^2 read-distortion surrogate under a fixed mean budget.   [oracle]

[P3] section 2.2: values are read by o = sum_j p_j v_j, so for fixed
attention p the read error is sum_j p_j dv_j, and the pages take the
diagonal surrogate sum_j p_j^2 ||dv_j||^2 (each token's value distortion
weighted by its squared attention probability) as the value error that
matters.  [P3] section 5 ("Composição Completa KV (2 bits)") pairs HeadQ
keys with a value policy weighted by that surrogate at 2 bits; section 6:
value compression should put its precision where the A^2-weighted error is.

Readings (the pages give no algorithm):
  weights: A_j = mean over probe queries q of p_j(q)^2, p(q) = softmax of
      q^T k_j / sqrt(d) over the sequence's raw keys; the probes of a KV head
      are the probe queries of all its query heads;
  surrogate: a value coded at b bits has expected distortion D_b ||v_j||^2,
      D_b = d * D(d, b) the relative MSE of the b-bit TQ-MSE quantiser (its
      Beta Lloyd-Max distortion per coordinate times d), so the surrogate of
      an assignment b_j is sum_j A_j ||v_j||^2 D_{b_j};
  policy: under a mean budget of bbar index bits per value coordinate the
      candidates are uniform bbar, two tiers (bbar-1, bbar+1) with half the
      tokens high, and (bbar-1, bbar+2) with a third high (widths in
      [1, 4]); R = floor(T * fraction) tokens per (batch, head) go high, the
      ones with the largest w_j = A_j ||v_j||^2 (ties to the lower index);
      the candidate with the smallest surrogate summed over all (batch,
      head) is taken (ties to the earlier candidate in the order above);
  layout: attention is invariant to the order of the (key, value) pairs, so
      the tokens of each (batch, head) are permuted (high tier first, each
      tier in increasing token order) and the high and low tiers are two
      ordinary packed caches; attention over the context is the log-sum-exp
      merge of attention over the two tiers.
"""
import numpy as np

from . import attention as at
from . import codebook as cb
from . import quantizer as qz


def a2_weights(Qp, K):
    """Qp [Np, d] probe queries of one KV head, K [T, d] raw keys -> A [T]."""
    _, p, _, _ = at.attend(Qp, K, np.zeros_like(np.asarray(K, dtype=np.float64)))
    return np.mean(p * p, axis=0)


def value_distortion(d, bits):
    """D_b: expected relative MSE of the b-bit TQ-MSE value quantiser."""
    c, t = cb.lloyd_max(d, bits)
    return d * cb.distortion(d, c, t)


def candidates(budget):
    """(b_lo, b_hi, num, den) in the policy's order; num/den of the tokens high."""
    out = [(budget, budget, 0, 1)]
    for b_lo, b_hi, num, den in ((budget - 1, budget + 1, 1, 2), (budget - 1, budget + 2, 1, 3)):
        if 1 <= b_lo and b_hi <= 4:
            out.append((b_lo, b_hi, num, den))
    return out


def n_high(T, num, den):
    return (T * num) // den


def select(w, R):
    """Boolean mask of the R largest w (ties to the lower index)."""
    w = np.asarray(w, dtype=np.float64)
    order = np.lexsort((np.arange(w.size), -w))   # by -w, then by index
    mask = np.zeros(w.size, dtype=bool)
    mask[order[:R]] = True
    return mask


def permutation(mask):
    """High tier first, each tier in increasing token order."""
    idx = np.arange(mask.size)
    return np.concatenate((idx[mask], idx[~mask]))


def plan(A, vnorm2, d, budget):
    """A, vnorm2 [BH, T] -> dict(option, R, perm [BH, T], surrogate per
    candidate)."""
    A = np.asarray(A, dtype=np.float64)
    w = A * np.asarray(vnorm2, dtype=np.float64)
    T = w.shape[1]
    cands = candidates(budget)
    sur = []
    for b_lo, b_hi, num, den in cands:
        R = n_high(T, num, den)
        D_lo, D_hi = value_distortion(d, b_lo), value_distortion(d, b_hi)
        total = 0.0
        for row in w:
            m = select(row, R)
            total += D_lo * row[~m].sum() + D_hi * row[m].sum()
        sur.append(total)
    k = int(np.argmin(sur))     # first minimum: the earlier candidate wins ties
    b_lo, b_hi, num, den = cands[k]
    R = n_high(T, num, den)
    perm = np.stack([permutation(select(row, R)) for row in w])
    return {"b_lo": b_lo, "b_hi": b_hi, "R": R, "perm": perm, "surrogate": sur, "candidates": cands}


def tiered_values(V, high, b_lo, b_hi, seed):
    """V [T, d] float64, high [T] bool -> V_hat [T, d] in token order: the
    high tokens through the b_hi-bit TQ-MSE quantiser, the rest through the
    b_lo-bit one (both with the rotation of `seed`)."""
    V = np.asarray(V, dtype=np.float64)
    d = V.shape[1]
    out = np.empty_like(V)
    for mask, bits in ((high, b_hi), (~high, b_lo)):
        if mask.any():
            st = qz.QState(d, qz.MSE, bits, seed)
            out[mask] = qz.dequantize(qz.quantize(V[mask], st), st)
    return out


def merge(out_a, lse_a, out_b, lse_b):
    """Attention over the union of two disjoint token sets from the two
    partial results: weights exp(lse_s - lse)."""
    lse = np.logaddexp(lse_a, lse_b)
    wa = np.exp(lse_a - lse)[..., None]
    wb = np.exp(lse_b - lse)[..., None]
    return wa * out_a + wb * out_b, lse


def surrogate_of(A, V, Vhat):
    """sum_j A_j ||v_hat_j - v_j||^2."""
    dv2 = np.sum((np.asarray(Vhat) - np.asarray(V)) ** 2, axis=1)
    return float(np.dot(A, dv2))


def expected_surrogate(A, V, high, b_lo, b_hi):
    d = V.shape[1]
    n2 = np.sum(np.asarray(V, dtype=np.float64) ** 2, axis=1)
    D = np.where(high, value_distortion(d, b_hi), value_distortion(d, b_lo))
    return float(np.sum(A * n2 * D))

